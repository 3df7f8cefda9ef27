"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): every source is compiled with the sanitizers on its host pass only
(the device code is unchanged), linked with a host driver that calls every
entry point with rejected arguments and with valid shapes up to the first
launch (tests/host/abi_driver.cpp), and run. Any sanitizer report fails the
test (halt_on_error)."""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from conftest import ROOT

sys.path.insert(0, os.path.join(ROOT, "bit_nf4_quantized_16_amd"))
import build as B  # noqa: E402

CLANG = "/opt/rocm/llvm/bin/clang++"
pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def test_abi_host_code_under_asan_and_ubsan():
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    with tempfile.TemporaryDirectory() as d:
        def comp(src):
            obj = os.path.join(d, os.path.basename(src) + ".o")
            r = subprocess.run([B.hipcc()] + B.compile_flags() + san + ["-c", src, "-o", obj],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return obj

        srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES] + [os.path.join(ROOT, "tests", "host", "abi_driver.cpp")]
        with ThreadPoolExecutor(max_workers=4) as ex:
            objs = list(ex.map(comp, srcs))
        exe = os.path.join(d, "abi_driver")
        r = subprocess.run([CLANG, "-fsanitize=address,undefined", "-o", exe] + objs +
                           ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0 and "driver ok" in r.stdout, (r.stdout[-2000:] + r.stderr[-4000:])
