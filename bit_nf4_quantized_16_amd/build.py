"""Build libqlora_nf4.so (HIP, gfx950) in-tree with hipcc.

    python bit_nf4_quantized_16_amd/build.py [--jobs N] [--verbose]

(run as a script: importing the package loads the library being rebuilt)

Every source is compiled for gfx950 only, with floating-point contraction
off (the quantization outputs are compared bit for bit) and without packed
fp32 instructions.
"""

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqlora_nf4.so")

SOURCES = ["quantize.hip", "dequant.hip", "gemv.hip", "lora.hip", "gemm_tiles.hip", "merge.hip", "qerror.hip", "dropout.hip", "optim.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return path


def compile_flags():
    return [
        "-x",
        "hip",
        "--offload-arch=" + ARCH,
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-ffp-contract=off",
        "-Xclang",
        "-target-feature",
        "-Xclang",
        "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-result",
        "-I" + INCLUDE,
        "-I" + CSRC,
    ]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # the host pass does not know the packed-fp32 feature name; that is expected
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (src, "\n".join(lines)))
    if verbose and lines:
        print("\n".join(lines), flush=True)
    return obj


def build(jobs=4, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    sys.exit(main())
