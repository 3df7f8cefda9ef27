"""The C-ABI library loads, exports every function include/qlora_nf4.h
declares, and rejects bad arguments before launching anything (so these
run without a GPU)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qlora_nf4.h")
LIB = os.path.join(ROOT, "bit_nf4_quantized_16_amd", "libqlora_nf4.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from bit_nf4_quantized_16_amd import _lib

    return _lib.load(LIB)


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 16
    from bit_nf4_quantized_16_amd import _lib

    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, "binding lacks " + n


def test_status_strings(lib):
    for code in range(-6, 1):
        s = lib.qlora_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.qlora_status_string(-99).decode() == "unknown status"


def test_size_helpers(lib):
    assert lib.nf4_packed_bytes(4096, 4096) == 4096 * 4096 // 2
    assert lib.nf4_packed_bytes(3, 5) == 8
    assert lib.nf4_num_blocks(4096, 4096, 64) == 262144
    assert lib.nf4_num_blocks(1, 65, 64) == 2
    assert lib.nf4_dq_num_groups(262144, 256) == 1024
    assert lib.nf4_dq_num_groups(257, 256) == 2
    assert lib.nf4_double_quant_workspace(1024) >= 8
    assert lib.qlora_linear_fwd_workspace(4096, 4096, 1024, 16) > 0
    # decode (T <= 16): U's tagged words and the epoch word when r > 0
    assert lib.qlora_linear_fwd_workspace(4096, 4096, 1, 0) == 0
    assert lib.qlora_linear_fwd_workspace(4096, 4096, 16, 16) >= 16 * 16 * 8 * 4
    assert lib.qlora_linear_bwd_workspace(4096, 4096, 1024, 16) > 0


# fake, 16-byte aligned device addresses: validation never dereferences them
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
P3 = ctypes.c_void_p(0x30000)
MIS = ctypes.c_void_p(0x10004)


def _err(lib):
    return lib.qlora_last_error().decode()


def test_quantize_rejects(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    assert lib.nf4_quantize(None, L.QL_F32, 4, 64, 64, P2, P3, None) == L.QL_ERR_NULL
    assert "W" in _err(lib)
    assert lib.nf4_quantize(P, L.QL_F32, 0, 64, 64, P2, P3, None) == L.QL_ERR_SHAPE
    assert lib.nf4_quantize(P, L.QL_F32, 4, -1, 64, P2, P3, None) == L.QL_ERR_SHAPE
    assert lib.nf4_quantize(P, L.QL_F32, 4, 64, 32, P2, P3, None) == L.QL_ERR_UNSUPPORTED
    assert lib.nf4_quantize(P, 7, 4, 64, 64, P2, P3, None) == L.QL_ERR_UNSUPPORTED
    assert lib.nf4_quantize(MIS, L.QL_F32, 4, 64, 64, P2, P3, None) == L.QL_ERR_ALIGN
    assert lib.nf4_quantize(P, L.QL_BF16, 4, 64, 64, None, P3, None) == L.QL_ERR_NULL


def test_double_quant_rejects(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    need = lib.nf4_double_quant_workspace(1000)
    assert lib.nf4_double_quant(P, 0, 256, P2, P3, P, P, need, None) == L.QL_ERR_SHAPE
    assert lib.nf4_double_quant(P, 1000, 128, P2, P3, P, P, need, None) == L.QL_ERR_UNSUPPORTED
    assert lib.nf4_double_quant(P, 1000, 256, None, P3, P, P, need, None) == L.QL_ERR_NULL
    assert lib.nf4_double_quant(P, 1000, 256, P2, P3, P, P, need - 1, None) == L.QL_ERR_WORKSPACE
    assert lib.nf4_double_quant(P, 1000, 256, P2, P3, P, None, need, None) == L.QL_ERR_WORKSPACE
    assert lib.nf4_double_quant(P, 1000, 256, P2, P3, MIS, P, need, None) == L.QL_ERR_ALIGN


def _weight(L, rows=256, cols=256, dq=256, **over):
    w = L.QlNf4Weight()
    w.rows, w.cols, w.blocksize, w.dq_blocksize = rows, cols, 64, dq
    w.packed, w.absmax, w.c8, w.dq_scale, w.dq_mean = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
    for k, v in over.items():
        setattr(w, k, v)
    return ctypes.byref(w)


def test_quantize_dq_rejects_and_sizes(lib):
    """nf4_quantize_dq validates like the two calls it replaces; its
    workspace holds one fp64 tree node per quantize workgroup when the size
    allows the fold, else the double quantization's tree levels."""
    from bit_nf4_quantized_16_amd import _lib as L

    need = lib.nf4_quantize_dq_workspace(64, 4096, L.QL_F32)
    # 262144 fp32 elements: 4096 constants, 64 workgroups of 64 constants
    assert need == 64 * 8
    assert lib.nf4_quantize_dq_workspace(64, 4096, L.QL_BF16) == 32 * 8
    # more than 16384 nodes: the three-launch path
    assert lib.nf4_quantize_dq_workspace(16384, 65536 + 256, L.QL_F32) == lib.nf4_double_quant_workspace(
        16384 * (65536 + 256) // 64)
    # a tail (n % 256 != 0) takes the three-launch path and its workspace
    assert lib.nf4_quantize_dq_workspace(3, 100, L.QL_F32) == lib.nf4_double_quant_workspace(5)
    assert lib.nf4_quantize_dq_workspace(0, 64, L.QL_F32) == 0
    assert lib.nf4_quantize_dq_workspace(64, 64, 7) == 0

    def call(W=P, dt=L.QL_F32, rows=64, cols=4096, bs=64, dqbs=256, c8=P2, ws=P3, wsb=need):
        return lib.nf4_quantize_dq(W, dt, rows, cols, bs, P, P2, dqbs, c8, P3, P, ws, wsb, None)

    assert call(W=None) == L.QL_ERR_NULL
    assert call(rows=0) == L.QL_ERR_SHAPE
    assert call(bs=128) == L.QL_ERR_UNSUPPORTED
    assert call(dqbs=64) == L.QL_ERR_UNSUPPORTED
    assert call(dt=9) == L.QL_ERR_UNSUPPORTED
    assert call(c8=None) == L.QL_ERR_NULL
    assert call(wsb=need - 1) == L.QL_ERR_WORKSPACE
    assert call(ws=None) == L.QL_ERR_WORKSPACE
    assert call(W=MIS) == L.QL_ERR_ALIGN


def test_dequantize_rejects(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    assert lib.nf4_dequantize(None, P, L.QL_BF16, None) == L.QL_ERR_NULL
    assert lib.nf4_dequantize(_weight(L, rows=0), P, L.QL_BF16, None) == L.QL_ERR_SHAPE
    assert lib.nf4_dequantize(_weight(L, blocksize=128), P, L.QL_BF16, None) == L.QL_ERR_UNSUPPORTED
    assert lib.nf4_dequantize(_weight(L, dq_blocksize=64), P, L.QL_BF16, None) == L.QL_ERR_UNSUPPORTED
    assert lib.nf4_dequantize(_weight(L, c8=None), P, L.QL_BF16, None) == L.QL_ERR_NULL
    assert lib.nf4_dequantize(_weight(L, dq=0, absmax=None), P, L.QL_BF16, None) == L.QL_ERR_NULL
    assert lib.nf4_dequantize(_weight(L, packed=0x10008), P, L.QL_BF16, None) == L.QL_ERR_ALIGN
    assert lib.nf4_dequantize(_weight(L), P, 5, None) == L.QL_ERR_UNSUPPORTED
    assert lib.nf4_dequantize(_weight(L), None, L.QL_BF16, None) == L.QL_ERR_NULL


def test_linear_fwd_rejects(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    need = lib.qlora_linear_fwd_workspace(256, 256, 64, 8)
    ok = dict(X=P, T=64, A=P2, B=P3, r=8, Y=P, U=None, ws=P, wsb=need)

    def call(w=None, **kw):
        a = dict(ok)
        a.update(kw)
        return lib.qlora_linear_fwd(w if w is not None else _weight(L), a["X"], a["T"], a["A"], a["B"], a["r"],
                                    2.0, a["Y"], a["U"], a["ws"], a["wsb"], None)

    assert call(w=_weight(L, cols=96)) == L.QL_ERR_SHAPE  # K % 64
    assert call(w=_weight(L, rows=100)) == L.QL_ERR_SHAPE  # N % 8
    assert call(T=-1) == L.QL_ERR_SHAPE
    assert call(r=129) == L.QL_ERR_SHAPE
    assert call(r=-1) == L.QL_ERR_SHAPE
    assert call(X=None) == L.QL_ERR_NULL
    assert call(A=None) == L.QL_ERR_NULL
    assert call(Y=MIS) == L.QL_ERR_ALIGN
    assert call(wsb=need - 1) == L.QL_ERR_WORKSPACE
    assert call(ws=None) == L.QL_ERR_WORKSPACE
    assert call(T=0) == L.QL_OK  # empty batch: no-op, nothing launched


def test_backward_sizing_without_adapter_gradients(lib):
    """dX alone (dA and dB NULL) at T > 2048: the workspace sizing once
    divided by the number of gradient columns, zero here, and raised SIGFPE
    in the caller's process. Without a GPU the call gets as far as its first
    launch and reports the HIP error."""
    from bit_nf4_quantized_16_amd import _lib as L

    for T in (2049, 4096, 8192):
        ws = lib.qlora_linear_bwd_workspace(4096, 4096, T, 16)
        s = lib.qlora_linear_bwd(_weight(L, rows=4096, cols=4096), P, P2, T, P3, P, 16, 2.0, P2, P3, None, None, 0, P,
                                 ws, None)
        assert s in (L.QL_OK, L.QL_ERR_HIP)


def test_fwd_u_in_launch_query(lib, monkeypatch):
    """Where the forward computes U inside its GEMM launch (host logic only:
    without a GPU the plan assumes 256 CUs): the 172-tile 7B gate/up shapes
    at T = 1024 with ranks 8 and 16; not the split-K down shape, other ranks,
    decode sizes or invalid sizes; QLORA_NF4_FWD_U=prepass turns it off, and
    the workspace then holds the projection's buffers instead of the words."""
    assert lib.qlora_linear_fwd_u_in_launch(11008, 4096, 1024, 16) == 1
    assert lib.qlora_linear_fwd_u_in_launch(11008, 4096, 1024, 8) == 1
    assert lib.qlora_linear_fwd_u_in_launch(4096, 11008, 1024, 16) == 0  # reduction split 4 ways
    assert lib.qlora_linear_fwd_u_in_launch(11008, 4096, 1024, 64) == 0
    assert lib.qlora_linear_fwd_u_in_launch(11008, 4096, 1024, 5) == 0
    assert lib.qlora_linear_fwd_u_in_launch(11008, 4096, 16, 16) == 0  # decode GEMV
    for bad in ((0, 4096, 1024, 16), (11008, 0, 1024, 16), (11008, 4096, 0, 16), (11008, 4096, 1024, -1)):
        assert lib.qlora_linear_fwd_u_in_launch(*bad) == 0
    words = lib.qlora_linear_fwd_workspace(11008, 4096, 1024, 16)
    monkeypatch.setenv("QLORA_NF4_FWD_U", "prepass")
    assert lib.qlora_linear_fwd_u_in_launch(11008, 4096, 1024, 16) == 0
    prepass = lib.qlora_linear_fwd_workspace(11008, 4096, 1024, 16)
    # words: 1024 x 16 x 8 B + the epoch word; prepass: bf16 s U padded to 64
    assert words >= 1024 * 16 * 8 + 8 and prepass >= 1024 * 64 * 2 and words != prepass


def test_bwd_g_in_launch_query(lib, monkeypatch):
    """Where the backward computes G = s dY B inside its dX GEMM launch (host
    logic, 256 CUs assumed): the 7B down shape at T = 1024 (172 unsplit dX
    tiles over K = 11008), not gate/up (their dX reduction is split), other
    ranks or invalid sizes; QLORA_NF4_FWD_U=prepass turns it off."""
    assert lib.qlora_linear_bwd_g_in_launch(4096, 11008, 1024, 16) == 1
    assert lib.qlora_linear_bwd_g_in_launch(4096, 11008, 1024, 8) == 1
    assert lib.qlora_linear_bwd_g_in_launch(11008, 4096, 1024, 16) == 0
    assert lib.qlora_linear_bwd_g_in_launch(4096, 11008, 1024, 32) == 0
    for bad in ((0, 4096, 1024, 16), (4096, 0, 1024, 16), (4096, 11008, 0, 16), (4096, 11008, 1024, -1)):
        assert lib.qlora_linear_bwd_g_in_launch(*bad) == 0
    words = lib.qlora_linear_bwd_workspace(4096, 11008, 1024, 16)
    monkeypatch.setenv("QLORA_NF4_FWD_U", "prepass")
    assert lib.qlora_linear_bwd_g_in_launch(4096, 11008, 1024, 16) == 0
    assert lib.qlora_linear_bwd_workspace(4096, 11008, 1024, 16) != words


def test_linear_fwd_noalloc_rejects(lib):
    """The entry point without a workspace validates like qlora_linear_fwd and
    turns down, before touching the GPU, a call whose scratch need is larger
    than the library's array."""
    from bit_nf4_quantized_16_amd import _lib as L

    def call(w=None, T=64, r=8, X=P, A=P2, B=P3, Y=P):
        return lib.qlora_linear_fwd_noalloc(w if w is not None else _weight(L), X, T, A, B, r, 2.0, Y, None, None)

    assert call(w=_weight(L, cols=96)) == L.QL_ERR_SHAPE
    assert call(w=_weight(L, rows=100)) == L.QL_ERR_SHAPE
    assert call(r=129) == L.QL_ERR_SHAPE
    assert call(T=-1) == L.QL_ERR_SHAPE
    assert call(T=0) == L.QL_OK
    m = re.search(r"#define QL_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == L.QL_NOALLOC_SCRATCH_BYTES
    # 2^20 tokens at rank 128: 256 MiB of bf16 s U staging alone
    big = 1 << 20
    assert lib.qlora_linear_fwd_workspace(256, 256, big, 128) > L.QL_NOALLOC_SCRATCH_BYTES
    assert call(T=big, r=128) == L.QL_ERR_WORKSPACE
    assert b"noalloc" in lib.qlora_last_error()


def test_paged_adamw_rejects(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    ok = dict(p=P, p16=None, g=P2, m=P3, v=P, n=1000, step=1, lr=2e-4, b1=0.9, b2=0.999, eps=1e-8, wd=0.0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.qlora_paged_adamw(a["p"], a["p16"], a["g"], a["m"], a["v"], a["n"], a["step"], a["lr"], a["b1"],
                                     a["b2"], a["eps"], a["wd"], None, 0, None, None)

    assert call(n=0) == L.QL_ERR_SHAPE
    assert call(step=0) == L.QL_ERR_SHAPE
    assert call(b1=1.0) == L.QL_ERR_UNSUPPORTED
    assert call(b2=-0.1) == L.QL_ERR_UNSUPPORTED
    assert call(eps=-1e-8) == L.QL_ERR_UNSUPPORTED
    assert call(lr=float("nan")) == L.QL_ERR_UNSUPPORTED
    assert call(wd=-0.5) == L.QL_ERR_UNSUPPORTED
    assert call(p=None) == L.QL_ERR_NULL
    assert call(g=None) == L.QL_ERR_NULL
    assert call(m=None) == L.QL_ERR_NULL
    assert call(v=MIS) == L.QL_ERR_ALIGN
    assert call(p16=MIS) == L.QL_ERR_ALIGN
    # two staging buffers of m and v, at most 2^21 elements each
    assert lib.qlora_paged_adamw_workspace(0) == 0
    assert lib.qlora_paged_adamw_workspace(100) == 4 * 128 * 4
    assert lib.qlora_paged_adamw_workspace(1 << 30) == 4 * (1 << 21) * 4


def test_linear_fwd_group_rejects(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    def descs(shapes):
        ws = []
        for rows, cols in shapes:
            w = L.QlNf4Weight()
            w.rows, w.cols, w.blocksize, w.dq_blocksize = rows, cols, 64, 256
            w.packed, w.absmax, w.c8, w.dq_scale, w.dq_mean = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
            ws.append(w)
        return ws

    def ptrs(vals, n):
        return (ctypes.c_void_p * max(n, 1))(*vals)

    def rows(*r):
        return (ctypes.c_int64 * len(r))(*r)

    # decode sizes: one GEMV workspace slice per layer; larger T: the largest
    # single-layer workspace, the layers running one after another
    one = lib.qlora_linear_fwd_workspace(256, 256, 16, 8)
    assert lib.qlora_linear_fwd_group_workspace(rows(256, 256, 512), 3, 256, 16, 8) == 3 * one
    assert lib.qlora_linear_fwd_group_workspace(rows(256, 512), 2, 256, 64, 8) == max(
        lib.qlora_linear_fwd_workspace(256, 256, 64, 8), lib.qlora_linear_fwd_workspace(512, 256, 64, 8))
    assert lib.qlora_linear_fwd_group_workspace(rows(256), 0, 256, 16, 8) == 0
    assert lib.qlora_linear_fwd_group_workspace(rows(256, 256, 256, 256, 256), 5, 256, 16, 8) == 0
    assert lib.qlora_linear_fwd_group_workspace(rows(256, 0), 2, 256, 16, 8) == 0
    assert lib.qlora_linear_fwd_group_workspace(None, 1, 256, 16, 8) == 0
    # above decode sizes one GEMM launch over all layers where the tile plan
    # favours it (q/k/v at T = 1024, whose single GEMMs split the reduction);
    # its workspace then holds every layer's bf16(s U)
    assert lib.qlora_linear_fwd_group_one_launch(rows(4096, 4096, 4096), 3, 4096, 1024, 16) == 1
    # (enough for both paths: layers of mixed formats run one after another)
    assert lib.qlora_linear_fwd_group_workspace(rows(4096, 4096, 4096), 3, 4096, 1024, 16) >= max(
        3 * 1024 * 64 * 2, lib.qlora_linear_fwd_workspace(4096, 4096, 1024, 16))
    assert lib.qlora_linear_fwd_group_one_launch(rows(11008, 11008), 2, 4096, 1024, 16) == 0  # 344 tiles: no
    assert lib.qlora_linear_fwd_group_one_launch(rows(11008, 11008), 2, 4096, 2048, 16) == 1
    assert lib.qlora_linear_fwd_group_one_launch(rows(4096, 4096, 4096), 3, 4096, 1024, 12) == 0  # r % 8
    assert lib.qlora_linear_fwd_group_one_launch(rows(4096, 4096, 4096), 3, 4096, 16, 16) == 0  # the GEMV
    assert lib.qlora_linear_fwd_group_one_launch(None, 3, 4096, 1024, 16) == 0

    def call(shapes=((256, 256), (512, 256)), nw=None, T=4, r=8, X=P, A=True, B=True, Y=P, wsb=None, ws=P):
        ds = descs(shapes)
        n = len(ds) if nw is None else nw
        wp = ptrs([ctypes.addressof(d) for d in ds], len(ds))
        need = lib.qlora_linear_fwd_group_workspace(rows(*[d.rows for d in ds]), len(ds), ds[0].cols, T, r)
        return lib.qlora_linear_fwd_group(wp, n, X, T, ptrs([P2] * len(ds), len(ds)) if A else None,
                                          ptrs([P3] * len(ds), len(ds)) if B else None, r, 2.0,
                                          ptrs([Y] * len(ds), len(ds)), None, ws,
                                          need if wsb is None else wsb, None)

    assert call(nw=0) == L.QL_ERR_SHAPE
    assert call(shapes=((256, 256),) * 5) == L.QL_ERR_SHAPE
    assert call(shapes=((256, 256), (256, 320))) == L.QL_ERR_SHAPE  # layers of different K
    assert call(shapes=((256, 256), (100, 256))) == L.QL_ERR_SHAPE  # N % 8
    assert call(r=129) == L.QL_ERR_SHAPE
    assert call(A=False) == L.QL_ERR_NULL
    assert call(X=None) == L.QL_ERR_NULL
    assert call(Y=MIS) == L.QL_ERR_ALIGN
    assert call(wsb=0) == L.QL_ERR_WORKSPACE
    assert call(T=64, wsb=0) == L.QL_ERR_WORKSPACE  # the one-after-another path checks it too
    assert call(T=0) == L.QL_OK
    assert lib.qlora_linear_fwd_group(None, 1, P, 4, None, None, 0, 1.0, None, None, None, 0, None) == L.QL_ERR_NULL


def test_linear_bwd_rejects(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    need = lib.qlora_linear_bwd_workspace(256, 256, 64, 8)

    def call(w=None, X=P, dY=P2, T=64, A=P3, B=P, r=8, U=None, dX=P, dA=P2, dB=P3, acc=0, ws=P, wsb=need):
        return lib.qlora_linear_bwd(w if w is not None else _weight(L), X, dY, T, A, B, r, 2.0, U, dX, dA, dB, acc,
                                    ws, wsb, None)

    assert call(w=_weight(L, cols=100)) == L.QL_ERR_SHAPE
    assert call(acc=2) == L.QL_ERR_UNSUPPORTED
    assert call(r=0) == L.QL_ERR_SHAPE  # dA/dB requested without adapters
    assert call(dY=None) == L.QL_ERR_NULL
    assert call(X=None) == L.QL_ERR_NULL  # dA needs X
    assert call(dA=MIS) == L.QL_ERR_ALIGN
    assert call(wsb=100) == L.QL_ERR_WORKSPACE
    assert call(T=0) == L.QL_OK
    assert call(dX=None, dA=None, dB=None) == L.QL_OK  # nothing requested


def test_linear_bwd_group_rejects(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    def descs(shapes, dq=256):
        ws = []
        for rows, cols in shapes:
            w = L.QlNf4Weight()
            w.rows, w.cols, w.blocksize, w.dq_blocksize = rows, cols, 64, dq
            w.packed, w.absmax, w.c8, w.dq_scale, w.dq_mean = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
            ws.append(w)
        return ws

    def ptrs(vals, n):
        return (ctypes.c_void_p * max(n, 1))(*vals)

    def rows(*r):
        return (ctypes.c_int64 * len(r))(*r)

    # G of every layer, one set of gradient operands, the summed dX's split
    # partials: more than the largest single-layer workspace, less than the sum
    one = [lib.qlora_linear_bwd_workspace(n, 4096, 1024, 16) for n in (11008, 11008)]
    grp = lib.qlora_linear_bwd_group_workspace(rows(11008, 11008), 2, 4096, 1024, 16)
    assert max(one) < grp < sum(one) + 2 * 1024 * 64 * 2
    assert lib.qlora_linear_bwd_group_workspace(rows(256), 0, 256, 16, 8) == 0
    assert lib.qlora_linear_bwd_group_workspace(rows(*[256] * 5), 5, 256, 16, 8) == 0
    assert lib.qlora_linear_bwd_group_workspace(rows(256, 0), 2, 256, 16, 8) == 0
    assert lib.qlora_linear_bwd_group_workspace(None, 1, 256, 16, 8) == 0
    assert lib.qlora_linear_bwd_group_workspace(rows(256), 1, 256, 16, 129) == 0

    def call(shapes=((256, 256), (512, 256)), nw=None, T=64, r=8, X=P, dY=P2, A=True, B=True, U=False, dX=P,
             dA=True, dB=True, acc=0, wsb=None, ws=P, dq=(256, 256)):
        ds = []
        for sh, q in zip(shapes, dq + (256,) * len(shapes)):
            ds += descs((sh,), q)
        n = len(ds) if nw is None else nw
        wp = ptrs([ctypes.addressof(d) for d in ds], len(ds))
        need = lib.qlora_linear_bwd_group_workspace(rows(*[d.rows for d in ds]), len(ds), ds[0].cols, T, r)
        arr = lambda v: ptrs([v] * len(ds), len(ds))
        return lib.qlora_linear_bwd_group(wp, n, X, arr(dY), T, arr(P3) if A else None, arr(P) if B else None, r,
                                          2.0, arr(P2) if U else None, dX, arr(P2) if dA else None,
                                          arr(P3) if dB else None, acc, ws, need if wsb is None else wsb, None)

    assert call(nw=0) == L.QL_ERR_SHAPE
    assert call(shapes=((256, 256),) * 5) == L.QL_ERR_SHAPE
    assert call(shapes=((256, 256), (256, 320))) == L.QL_ERR_SHAPE  # layers of different K
    assert call(shapes=((256, 256), (100, 256))) == L.QL_ERR_SHAPE  # N % 8
    assert call(dq=(256, 0)) == L.QL_ERR_UNSUPPORTED  # formats mixed
    assert call(r=129) == L.QL_ERR_SHAPE
    assert call(r=0, A=False, B=False) == L.QL_ERR_SHAPE  # dA/dB requested without adapters
    assert call(acc=2) == L.QL_ERR_UNSUPPORTED
    assert call(A=False) == L.QL_ERR_NULL
    assert call(dY=None) == L.QL_ERR_NULL
    assert call(X=None) == L.QL_ERR_NULL  # dA needs X
    assert call(dX=MIS) == L.QL_ERR_ALIGN
    assert call(wsb=0) == L.QL_ERR_WORKSPACE
    assert call(T=0) == L.QL_OK
    assert call(dX=None, dA=False, dB=False) == L.QL_OK  # nothing requested
    assert lib.qlora_linear_bwd_group(None, 1, P, None, 4, None, None, 0, 1.0, None, P, None, None, 0, None, 0,
                                      None) == L.QL_ERR_NULL


def test_merge_rejects(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    def call(w=None, A=P2, B=P3, r=8, out=P):
        return lib.qlora_merge(w if w is not None else _weight(L), A, B, r, 0.5, out, None)

    assert call(w=_weight(L, cols=96)) == L.QL_ERR_SHAPE  # K % 64
    assert call(w=_weight(L, rows=100)) == L.QL_ERR_SHAPE  # N % 8
    assert call(r=129) == L.QL_ERR_SHAPE
    assert call(r=-1) == L.QL_ERR_SHAPE
    assert call(A=None) == L.QL_ERR_NULL
    assert call(B=MIS) == L.QL_ERR_ALIGN
    assert call(out=None) == L.QL_ERR_NULL
    assert call(w=_weight(L, c8=None)) == L.QL_ERR_NULL


def test_quant_error_rejects(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    need = lib.q4_quant_error_workspace(64, 4096, L.QL_F32)
    assert need > 0 and lib.q4_quant_error_workspace(0, 4, L.QL_F32) == 0

    def call(W=P, dt=L.QL_F32, rows=64, cols=4096, bs=64, grid=L.QL_GRID_UNIFORM, stats=P2, ws=P3, wsb=need):
        return lib.q4_quant_error(W, dt, rows, cols, bs, grid, stats, ws, wsb, None)

    assert call(rows=0) == L.QL_ERR_SHAPE
    assert call(bs=32) == L.QL_ERR_UNSUPPORTED
    assert call(dt=9) == L.QL_ERR_UNSUPPORTED
    assert call(grid=2) == L.QL_ERR_UNSUPPORTED
    assert call(W=None) == L.QL_ERR_NULL
    assert call(stats=MIS) == L.QL_ERR_ALIGN
    assert call(wsb=need - 1) == L.QL_ERR_WORKSPACE
    assert call(ws=None) == L.QL_ERR_WORKSPACE


def test_dropout_entries_reject(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    need = lib.qlora_linear_fwd_dropout_workspace(256, 256, 64, 8)
    assert need > lib.qlora_linear_fwd_workspace(256, 256, 64, 8)  # X * keep is staged

    def fwd(keep=P, p=0.1, wsb=need, T=64):
        return lib.qlora_linear_fwd_dropout(_weight(L), P, T, P2, P3, 8, 2.0, keep, p, P, None, P, wsb, None)

    assert fwd(keep=None) == L.QL_ERR_NULL
    assert fwd(keep=MIS) == L.QL_ERR_ALIGN
    assert fwd(p=1.0) == L.QL_ERR_UNSUPPORTED
    assert fwd(p=-0.1) == L.QL_ERR_UNSUPPORTED
    assert fwd(wsb=need - 1) == L.QL_ERR_WORKSPACE
    assert fwd(T=0) == L.QL_OK
    bneed = lib.qlora_linear_bwd_dropout_workspace(256, 256, 64, 8)

    def bwd(keep=P, p=0.1, wsb=bneed):
        return lib.qlora_linear_bwd_dropout(_weight(L), P, P2, 64, P3, P, 8, 2.0, keep, p, None, P, P2, P3, 0, P, wsb,
                                            None)

    assert bwd(keep=None) == L.QL_ERR_NULL
    assert bwd(p=1.5) == L.QL_ERR_UNSUPPORTED
    assert bwd(wsb=bneed - 1) == L.QL_ERR_WORKSPACE


def test_timer_ids(lib):
    from bit_nf4_quantized_16_amd import _lib as L

    assert lib.qlora_timer_arm(0) == L.QL_ERR_UNSUPPORTED
    assert lib.qlora_timer_arm(99) == L.QL_ERR_UNSUPPORTED
    assert lib.qlora_timer_arm(L.QL_KERNEL_GEMM_FWD) == L.QL_OK
    n = ctypes.c_int64(-1)
    ms = ctypes.c_double(-1)
    assert lib.qlora_timer_read(L.QL_KERNEL_GEMM_FWD, ctypes.byref(n), ctypes.byref(ms)) == L.QL_OK
    assert n.value == 0 and ms.value == 0.0
    assert lib.qlora_timer_disarm(L.QL_KERNEL_GEMM_FWD) == L.QL_OK
