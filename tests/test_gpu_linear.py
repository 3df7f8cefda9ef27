"""GPU parity of the LoRA linear layer on the NF4 base (forward: dequant-GEMV
for T <= 16, dequant-in-LDS MFMA GEMM above; backward: transposed dequant
GEMM for dX and the LoRA gradients) against the fp64 CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, bf16_to_np, f32_to_np, normwise_rel_err, oracle_weight

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import bit_nf4_quantized_16_amd as qn

    assert torch.cuda.is_available()
    return qn


def _run(qn, case, W=None, dq=True, accumulate_from=None):
    """Quantize case.W on the GPU, run forward and backward, compare all
    outputs with the oracle. Returns the errors."""
    W = case.W if W is None else W
    w = qn.quantize_weight(W.contiguous().cuda(), double_quant=dq)
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    s = case.scale
    Y, U = qn.qlora_linear_fwd(w, X, A, B, s)
    dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U)
    torch.cuda.synchronize()
    ref = oracle_weight(W.numpy(), double_quant=dq)
    Xn, dYn, An, Bn = (bf16_to_np(t) for t in (case.X, case.dY, case.A, case.B))
    H, Uo = oracle.lora_forward(Xn, ref["wd"], An, Bn, s)
    dXo, dAo, dBo, _, _ = oracle.lora_backward(Xn, dYn, ref["wd"], An, Bn, s)
    errs = dict(
        H=normwise_rel_err(bf16_to_np(Y), H),
        U=normwise_rel_err(f32_to_np(U), Uo),
        dX=normwise_rel_err(bf16_to_np(dX), dXo),
        dA=normwise_rel_err(f32_to_np(dA), dAo),
        dB=normwise_rel_err(f32_to_np(dB), dBo),
    )
    for k, v in errs.items():
        assert v <= TOL, "%s: %s error %.3e > %.0e (%s)" % (case.name, k, v, TOL, errs)
    return errs, (w, X, dY, A, B, Y, dX, dA, dB)


def test_tiny_256_config(qn):
    errs, _ = _run(qn, workloads.tiny_256())
    # the oracle's reduction is fp64 and the inputs bf16: the remaining error is
    # the bf16 rounding of the outputs, far inside the bar
    assert errs["H"] < 5e-3 and errs["dX"] < 5e-3


@pytest.mark.parametrize("T", [1, 2, 5, 16, 17, 31, 128, 300])
def test_token_counts_cross_gemv_and_gemm(qn, T):
    W = workloads.normal_weight(256, 320, 0.02, seed=T)
    case = workloads.lora_case("T%d" % T, W, T, 8, 16.0, 1 / 320, 0.05, seed=T)
    _run(qn, case)


@pytest.mark.parametrize("N,K,T,r", [(200, 320, 300, 5), (136, 64, 129, 1), (8, 128, 3, 3), (520, 1088, 257, 70),
                                     (264, 192, 40, 128), (64, 64, 1, 16)])
def test_ragged_shapes_and_ranks(qn, N, K, T, r):
    W = workloads.normal_weight(N, K, 0.02, seed=N + K)
    case = workloads.lora_case("N%dK%dT%dr%d" % (N, K, T, r), W, T, r, 2.0 * r, 1 / K, 0.05, seed=N * 7 + T)
    _run(qn, case)


# decode path: every rank-tile variant of the fused GEMV (1, 2, 3->4, 7->8 and
# 8 tiles of 16), a half last K step (K % 128 == 64), N below one 16-row tile,
# several passes over K (K = 4160: 33 steps of 128) and the base alone
@pytest.mark.parametrize("N,K,T,r", [(200, 320, 3, 5), (136, 64, 1, 24), (264, 192, 16, 40), (520, 1088, 7, 100),
                                     (8, 128, 2, 128), (96, 4160, 16, 16), (48, 4160, 5, 64), (72, 256, 1, 0),
                                     (24, 1472, 16, 8), (24, 1536, 16, 8), (40, 11008, 2, 16), (40, 11008, 3, 16),
                                     # more 256-wide steps per wave than are issued up front (the ring of
                                     # loads) for each width of x: T <= 2, <= 4, <= 8
                                     (24, 16448, 1, 16), (24, 8256, 4, 8), (24, 6208, 8, 8),
                                     # 2..5 steps per wave, all issued up front (K = 4096 .. 10240),
                                     # for the three narrowest widths of x (T = 1, 3, 6); the widths
                                     # whose register budget is smaller take the ring there instead
                                     (40, 4096, 1, 16), (40, 6144, 1, 16), (40, 8192, 1, 16), (40, 10240, 1, 16),
                                     (40, 4096, 3, 16), (40, 6144, 3, 16), (40, 8192, 3, 16), (40, 10240, 3, 16),
                                     (40, 4096, 6, 16), (40, 6144, 6, 16), (40, 8192, 6, 16), (40, 10240, 6, 16)])
def test_gemv_ranks_and_ragged_k(qn, N, K, T, r):
    W = workloads.normal_weight(N, K, 0.02, seed=N + 3 * K)
    case = workloads.lora_case("gemv_N%dK%dT%dr%d" % (N, K, T, r), W, T, r, 2.0 * max(r, 1), 1 / K, 0.05,
                               seed=N * 5 + T)
    if r == 0:
        w = qn.quantize_weight(W.cuda())
        Y, U = qn.qlora_linear_fwd(w, case.X.cuda())
        assert U is None
        ref = oracle_weight(W.numpy())
        H = bf16_to_np(case.X).astype(np.float64) @ ref["wd"].T
        assert normwise_rel_err(bf16_to_np(Y), H) <= TOL
    else:
        _run(qn, case)


@pytest.mark.parametrize("T", [1, 16])
def test_gemv_output_without_saved_u(qn, T):
    """The decode path gives the same Y, bit for bit, whether U goes to the
    caller's buffer or to the workspace."""
    W = workloads.normal_weight(264, 1024, 0.02, seed=7)
    case = workloads.lora_case("gemv_u", W, T, 16, 32.0, 1 / 1024, 0.05, seed=8)
    w = qn.quantize_weight(W.cuda())
    X, A, B = (t.cuda() for t in (case.X, case.A, case.B))
    Y1, U1 = qn.qlora_linear_fwd(w, X, A, B, case.scale)
    Y2, U2 = qn.qlora_linear_fwd(w, X, A, B, case.scale, save_u=False)
    assert U2 is None and torch.equal(Y1, Y2)


@pytest.mark.parametrize("N,K,T,r", [(264, 1024, 1, 16), (200, 4160, 5, 40), (96, 1536, 16, 128), (40, 11008, 3, 16)])
def test_gemv_local_u_is_bitwise_the_shared_one(qn, monkeypatch, N, K, T, r):
    """Forcing every workgroup to compute U itself (the path taken should the
    wait for the shared U ever run out) gives the same Y and U bit for bit."""
    W = workloads.normal_weight(N, K, 0.02, seed=K + r)
    case = workloads.lora_case("gemv_ulocal", W, T, r, 2.0 * r, 1 / K, 0.05, seed=T + r)
    w = qn.quantize_weight(W.cuda())
    X, A, B = (t.cuda() for t in (case.X, case.A, case.B))
    Y1, U1 = qn.qlora_linear_fwd(w, X, A, B, case.scale)
    monkeypatch.setenv("QLORA_NF4_GEMV_SPIN", "0")
    Y2, U2 = qn.qlora_linear_fwd(w, X, A, B, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(U1, U2)


@pytest.mark.parametrize("shapes,K,T,r", [(((264, 1024), (72, 1024), (520, 1024)), 1024, 1, 16),
                                           (((200, 4160), (8, 4160)), 4160, 5, 40),
                                           (((96, 1536), (136, 1536), (24, 1536), (264, 1536)), 1536, 16, 8),
                                           (((264, 320), (72, 320)), 320, 3, 0),
                                           (((4096, 4096),) * 3, 4096, 1, 16),
                                           (((11008, 4096),) * 2, 4096, 16, 64),
                                           (((256, 320), (520, 320)), 320, 40, 16)])
def test_fwd_group_is_bitwise_the_single_calls(qn, shapes, K, T, r):
    """Layers that share X in one grouped call give the same Y and U, bit for
    bit, as one qlora_linear_fwd call each (T <= 16: one GEMV launch over all
    of them; T = 40: the layers one after another)."""
    ws, As, Bs = [], [], []
    for i, (N, _) in enumerate(shapes):
        W = workloads.normal_weight(N, K, 0.02, seed=N + i)
        # (r = 0: the case's adapters of rank 1 are not passed)
        case = workloads.lora_case("grp%d" % i, W, T, max(r, 1), 2.0 * max(r, 1), 1 / K, 0.05, seed=T + 11 * i)
        ws.append(qn.quantize_weight(W.cuda()))
        As.append(case.A.cuda())
        Bs.append(case.B.cuda())
        if i == 0:
            X, s = case.X.cuda(), case.scale
    outs = qn.qlora_linear_fwd_group(ws, X, As if r else None, Bs if r else None, s)
    for i, w in enumerate(ws):
        Y1, U1 = qn.qlora_linear_fwd(w, X, As[i] if r else None, Bs[i] if r else None, s)
        Y2, U2 = outs[i]
        torch.cuda.synchronize()
        assert torch.equal(Y1, Y2), "layer %d: Y differs" % i
        assert (U1 is None and U2 is None) or torch.equal(U1, U2), "layer %d: U differs" % i


def test_without_double_quant(qn):
    case = workloads.tiny_256()
    _run(qn, case, dq=False)
    W = workloads.normal_weight(384, 512, 0.02, seed=5)
    _run(qn, workloads.lora_case("nodq_gemm", W, 200, 16, 32.0, 1 / 512, 0.05, seed=5), dq=False)


@pytest.mark.parametrize("T", [4, 96])
def test_zero_base_isolates_the_lora_branch(qn, T):
    # an all-zero W quantizes to code 7 (value 0): H = s U B^T and dX = G A
    # exactly in the oracle, so a broken LoRA branch cannot hide under the base
    W = torch.zeros(256, 256)
    case = workloads.lora_case("zeroW", W, T, 8, 16.0, 1 / 16, 0.5, seed=11)
    errs, _ = _run(qn, case)
    assert errs["H"] < 1e-2 and errs["dX"] < 1e-2


@pytest.mark.parametrize("T", [4, 160])
def test_big_adapter_variant(qn, T):
    W = workloads.normal_weight(256, 256, 0.02, seed=12)
    case = workloads.lora_case("bigB", W, T, 8, 16.0, 1 / 16, 1.0, seed=12)
    _run(qn, case)


@pytest.mark.parametrize("T", [8, 256])
def test_rank_zero_is_the_base_matmul(qn, T):
    W = workloads.normal_weight(256, 512, 0.02, seed=13)
    w = qn.quantize_weight(W.cuda())
    X = workloads.bf16_normal((T, 512), 1.0, 14).cuda()
    dY = workloads.bf16_normal((T, 256), 1.0, 15).cuda()
    Y, U = qn.qlora_linear_fwd(w, X)
    dX, dA, dB = qn.qlora_linear_bwd(w, None, dY)
    assert U is None and dA is None and dB is None
    ref = oracle_weight(W.numpy())
    assert normwise_rel_err(bf16_to_np(Y), bf16_to_np(X).astype(np.float64) @ ref["wd"].T) <= TOL
    assert normwise_rel_err(bf16_to_np(dX), bf16_to_np(dY).astype(np.float64) @ ref["wd"]) <= TOL


@pytest.mark.parametrize("T", [16, 512])
def test_fused_matmul_matches_torch_on_dequantized_weight(qn, T):
    """Library-routine check: the fused kernels against torch.matmul on the
    nf4_dequantize output (same W', fp32 matmul), at a tight tolerance."""
    W = workloads.normal_weight(1024, 2048, 0.02, seed=16)
    w = qn.quantize_weight(W.cuda())
    Wd = qn.nf4_dequantize(w).float()
    X = workloads.bf16_normal((T, 2048), 1.0, 17).cuda()
    dY = workloads.bf16_normal((T, 1024), 1.0, 18).cuda()
    Y, _ = qn.qlora_linear_fwd(w, X)
    dX, _, _ = qn.qlora_linear_bwd(w, None, dY)
    Yr = X.float() @ Wd.T
    dXr = dY.float() @ Wd
    assert normwise_rel_err(bf16_to_np(Y), Yr.cpu().numpy()) < 4e-3
    assert normwise_rel_err(bf16_to_np(dX), dXr.cpu().numpy()) < 4e-3


def test_bitwise_deterministic(qn):
    W = workloads.normal_weight(512, 512, 0.02, seed=19)
    case = workloads.lora_case("det", W, 300, 16, 32.0, 1 / 512, 0.05, seed=19)
    _, o1 = _run(qn, case)
    _, o2 = _run(qn, case)
    for a, b in zip(o1[5:], o2[5:]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("r", [16, 40, 128])
def test_split_projections_deterministic(qn, r):
    """At few tokens the LoRA projections split their reduction over several
    workgroups (the last to arrive adds the partials in order): parity with
    the oracle, and three calls in a row (reusing the workspace and its
    stale counters) give the same bits."""
    W = workloads.normal_weight(5120, 5120, 0.02, seed=23 + r)
    case = workloads.lora_case("splitproj_r%d" % r, W, 256, r, 2.0 * r, 1 / 5120, 0.05, seed=23)
    _, (w, X, dY, A, B, Y, dX, dA, dB) = _run(qn, case)
    for _ in range(2):
        Y2, U2 = qn.qlora_linear_fwd(w, X, A, B, case.scale)
        dX2, dA2, dB2 = qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, U=U2)
        dX3, dA3, dB3 = qn.qlora_linear_bwd(w, X, dY, A, B, case.scale)  # U recomputed
        torch.cuda.synchronize()
        for a, b in ((Y2, Y), (dX2, dX), (dA2, dA), (dB2, dB), (dX3, dX), (dA3, dA)):
            assert torch.equal(a, b)
        assert normwise_rel_err(f32_to_np(dB3), f32_to_np(dB)) < 1e-6


def test_gradient_accumulation(qn):
    W = workloads.normal_weight(256, 256, 0.02, seed=20)
    case = workloads.lora_case("acc", W, 64, 8, 16.0, 1 / 256, 0.05, seed=20)
    w = qn.quantize_weight(W.cuda())
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    _, dA1, dB1 = qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, need_dx=False)
    dA = dA1.clone()
    dB = dB1.clone()
    qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, need_dx=False, dA=dA, dB=dB, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dA, dA1 + dA1) and torch.equal(dB, dB1 + dB1)


def test_autograd_function(qn):
    W = workloads.normal_weight(256, 256, 0.02, seed=21)
    case = workloads.lora_case("autograd", W, 48, 8, 16.0, 1 / 256, 0.05, seed=21)
    w = qn.quantize_weight(W.cuda())
    X = case.X.cuda().requires_grad_(True)
    A = case.A.cuda().requires_grad_(True)
    B = case.B.cuda().requires_grad_(True)
    Y = qn.QLoRALinearFunction.apply(X, A, B, w, case.scale)
    Y.backward(case.dY.cuda())
    ref = oracle_weight(W.numpy())
    Xn, dYn, An, Bn = (bf16_to_np(t) for t in (case.X, case.dY, case.A, case.B))
    dXo, dAo, dBo, _, _ = oracle.lora_backward(Xn, dYn, ref["wd"], An, Bn, case.scale)
    assert normwise_rel_err(bf16_to_np(X.grad), dXo) <= TOL
    assert normwise_rel_err(bf16_to_np(A.grad), dAo) <= TOL
    assert normwise_rel_err(bf16_to_np(B.grad), dBo) <= TOL


def test_frozen_base_is_not_written(qn):
    W = workloads.normal_weight(256, 256, 0.02, seed=22)
    case = workloads.lora_case("frozen", W, 64, 8, 16.0, 1 / 256, 0.05, seed=22)
    w = qn.quantize_weight(W.cuda())
    before = [t.clone() for t in (w.packed, w.c8, w.dq_scale, w.dq_mean)]
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    Y, U = qn.qlora_linear_fwd(w, X, A, B, case.scale)
    qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, U=U)
    torch.cuda.synchronize()
    for a, b in zip(before, (w.packed, w.c8, w.dq_scale, w.dq_mean)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("tile", ["128", "256"])
@pytest.mark.parametrize("N,K,T,r", [(200, 320, 300, 5), (520, 1088, 257, 70), (256, 256, 17, 8), (768, 512, 600, 16),
                                     (264, 192, 40, 128), (1024, 320, 513, 64)])
def test_both_gemm_tiles(qn, monkeypatch, tile, N, K, T, r):
    """The forward and dX GEMMs come in a 128x128 and a 256x256 tile; force
    each (the launcher otherwise picks by shape) on ragged multi-tile cases."""
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", tile)
    W = workloads.normal_weight(N, K, 0.02, seed=N + 3 * K)
    case = workloads.lora_case("tile%s_N%dK%dT%dr%d" % (tile, N, K, T, r), W, T, r, 2.0 * r, 1 / K, 0.05, seed=T)
    _run(qn, case)


@pytest.mark.parametrize("splits", ["2", "3", "5"])
@pytest.mark.parametrize("N,K,T,r", [(512, 1024, 200, 16), (264, 2048, 300, 5), (1024, 640, 96, 64)])
def test_split_reduction(qn, monkeypatch, splits, N, K, T, r):
    """Split-K for grids too small to fill the chip: forced split counts of
    the 256x256 tile, ragged shapes, both GEMMs."""
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", "256")
    monkeypatch.setenv("QLORA_NF4_GEMM_SPLITS", splits)
    W = workloads.normal_weight(N, K, 0.02, seed=N + K + int(splits))
    case = workloads.lora_case("split%s_N%dK%dT%d" % (splits, N, K, T), W, T, r, 2.0 * r, 1 / K, 0.05, seed=T + 1)
    _run(qn, case)


@pytest.mark.parametrize("need_da,need_db", [(False, False), (True, False), (False, True)])
def test_long_batch_backward_with_gradients_skipped(qn, need_da, need_db):
    """T > 2048 (the adapter gradients split over tokens) with some of dA, dB
    not asked for; dX alone once crashed the caller's process in the
    workspace sizing."""
    T, N, K, r = 2300, 264, 320, 16
    W = workloads.normal_weight(N, K, 0.02, seed=31)
    case = workloads.lora_case("longT", W, T, r, 32.0, 1 / K, 0.05, seed=31)
    w = qn.quantize_weight(W.cuda())
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, need_da=need_da, need_db=need_db)
    torch.cuda.synchronize()
    ref = oracle_weight(W.numpy())
    Xn, dYn, An, Bn = (bf16_to_np(t) for t in (case.X, case.dY, case.A, case.B))
    dXo, dAo, dBo, _, _ = oracle.lora_backward(Xn, dYn, ref["wd"], An, Bn, case.scale)
    assert normwise_rel_err(bf16_to_np(dX), dXo) <= TOL
    assert (dA is None) == (not need_da) and (dB is None) == (not need_db)
    if need_da:
        assert normwise_rel_err(f32_to_np(dA), dAo) <= TOL
    if need_db:
        assert normwise_rel_err(f32_to_np(dB), dBo) <= TOL


def test_decode_calls_on_two_streams_at_once(qn):
    """Decode GEMVs (U handed over in tagged words inside each launch) issued
    on two streams at the same time, several rounds: every Y and U equals
    the same call made alone."""
    cases = []
    for i, (N, K, T, r) in enumerate([(4096, 4096, 1, 16), (11008, 4096, 16, 16), (1024, 4096, 5, 8),
                                      (4096, 11008, 1, 64)]):
        W = workloads.normal_weight(N, K, 0.02, seed=110 + i)
        X = workloads.bf16_normal((T, K), 1.0, seed=120 + i).cuda()
        A = workloads.bf16_normal((r, K), 1.0 / K, seed=130 + i).cuda()
        B = workloads.bf16_normal((N, r), 0.01, seed=140 + i).cuda()
        cases.append((qn.quantize_weight(W.cuda()), X, A, B))
    alone = []
    for w, X, A, B in cases:
        alone.append([t.clone() for t in qn.qlora_linear_fwd(w, X, A, B, 2.0)])
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        outs = []
        for i, (w, X, A, B) in enumerate(cases):
            with torch.cuda.stream(streams[i % 2]):
                outs.append(qn.qlora_linear_fwd(w, X, A, B, 2.0))
        torch.cuda.synchronize()
        for i, (o, a) in enumerate(zip(outs, alone)):
            for x, y in zip(o, a):
                assert torch.equal(x, y), "call %d, repetition %d" % (i, rep)
