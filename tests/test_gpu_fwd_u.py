"""The forward with U = X A^T computed inside the dequant GEMM launch (its
first workgroups hand U to the tiles through words tagged for the launch)
against the forward with a separate projection launch first: Y and U bit
for bit, the oracle within the usual bar, ragged token counts, and the
tile's local fallback (forced from the host, so every kernel still ends
normally). A captured forward (its tag mixes in an epoch word that a kernel
recorded before it advances at every replay) replayed with new inputs
equals the eager calls bit for bit, also when the tiles form U themselves.
The same for the backward with G = s dY B inside the dX launch (dX, dA, dB,
subsets of them, accumulation, the autograd wrapper)."""

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


# (N, K, T, r): several tiles and token blocks, ragged T (a last 16-token
# block and a last 256-token tile that are partial), rank 8 and 16
SHAPES = [(1024, 512, 300, 16), (520, 256, 33, 8), (2048, 1024, 257, 16), (264, 192, 1000, 8)]


def _case(N, K, T, r, seed):
    W = workloads.normal_weight(N, K, 0.02, seed=seed)
    return W, workloads.lora_case("fwd_u_N%dK%dT%d" % (N, K, T), W, T, r, 2.0 * r, 1 / K, 0.05, seed=seed + 1)


def _fwd(qn, w, case):
    X, A, B = (t.cuda() for t in (case.X, case.A, case.B))
    Y, U = qn.qlora_linear_fwd(w, X, A, B, case.scale)
    torch.cuda.synchronize()
    return Y, U


@pytest.mark.parametrize("N,K,T,r", SHAPES)
def test_in_launch_u_equals_prepass_and_oracle(qn, monkeypatch, N, K, T, r):
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", "256")
    W, case = _case(N, K, T, r, seed=N + T)
    assert qn.lib.qlora_linear_fwd_u_in_launch(N, K, T, r) == 1
    w = qn.quantize_weight(W.cuda())
    Y1, U1 = _fwd(qn, w, case)
    monkeypatch.setenv("QLORA_NF4_FWD_U", "prepass")
    assert qn.lib.qlora_linear_fwd_u_in_launch(N, K, T, r) == 0
    Y2, U2 = _fwd(qn, w, case)
    assert torch.equal(U1, U2) and torch.equal(Y1, Y2)
    ref = oracle_weight(W.numpy())
    H, Uo = oracle.lora_forward(bf16_to_np(case.X), ref["wd"], bf16_to_np(case.A), bf16_to_np(case.B), case.scale)
    assert normwise_rel_err(bf16_to_np(Y1), H) <= TOL
    assert normwise_rel_err(f32_to_np(U1), Uo) <= TOL


def test_in_launch_u_at_the_7b_mlp_shape(qn, monkeypatch):
    """The 7B gate shape at T = 1024, r = 16 (the default plan takes the
    in-launch U there): bitwise equal to the separate projection."""
    N, K, T, r = 11008, 4096, 1024, 16
    assert qn.lib.qlora_linear_fwd_u_in_launch(N, K, T, r) == 1
    W = workloads.normal_weight(N, K, 0.02, seed=5)
    X = workloads.bf16_normal((T, K), 1.0, seed=6).cuda()
    A = workloads.bf16_normal((r, K), 1.0 / K, seed=7).cuda()
    B = workloads.bf16_normal((N, r), 0.01, seed=8).cuda()
    w = qn.quantize_weight(W.cuda())
    Y1, U1 = qn.qlora_linear_fwd(w, X, A, B, 2.0)
    torch.cuda.synchronize()
    monkeypatch.setenv("QLORA_NF4_FWD_U", "prepass")
    Y2, U2 = qn.qlora_linear_fwd(w, X, A, B, 2.0)
    torch.cuda.synchronize()
    assert torch.equal(U1, U2) and torch.equal(Y1, Y2)


@pytest.mark.parametrize("N,K,T,r", SHAPES[:2])
def test_local_u_fallback(qn, monkeypatch, N, K, T, r):
    """QLORA_NF4_GEMM_SPIN=-1: every tile forms its U values itself (fp32
    sums in k order) instead of reading the words. U_out still comes from
    the projection workgroups (bit for bit); Y is within the oracle's bar
    and within bf16 rounding of the separate-projection result."""
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", "256")
    W, case = _case(N, K, T, r, seed=3 * N + T)
    w = qn.quantize_weight(W.cuda())
    Y2, U2 = _fwd(qn, w, case)
    monkeypatch.setenv("QLORA_NF4_GEMM_SPIN", "-1")
    Y1, U1 = _fwd(qn, w, case)
    assert torch.equal(U1, U2)
    assert normwise_rel_err(bf16_to_np(Y1), bf16_to_np(Y2).astype("float64")) <= 1e-2
    ref = oracle_weight(W.numpy())
    H, _ = oracle.lora_forward(bf16_to_np(case.X), ref["wd"], bf16_to_np(case.A), bf16_to_np(case.B), case.scale)
    assert normwise_rel_err(bf16_to_np(Y1), H) <= TOL


@pytest.mark.parametrize("spin", [None, "-1"])
def test_captured_forward_replays_equal_eager_in_launch(qn, monkeypatch, spin):
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", "256")
    if spin is not None:
        monkeypatch.setenv("QLORA_NF4_GEMM_SPIN", spin)
    N, K, T, r = 1024, 512, 300, 16
    W, case = _case(N, K, T, r, seed=77)
    w = qn.quantize_weight(W.cuda())
    A, B = case.A.cuda(), case.B.cuda()
    X = torch.empty(T, K, dtype=torch.bfloat16, device="cuda")
    xs = [workloads.bf16_normal((T, K), 1.0, seed=80 + i).cuda() for i in range(4)]
    X.copy_(xs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qn.qlora_linear_fwd(w, X, A, B, case.scale)  # warm-up before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Y, U = qn.qlora_linear_fwd(w, X, A, B, case.scale)
    for rep in range(1, 7):
        X.copy_(xs[rep % 4])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Ye, Ue = qn.qlora_linear_fwd(w, xs[rep % 4], A, B, case.scale)
        torch.cuda.synchronize()
        assert torch.equal(Y, Ye) and torch.equal(U, Ue), "replay %d differs from the eager call" % rep


def test_in_launch_u_without_u_out(qn, monkeypatch):
    """save_u=False (U_out NULL): the projection workgroups still hand U to
    the tiles; Y equals the separate projection's bit for bit."""
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", "256")
    N, K, T, r = 2048, 1024, 257, 16
    W, case = _case(N, K, T, r, seed=91)
    w = qn.quantize_weight(W.cuda())
    X, A, B = (t.cuda() for t in (case.X, case.A, case.B))
    Y1, U1 = qn.qlora_linear_fwd(w, X, A, B, case.scale, save_u=False)
    monkeypatch.setenv("QLORA_NF4_FWD_U", "prepass")
    Y2, _ = qn.qlora_linear_fwd(w, X, A, B, case.scale, save_u=False)
    torch.cuda.synchronize()
    assert U1 is None and torch.equal(Y1, Y2)


# (N, K, T, r) where the dX GEMM (output K, reduction N) runs unsplit 256
# tiles with the tile forced: G = s dY B inside its launch
BWD_SHAPES = [(512, 1024, 300, 16), (256, 520 // 8 * 64, 33, 8), (1024, 2048, 257, 16)]


def _bwd(qn, w, case, U, **kw):
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    out = qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, U=U, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("N,K,T,r", BWD_SHAPES)
@pytest.mark.parametrize("with_u", [True, False])
def test_in_launch_g_equals_prepass_and_oracle(qn, monkeypatch, N, K, T, r, with_u):
    """dX, dA and dB with G computed by the dX GEMM's first workgroups (which
    also write G^T and, from U_saved, U^T for the gradient kernel) equal
    the separate projection's bit for bit, with U saved or recomputed, and
    stay within the oracle's bar."""
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", "256")
    W, case = _case(N, K, T, r, seed=7 * N + T)
    assert qn.lib.qlora_linear_bwd_g_in_launch(N, K, T, r) == 1
    w = qn.quantize_weight(W.cuda())
    _, U = _fwd(qn, w, case)
    U = U if with_u else None
    g1 = _bwd(qn, w, case, U)
    monkeypatch.setenv("QLORA_NF4_FWD_U", "prepass")
    assert qn.lib.qlora_linear_bwd_g_in_launch(N, K, T, r) == 0
    g2 = _bwd(qn, w, case, U)
    for a, b, name in zip(g1, g2, ("dX", "dA", "dB")):
        assert torch.equal(a, b), name
    ref = oracle_weight(W.numpy())
    dXo, dAo, dBo, _, _ = oracle.lora_backward(bf16_to_np(case.X), bf16_to_np(case.dY), ref["wd"],
                                               bf16_to_np(case.A), bf16_to_np(case.B), case.scale)
    assert normwise_rel_err(bf16_to_np(g1[0]), dXo) <= TOL
    assert normwise_rel_err(f32_to_np(g1[1]), dAo) <= TOL
    assert normwise_rel_err(f32_to_np(g1[2]), dBo) <= TOL


def test_in_launch_g_dx_only_and_7b_down(qn, monkeypatch):
    """The 7B down projection at T = 1024 (its dX GEMM has 172 tiles, the
    default plan puts G inside): dX alone and all three gradients equal the
    separate projection's bit for bit."""
    N, K, T, r = 4096, 11008, 1024, 16
    assert qn.lib.qlora_linear_bwd_g_in_launch(N, K, T, r) == 1
    W = workloads.normal_weight(N, K, 0.02, seed=15)
    X = workloads.bf16_normal((T, K), 1.0, seed=16).cuda()
    dY = workloads.bf16_normal((T, N), 1.0, seed=17).cuda()
    A = workloads.bf16_normal((r, K), 1.0 / K, seed=18).cuda()
    B = workloads.bf16_normal((N, r), 0.01, seed=19).cuda()
    w = qn.quantize_weight(W.cuda())
    _, U = qn.qlora_linear_fwd(w, X, A, B, 2.0)
    a1 = qn.qlora_linear_bwd(w, X, dY, A, B, 2.0, U=U)
    x1, _, _ = qn.qlora_linear_bwd(w, X, dY, A, B, 2.0, U=U, need_da=False, need_db=False)
    torch.cuda.synchronize()
    monkeypatch.setenv("QLORA_NF4_FWD_U", "prepass")
    a2 = qn.qlora_linear_bwd(w, X, dY, A, B, 2.0, U=U)
    torch.cuda.synchronize()
    for a, b, name in zip(a1, a2, ("dX", "dA", "dB")):
        assert torch.equal(a, b), name
    assert torch.equal(x1, a2[0])


def test_in_launch_g_local_fallback(qn, monkeypatch):
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", "256")
    N, K, T, r = BWD_SHAPES[0]
    W, case = _case(N, K, T, r, seed=99)
    w = qn.quantize_weight(W.cuda())
    _, U = _fwd(qn, w, case)
    g2 = _bwd(qn, w, case, U)
    monkeypatch.setenv("QLORA_NF4_GEMM_SPIN", "-1")
    g1 = _bwd(qn, w, case, U)
    assert torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])  # G^T and U^T come from the projection
    assert normwise_rel_err(bf16_to_np(g1[0]), bf16_to_np(g2[0]).astype("float64")) <= 1e-2
    ref = oracle_weight(W.numpy())
    dXo, _, _, _, _ = oracle.lora_backward(bf16_to_np(case.X), bf16_to_np(case.dY), ref["wd"], bf16_to_np(case.A),
                                           bf16_to_np(case.B), case.scale)
    assert normwise_rel_err(bf16_to_np(g1[0]), dXo) <= TOL


@pytest.mark.parametrize("spin", [None, "-1"])
def test_captured_backward_replays_equal_eager_in_launch(qn, monkeypatch, spin):
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", "256")
    if spin is not None:
        monkeypatch.setenv("QLORA_NF4_GEMM_SPIN", spin)
    N, K, T, r = BWD_SHAPES[0]
    W, case = _case(N, K, T, r, seed=123)
    w = qn.quantize_weight(W.cuda())
    X, A, B = case.X.cuda(), case.A.cuda(), case.B.cuda()
    _, U = qn.qlora_linear_fwd(w, X, A, B, case.scale)
    dY = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    dys = [workloads.bf16_normal((T, N), 1.0, seed=130 + i).cuda() for i in range(4)]
    dY.copy_(dys[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, U=U)  # warm-up before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, U=U)
    for rep in range(1, 7):
        dY.copy_(dys[rep % 4])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = qn.qlora_linear_bwd(w, X, dys[rep % 4], A, B, case.scale, U=U)
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), "replay %d differs from the eager call" % rep


@pytest.mark.parametrize("need", [(True, True, False), (True, False, True), (False, True, False), (False, False, True)])
def test_in_launch_g_partial_outputs_and_accumulation(qn, monkeypatch, need):
    """Subsets of (dX, dA, dB), and dA, dB added to existing gradients, with
    G inside the dX launch where dX is asked for: bitwise the separate
    projection's results."""
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", "256")
    N, K, T, r = BWD_SHAPES[2]
    need_dx, need_da, need_db = need
    W, case = _case(N, K, T, r, seed=31 + sum(need))
    w = qn.quantize_weight(W.cuda())
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    _, U = qn.qlora_linear_fwd(w, X, A, B, case.scale)
    dA0 = workloads.bf16_normal((r, K), 0.1, seed=40).float().cuda()
    dB0 = workloads.bf16_normal((N, r), 0.1, seed=41).float().cuda()

    def run():
        dA, dB = dA0.clone(), dB0.clone()
        out = qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, U=U, need_dx=need_dx, need_da=need_da, need_db=need_db,
                                  dA=dA if need_da else None, dB=dB if need_db else None, accumulate=True)
        torch.cuda.synchronize()
        return out

    assert qn.lib.qlora_linear_bwd_g_in_launch(N, K, T, r) == 1
    g1 = run()
    monkeypatch.setenv("QLORA_NF4_FWD_U", "prepass")
    g2 = run()
    for a, b, want, name in zip(g1, g2, need, ("dX", "dA", "dB")):
        assert (a is None) == (not want) and (b is None) == (not want), name
        if want:
            assert torch.equal(a, b), name


def test_autograd_with_u_and_g_inside_the_launches(qn, monkeypatch):
    """The autograd wrapper at a shape where both the forward's U and the
    backward's G run inside their GEMM launches: gradients bitwise those of
    the separate projections, and within the oracle's bar."""
    monkeypatch.setenv("QLORA_NF4_GEMM_TILE", "256")
    N, K, T, r = 512, 1024, 300, 16
    assert qn.lib.qlora_linear_fwd_u_in_launch(N, K, T, r) == 1
    assert qn.lib.qlora_linear_bwd_g_in_launch(N, K, T, r) == 1
    W, case = _case(N, K, T, r, seed=77)
    w = qn.quantize_weight(W.cuda())

    def run():
        X = case.X.cuda().requires_grad_(True)
        A = case.A.cuda().requires_grad_(True)
        B = case.B.cuda().requires_grad_(True)
        Y = qn.QLoRALinearFunction.apply(X, A, B, w, case.scale)
        Y.backward(case.dY.cuda())
        torch.cuda.synchronize()
        return Y.detach(), X.grad, A.grad, B.grad

    r1 = run()
    monkeypatch.setenv("QLORA_NF4_FWD_U", "prepass")
    r2 = run()
    for a, b, name in zip(r1, r2, ("Y", "dX", "dA", "dB")):
        assert torch.equal(a, b), name
    ref = oracle_weight(W.numpy())
    dXo, dAo, dBo, _, _ = oracle.lora_backward(bf16_to_np(case.X), bf16_to_np(case.dY), ref["wd"],
                                               bf16_to_np(case.A), bf16_to_np(case.B), case.scale)
    assert normwise_rel_err(bf16_to_np(r1[1]), dXo) <= TOL
    assert normwise_rel_err(f32_to_np(r1[2].float()), dAo) <= TOL
    assert normwise_rel_err(f32_to_np(r1[3].float()), dBo) <= TOL


@pytest.mark.parametrize("N,K", [(11008, 4096), (4096, 11008)])
def test_in_launch_u_and_g_at_t4096(qn, monkeypatch, N, K):
    """T = 4096, r = 16 at the 7B MLP shapes: 256 projection workgroups and
    688 tiles, so the tiles run in several rounds after the projection
    workgroups. Forward (U inside) and backward (G inside) bitwise the
    separate projections'."""
    T, r = 4096, 16
    assert qn.lib.qlora_linear_fwd_u_in_launch(N, K, T, r) == 1
    assert qn.lib.qlora_linear_bwd_g_in_launch(N, K, T, r) == 1
    W = workloads.normal_weight(N, K, 0.02, seed=N // 64 + 1)
    X = workloads.bf16_normal((T, K), 1.0, seed=50).cuda()
    dY = workloads.bf16_normal((T, N), 1.0, seed=51).cuda()
    A = workloads.bf16_normal((r, K), 1.0 / K, seed=52).cuda()
    B = workloads.bf16_normal((N, r), 0.01, seed=53).cuda()
    w = qn.quantize_weight(W.cuda())

    def run():
        Y, U = qn.qlora_linear_fwd(w, X, A, B, 2.0)
        g = qn.qlora_linear_bwd(w, X, dY, A, B, 2.0, U=U)
        torch.cuda.synchronize()
        return (Y, U) + tuple(g)

    r1 = run()
    monkeypatch.setenv("QLORA_NF4_FWD_U", "prepass")
    r2 = run()
    for a, b, name in zip(r1, r2, ("Y", "U", "dX", "dA", "dB")):
        assert torch.equal(a, b), name


def test_in_launch_calls_on_two_streams_at_once(qn):
    """Two forwards with U inside (7B gate and up shapes) and two backwards
    with G inside (down shape) issued on two streams at the same time, so
    their projection workgroups and tiles share the chip: every output
    equals the same call made alone."""
    T, r = 1024, 16
    shapes = [(11008, 4096), (11008, 4096), (4096, 11008), (4096, 11008)]
    cases = []
    for i, (N, K) in enumerate(shapes):
        W = workloads.normal_weight(N, K, 0.02, seed=60 + i)
        X = workloads.bf16_normal((T, K), 1.0, seed=70 + i).cuda()
        dY = workloads.bf16_normal((T, N), 1.0, seed=80 + i).cuda()
        A = workloads.bf16_normal((r, K), 1.0 / K, seed=90 + i).cuda()
        B = workloads.bf16_normal((N, r), 0.01, seed=100 + i).cuda()
        cases.append((qn.quantize_weight(W.cuda()), X, dY, A, B))

    def call(i):
        w, X, dY, A, B = cases[i]
        if i < 2:
            return qn.qlora_linear_fwd(w, X, A, B, 2.0)
        return qn.qlora_linear_bwd(w, X, dY, A, B, 2.0)

    alone = []
    for i in range(4):
        alone.append([t.clone() for t in call(i) if t is not None])
        torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    together = [None] * 4
    for rep in range(3):
        for pair in ((0, 1), (2, 3)):
            with torch.cuda.stream(s1):
                together[pair[0]] = call(pair[0])
            with torch.cuda.stream(s2):
                together[pair[1]] = call(pair[1])
        torch.cuda.synchronize()
        for i in range(4):
            got = [t for t in together[i] if t is not None]
            for a, b in zip(got, alone[i]):
                assert torch.equal(a, b), "call %d, repetition %d" % (i, rep)
