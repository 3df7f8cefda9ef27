"""GPU parity of the grouped backward (qlora_linear_bwd_group): layers that
read the same X, their input gradients summed in one dequant GEMM launch,
against the fp64 CPU oracle (the sum of each layer's oracle backward), and
against the single-layer call where the two must agree bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, bf16_to_np, f32_to_np, normwise_rel_err, oracle_cols, oracle_constants, oracle_weight
from gpu_util import sample_indices

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import bit_nf4_quantized_16_amd as qn

    assert torch.cuda.is_available()
    return qn


def _layers(shapes, K, T, r, seed, zero_w=False):
    """Seeded weights and adapters of layers that share X (the first case's)."""
    cases = []
    for i, N in enumerate(shapes):
        W = torch.zeros(N, K) if zero_w else workloads.normal_weight(N, K, 0.02, seed=seed + 13 * i)
        cases.append(workloads.lora_case("grp%d" % i, W, T, max(r, 1), 2.0 * max(r, 1), 1 / K, 0.05,
                                         seed=seed + 7 * i))
    return cases


@pytest.mark.parametrize("shapes,K,T,r", [((264, 72), 320, 40, 8),
                                           ((256, 520, 64), 1024, 300, 16),
                                           ((200, 8, 136, 96), 1536, 17, 40),
                                           ((1024, 512), 640, 700, 64),
                                           ((264, 320), 256, 33, 0)])
def test_bwd_group_matches_oracle(qn, shapes, K, T, r):
    cases = _layers(shapes, K, T, r, seed=T + K)
    s = cases[0].scale
    X = cases[0].X
    ws = [qn.quantize_weight(c.W.cuda()) for c in cases]
    dYs = [c.dY.cuda() for c in cases]
    As = [c.A.cuda() for c in cases] if r else None
    Bs = [c.B.cuda() for c in cases] if r else None
    Us = [qn.qlora_linear_fwd(w, X.cuda(), As[i], Bs[i], s)[1] for i, w in enumerate(ws)] if r else None
    dX, dAs, dBs = qn.qlora_linear_bwd_group(ws, X.cuda(), dYs, As, Bs, s, Us=Us, need_da=r > 0, need_db=r > 0)
    torch.cuda.synchronize()
    Xn = bf16_to_np(X)
    dXo = np.zeros((T, K))
    for i, c in enumerate(cases):
        wd = oracle_weight(c.W.numpy())["wd"]
        An = bf16_to_np(c.A) if r else np.zeros((1, K), np.float32)
        Bn = bf16_to_np(c.B) if r else np.zeros((c.W.shape[0], 1), np.float32)
        dXi, dAo, dBo, _, _ = oracle.lora_backward(Xn, bf16_to_np(c.dY), wd, An, Bn, s)
        dXo += dXi
        if r:
            assert normwise_rel_err(f32_to_np(dAs[i]), dAo) <= TOL, "layer %d: dA" % i
            assert normwise_rel_err(f32_to_np(dBs[i]), dBo) <= TOL, "layer %d: dB" % i
    err = normwise_rel_err(bf16_to_np(dX), dXo)
    assert err <= TOL, "dX error %.3e" % err


@pytest.mark.parametrize("T", [40, 1024])
def test_bwd_group_zero_base_isolates_the_rank_steps(qn, T):
    """All weights zero (codes 7): dX = sum of G_i A_i, which only the rank
    steps of each layer (one per layer, on different splits) produce."""
    K, r = 512, 16
    cases = _layers((264, 512, 128), K, T, r, seed=5, zero_w=True)
    for c in cases:  # adapters big enough to dominate
        c.B.copy_(c.B.float().mul(20.0).bfloat16())
    s = cases[0].scale
    ws = [qn.quantize_weight(c.W.cuda()) for c in cases]
    dX, _, _ = qn.qlora_linear_bwd_group(ws, cases[0].X.cuda(), [c.dY.cuda() for c in cases],
                                         [c.A.cuda() for c in cases], [c.B.cuda() for c in cases], s,
                                         need_da=False, need_db=False)
    torch.cuda.synchronize()
    Xn = bf16_to_np(cases[0].X)
    dXo = sum(oracle.lora_backward(Xn, bf16_to_np(c.dY), np.zeros((c.W.shape[0], K), np.float32), bf16_to_np(c.A),
                                   bf16_to_np(c.B), s)[0] for c in cases)
    assert np.max(np.abs(dXo)) > 0
    err = normwise_rel_err(bf16_to_np(dX), dXo)
    assert err <= TOL, "dX error %.3e" % err


@pytest.mark.parametrize("N,K,T,r", [(264, 320, 40, 8), (11008, 4096, 1024, 16), (4096, 11008, 1024, 16),
                                     (4096, 4096, 1024, 16), (1024, 512, 64, 0)])
def test_bwd_group_of_one_is_bitwise_the_single_call(qn, N, K, T, r):
    """One layer: dX, dA and dB equal qlora_linear_bwd's bit for bit (the same
    plan and accumulation order; the down shape's single call forms G inside
    its dX launch, which gives the same bits as the projection launch)."""
    case = workloads.lora_case("one", workloads.normal_weight(N, K, 0.02, seed=N), T, max(r, 1), 32.0, 1 / K, 0.01,
                               seed=K)
    w = qn.quantize_weight(case.W.cuda())
    X, dY = case.X.cuda(), case.dY.cuda()
    A, B = (case.A.cuda(), case.B.cuda()) if r else (None, None)
    s = case.scale
    U = qn.qlora_linear_fwd(w, X, A, B, s)[1] if r else None
    dX1, dA1, dB1 = qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U, need_da=r > 0, need_db=r > 0)
    dX2, dA2, dB2 = qn.qlora_linear_bwd_group([w], X, [dY], [A] if r else None, [B] if r else None, s,
                                              Us=[U] if r else None, need_da=r > 0, need_db=r > 0)
    torch.cuda.synchronize()
    assert torch.equal(dX1, dX2)
    if r:
        assert torch.equal(dA1, dA2[0]) and torch.equal(dB1, dB2[0])


@pytest.mark.parametrize("shapes,K,T", [((256, 512), 1024, 300), ((11008, 11008), 4096, 1024),
                                        ((4096, 4096, 4096), 4096, 1024), ((1024, 2048), 512, 4096)])
def test_bwd_group_rank0_is_the_stacked_weight(qn, shapes, K, T):
    """Without adapters and without double quantization (blockwise
    constants, so the stacked weight's codes and constants are the layers'
    concatenated), the grouped dX equals one qlora_linear_bwd on the weight
    stacked along N with dY concatenated along N, bit for bit: the same
    reduction steps in the same order under the same plan."""
    ws, dYs = [], []
    for i, N in enumerate(shapes):
        W = workloads.normal_weight(N, K, 0.02, seed=N + i)
        ws.append(qn.quantize_weight(W.cuda(), double_quant=False))
        dYs.append(workloads.bf16_normal((T, N), 1.0, seed=T + i).cuda())
    stacked = qn.NF4Weight(sum(shapes), K, torch.cat([w.packed for w in ws]), absmax=torch.cat([w.absmax for w in ws]))
    dY_cat = torch.cat(dYs, dim=1).contiguous()
    X = workloads.bf16_normal((T, K), 1.0, seed=1).cuda()
    dX1, _, _ = qn.qlora_linear_bwd(stacked, X, dY_cat, need_da=False, need_db=False)
    dX2, _, _ = qn.qlora_linear_bwd_group(ws, X, dYs, need_da=False, need_db=False)
    torch.cuda.synchronize()
    assert torch.equal(dX1, dX2)


def test_bwd_group_gradient_accumulation(qn):
    cases = _layers((264, 136), 320, 48, 8, seed=3)
    s = cases[0].scale
    ws = [qn.quantize_weight(c.W.cuda()) for c in cases]
    X = cases[0].X.cuda()
    args = (ws, X, [c.dY.cuda() for c in cases], [c.A.cuda() for c in cases], [c.B.cuda() for c in cases], s)
    _, dA1, dB1 = qn.qlora_linear_bwd_group(*args, need_dx=False)
    dA0 = [torch.full_like(a, 0.5) for a in dA1]
    dB0 = [torch.full_like(b, -0.25) for b in dB1]
    dAacc = [a.clone() for a in dA0]
    dBacc = [b.clone() for b in dB0]
    qn.qlora_linear_bwd_group(*args, need_dx=False, dAs=dAacc, dBs=dBacc, accumulate=True)
    torch.cuda.synchronize()
    for i in range(len(ws)):
        torch.testing.assert_close(dAacc[i], dA0[i] + dA1[i], rtol=1e-6, atol=1e-6)
        torch.testing.assert_close(dBacc[i], dB0[i] + dB1[i], rtol=1e-6, atol=1e-6)


def test_bwd_group_graph_replays(qn):
    """Captured once, replayed with new dY each time: every replay equals the
    eager call bit for bit."""
    cases = _layers((11008, 11008), 4096, 1024, 16, seed=9)
    s = cases[0].scale
    ws = [qn.quantize_weight(c.W.cuda()) for c in cases]
    X = cases[0].X.cuda()
    As = [c.A.cuda() for c in cases]
    Bs = [c.B.cuda() for c in cases]
    dYs = [c.dY.cuda() for c in cases]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qn.qlora_linear_bwd_group(ws, X, dYs, As, Bs, s, need_da=False, need_db=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dXg, _, _ = qn.qlora_linear_bwd_group(ws, X, dYs, As, Bs, s, need_da=False, need_db=False)
    for rep in range(3):
        for i, d in enumerate(dYs):
            d.copy_(workloads.bf16_normal(tuple(d.shape), 1.0, seed=100 * rep + i).cuda())
        graph.replay()
        torch.cuda.synchronize()
        want, _, _ = qn.qlora_linear_bwd_group(ws, X, dYs, As, Bs, s, need_da=False, need_db=False)
        torch.cuda.synchronize()
        assert torch.equal(dXg, want), "replay %d" % rep


def test_bwd_group_full_size_gate_up(qn):
    """The 7B MLP's gate and up (11008x4096 each, T = 1024, r = 16, as the
    bench step runs them): the summed dX on sampled columns against the
    oracle, which dequantizes those columns of both weights itself."""
    print("full-size grouped case gate+up", flush=True)
    cases = [workloads.mlp_7b("gate"), workloads.mlp_7b("up")]
    s = cases[0].scale
    X = cases[0].X
    ws = [qn.quantize_weight(c.W.cuda()) for c in cases]
    dX, dAs, dBs = qn.qlora_linear_bwd_group(ws, X.cuda(), [c.dY.cuda() for c in cases],
                                             [c.A.cuda() for c in cases], [c.B.cuda() for c in cases], s)
    torch.cuda.synchronize()
    K = cases[0].W.shape[1]
    cols = sample_indices(K, 24, seed=K + 5)
    Xn = bf16_to_np(X)
    dXo = 0.0
    for i, c in enumerate(cases):
        Wn = c.W.numpy()
        wd_c = oracle_cols(Wn, cols, oracle_constants(Wn))
        dXi, dAi, _, _, _ = oracle.lora_backward(Xn[:, cols], bf16_to_np(c.dY), wd_c, bf16_to_np(c.A)[:, cols],
                                                 bf16_to_np(c.B), s)
        dXo = dXo + dXi
        assert normwise_rel_err(f32_to_np(dAs[i])[:, cols], dAi) <= TOL, "layer %d: dA" % i
    err = normwise_rel_err(bf16_to_np(dX)[:, cols], dXo)
    assert err <= TOL, "dX error %.3e" % err


@pytest.mark.parametrize("shapes,K,T,r", [((264, 512, 128), 320, 48, 8), ((1024, 1024, 1024), 2048, 512, 16)])
def test_group_autograd_function(qn, shapes, K, T, r):
    """QLoRAGroupFunction: the grouped forward and backward through autograd;
    X receives the summed input gradient of the layers, each adapter its own
    (against the oracle)."""
    cases = _layers(shapes, K, T, r, seed=31)
    s = cases[0].scale
    ws = [qn.quantize_weight(c.W.cuda()) for c in cases]
    X = cases[0].X.cuda().requires_grad_(True)
    ad = []
    for c in cases:
        ad += [c.A.cuda().requires_grad_(True), c.B.cuda().requires_grad_(True)]
    Ys = qn.QLoRAGroupFunction.apply(X, s, ws, *ad)
    torch.autograd.backward(Ys, [c.dY.cuda() for c in cases])
    Xn = bf16_to_np(cases[0].X)
    dXo = 0.0
    for i, c in enumerate(cases):
        An, Bn = bf16_to_np(c.A), bf16_to_np(c.B)
        wd = oracle_weight(c.W.numpy())["wd"]
        H, _ = oracle.lora_forward(Xn, wd, An, Bn, s)
        assert normwise_rel_err(bf16_to_np(Ys[i]), H) <= TOL, "layer %d: Y" % i
        dXi, dAo, dBo, _, _ = oracle.lora_backward(Xn, bf16_to_np(c.dY), wd, An, Bn, s)
        dXo = dXo + dXi
        assert normwise_rel_err(bf16_to_np(ad[2 * i].grad), dAo) <= TOL, "layer %d: dA" % i
        assert normwise_rel_err(bf16_to_np(ad[2 * i + 1].grad), dBo) <= TOL, "layer %d: dB" % i
    assert normwise_rel_err(bf16_to_np(X.grad), dXo) <= TOL
