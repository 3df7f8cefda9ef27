"""GPU parity of the grouped forward above decode sizes (qlora_linear_fwd_group
at T > 16 where it runs one GEMM launch over all layers' row tiles): Y and U
of every layer against the fp64 CPU oracle, U bitwise the single calls', and
Y bitwise one call on the stacked weight where the two plans coincide."""

import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, bf16_to_np, f32_to_np, normwise_rel_err, oracle_constants, oracle_rows, oracle_weight
from gpu_util import sample_indices

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import bit_nf4_quantized_16_amd as qn

    assert torch.cuda.is_available()
    return qn


def _one_launch(qn, rows, K, T, r):
    import ctypes

    return qn.lib.qlora_linear_fwd_group_one_launch((ctypes.c_int64 * len(rows))(*rows), len(rows), K, T, r) == 1


def _layers(shapes, K, T, r, seed):
    cases = []
    for i, N in enumerate(shapes):
        W = workloads.normal_weight(N, K, 0.02, seed=seed + 13 * i)
        cases.append(workloads.lora_case("fg%d" % i, W, T, max(r, 1), 2.0 * max(r, 1), 1 / K, 0.05,
                                         seed=seed + 7 * i))
    return cases


# (2048-wide reductions split in two; ragged N and T; 3 and 2 layers)
@pytest.mark.parametrize("shapes,K,T,r", [((1024, 1024, 1024), 2048, 512, 16),
                                           ((1032, 264, 520), 2048, 300, 8),
                                           ((2048, 512), 2048, 700, 64)])
def test_fwd_group_gemm_matches_oracle(qn, shapes, K, T, r):
    assert _one_launch(qn, shapes, K, T, r), "the shape should take the one-launch path"
    cases = _layers(shapes, K, T, r, seed=T + K)
    s = cases[0].scale
    X = cases[0].X
    ws = [qn.quantize_weight(c.W.cuda()) for c in cases]
    outs = qn.qlora_linear_fwd_group(ws, X.cuda(), [c.A.cuda() for c in cases], [c.B.cuda() for c in cases], s)
    singles = [qn.qlora_linear_fwd(w, X.cuda(), c.A.cuda(), c.B.cuda(), s) for w, c in zip(ws, cases)]
    torch.cuda.synchronize()
    Xn = bf16_to_np(X)
    for i, c in enumerate(cases):
        Y, U = outs[i]
        H, Uo = oracle.lora_forward(Xn, oracle_weight(c.W.numpy())["wd"], bf16_to_np(c.A), bf16_to_np(c.B), s)
        assert normwise_rel_err(bf16_to_np(Y), H) <= TOL, "layer %d: Y" % i
        assert normwise_rel_err(f32_to_np(U), Uo) <= TOL, "layer %d: U" % i
        assert torch.equal(U, singles[i][1]), "layer %d: U differs from the single call's" % i
        # the same products summed in another split order: one bf16 step apart at most
        d = (Y.float() - singles[i][0].float()).abs().max().item()
        assert d <= 2.0 ** -7 * singles[i][0].float().abs().max().item(), "layer %d: Y vs single %.3e" % (i, d)


@pytest.mark.parametrize("shapes,K,T", [((1024, 1024, 1024), 2048, 512), ((4096, 4096, 4096), 4096, 1024),
                                        ((11008, 11008), 4096, 256)])
def test_fwd_group_gemm_rank0_is_the_stacked_weight(qn, shapes, K, T):
    """Without adapters and without double quantization, layers of whole
    256-row tiles: the grouped launch runs the stacked weight's tiles under
    the same plan, so each Y is bitwise its columns of one call on the weight
    stacked along N."""
    assert _one_launch(qn, shapes, K, T, 0)
    ws = []
    for i, N in enumerate(shapes):
        W = workloads.normal_weight(N, K, 0.02, seed=N + i)
        ws.append(qn.quantize_weight(W.cuda(), double_quant=False))
    stacked = qn.NF4Weight(sum(shapes), K, torch.cat([w.packed for w in ws]), absmax=torch.cat([w.absmax for w in ws]))
    X = workloads.bf16_normal((T, K), 1.0, seed=3).cuda()
    Ycat, _ = qn.qlora_linear_fwd(stacked, X)
    outs = qn.qlora_linear_fwd_group(ws, X)
    torch.cuda.synchronize()
    c0 = 0
    for (Y, _), N in zip(outs, shapes):
        assert torch.equal(Y, Ycat[:, c0:c0 + N]), "columns %d.. differ" % c0
        c0 += N


def test_fwd_group_gemm_full_size_qkv(qn):
    """q, k, v of the 7B attention (4096x4096 each) at T = 1024, r = 16, the
    shape whose single GEMMs split their reduction: sampled rows of every Y
    and the whole U against the oracle."""
    print("full-size grouped forward q/k/v T=1024", flush=True)
    T, K, r = 1024, 4096, 16
    assert _one_launch(qn, (4096,) * 3, K, T, r)
    cases = [workloads.lora_case("qkv%d" % i, workloads.normal_weight(4096, K, 0.02, seed=60 + i, outlier_frac=1e-3),
                                 T, r, 32.0, 1 / K, 0.01, seed=60 + i) for i in range(3)]
    s = cases[0].scale
    X = cases[0].X
    ws = [qn.quantize_weight(c.W.cuda()) for c in cases]
    outs = qn.qlora_linear_fwd_group(ws, X.cuda(), [c.A.cuda() for c in cases], [c.B.cuda() for c in cases], s)
    torch.cuda.synchronize()
    Xn = bf16_to_np(X)
    for i, c in enumerate(cases):
        Wn = c.W.numpy()
        rows = sample_indices(4096, 24, seed=70 + i)
        _, wd_r = oracle_rows(Wn, rows, oracle_constants(Wn))
        Bn = bf16_to_np(c.B)
        H_r, Uo = oracle.lora_forward(Xn, wd_r, bf16_to_np(c.A), Bn[rows], s)
        Y, U = outs[i]
        assert normwise_rel_err(bf16_to_np(Y)[:, rows], H_r) <= TOL, "layer %d: Y" % i
        assert normwise_rel_err(f32_to_np(U), Uo) <= TOL, "layer %d: U" % i


def test_fwd_group_gemm_graph_replays(qn):
    """Captured once, replayed with new X each time: every replay equals the
    eager call bit for bit."""
    shapes, K, T, r = (1024, 1024, 1024), 2048, 512, 16
    cases = _layers(shapes, K, T, r, seed=8)
    s = cases[0].scale
    ws = [qn.quantize_weight(c.W.cuda()) for c in cases]
    As = [c.A.cuda() for c in cases]
    Bs = [c.B.cuda() for c in cases]
    X = cases[0].X.cuda()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qn.qlora_linear_fwd_group(ws, X, As, Bs, s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = qn.qlora_linear_fwd_group(ws, X, As, Bs, s)
    for rep in range(3):
        X.copy_(workloads.bf16_normal((T, K), 1.0, seed=200 + rep).cuda())
        graph.replay()
        torch.cuda.synchronize()
        want = qn.qlora_linear_fwd_group(ws, X, As, Bs, s)
        torch.cuda.synchronize()
        for i, ((Y, U), (Yw, Uw)) in enumerate(zip(outs, want)):
            assert torch.equal(Y, Yw) and torch.equal(U, Uw), "replay %d, layer %d" % (rep, i)


def test_fwd_group_mixed_formats_run_one_call_per_layer(qn):
    """A group whose layers differ in double quantization takes the
    one-after-another path (the workspace query covers it): Y and U bitwise
    one qlora_linear_fwd per layer."""
    shapes, K, T, r = (1024, 1024, 1024), 2048, 512, 16
    assert _one_launch(qn, shapes, K, T, r)
    cases = _layers(shapes, K, T, r, seed=21)
    s = cases[0].scale
    ws = [qn.quantize_weight(c.W.cuda(), double_quant=(i != 1)) for i, c in enumerate(cases)]
    X = cases[0].X.cuda()
    As = [c.A.cuda() for c in cases]
    Bs = [c.B.cuda() for c in cases]
    outs = qn.qlora_linear_fwd_group(ws, X, As, Bs, s)
    for i, w in enumerate(ws):
        Y1, U1 = qn.qlora_linear_fwd(w, X, As[i], Bs[i], s)
        torch.cuda.synchronize()
        assert torch.equal(outs[i][0], Y1) and torch.equal(outs[i][1], U1), "layer %d" % i
