"""GPU parity at the full sizes of the 7B and 65B workloads, in the launch
configuration bench.py times (default tile and split plan): the whole tensor
is quantized and run through forward and backward on the GPU, and sampled
rows / columns of every output are compared with the oracle, which computes
them one by one from the same seeded inputs (its steps applied to the
sampled rows' or columns' blocks; the double-quantization constants of the
whole tensor are compared bit for bit)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, bf16_to_np, f32_to_np, normwise_rel_err, oracle_cols, oracle_constants, oracle_rows
from gpu_util import oracle_weight
from gpu_util import sample_indices, u8_to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import bit_nf4_quantized_16_amd as qn

    assert torch.cuda.is_available()
    return qn


CASES = {
    "attn_4096x4096_T1_r16": lambda: workloads.attn_proj_7b(1),
    "attn_4096x4096_T16_r16": lambda: workloads.attn_proj_7b(16),
    "mlp_gate_11008x4096_T1024_r16": lambda: workloads.mlp_7b("gate"),
    "mlp_down_4096x11008_T1024_r16": lambda: workloads.mlp_7b("down"),
    "stack7b_o_4096x4096_T4096_r64": lambda: workloads.llama7b_layer_linear("o"),
    "stack7b_up_11008x4096_T4096_r64": lambda: workloads.llama7b_layer_linear("up"),
    "65b_sq_8192x8192_T4096_r64": lambda: workloads.llama65b_linear("sq"),
    "65b_up_22016x8192_T4096_r64": lambda: workloads.llama65b_linear("up"),
    "65b_down_8192x22016_T4096_r64": lambda: workloads.llama65b_linear("down"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_full_size_sampled_outputs(qn, name):
    case = CASES[name]()
    print("full-size case", name, flush=True)
    W = case.W
    N, K = W.shape
    s = case.scale
    w = qn.quantize_weight(W.cuda(), double_quant=True)
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    Y, U = qn.qlora_linear_fwd(w, X, A, B, s)
    dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U)
    torch.cuda.synchronize()

    Wn = W.numpy()
    consts = oracle_constants(Wn)
    assert np.array_equal(u8_to_np(w.c8), consts["c8"]), "E4M3 codes differ"
    assert np.array_equal(f32_to_np(w.dq_scale).view(np.uint32), consts["scale"].view(np.uint32)), "scales differ"
    assert f32_to_np(w.dq_mean).view(np.uint32)[0] == np.float32(consts["mean"]).view(np.uint32), "mean differs"

    rows = sample_indices(N, 40, seed=N)
    cols = sample_indices(K, 24, seed=K + 1)
    packed_r, wd_r = oracle_rows(Wn, rows, consts)
    gp = u8_to_np(w.packed).reshape(N, K // 2)[rows]
    assert np.array_equal(gp, packed_r), "packed codes of the sampled rows differ"
    wd_c = oracle_cols(Wn, cols, consts)

    Xn, dYn, An, Bn = (bf16_to_np(t) for t in (case.X, case.dY, case.A, case.B))
    # rows: H[:, R] and dB[R] (dB's rows need U of the whole X, which this call has)
    H_r, U_o = oracle.lora_forward(Xn, wd_r, An, Bn[rows], s)
    _, _, dB_r, _, _ = oracle.lora_backward(Xn, dYn[:, rows], wd_r, An, Bn[rows], s)
    # columns: dX[:, C] and dA[:, C] (G = s dY B over all N)
    dX_c, dA_c, _, _, _ = oracle.lora_backward(Xn[:, cols], dYn, wd_c, An[:, cols], Bn, s)

    errs = dict(
        H=normwise_rel_err(bf16_to_np(Y)[:, rows], H_r),
        U=normwise_rel_err(f32_to_np(U), U_o),
        dX=normwise_rel_err(bf16_to_np(dX)[:, cols], dX_c),
        dA=normwise_rel_err(f32_to_np(dA)[:, cols], dA_c),
        dB=normwise_rel_err(f32_to_np(dB)[rows], dB_r),
    )
    print(name, {k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL, "%s: %s error %.3e > %.0e" % (name, k, v, TOL)


@pytest.mark.parametrize("zero_w", [False, True])
def test_decode_full_4096x4096_every_output(qn, zero_w):
    """The decode forward at the 4096 x 4096 attention shape (0.1 % outliers
    x20, r = 16, alpha = 32) at T = 1 and T = 16, in the launch configuration
    the benchmark times: every packed code bit for bit, and every element of
    Y and U against the oracle. With an all-zero weight (every code 7) only
    the adapter branch is left, so Y = s (X A^T) B^T checks that branch at
    this size, where it is under 1 % of H otherwise."""
    case = workloads.attn_proj_7b(16)
    W = torch.zeros(4096, 4096) if zero_w else case.W
    print("decode full 4096x4096 zero_w=%s" % zero_w, flush=True)
    w = qn.quantize_weight(W.cuda(), double_quant=True)
    A, B = case.A.cuda(), case.B.cuda()
    ref = oracle_weight(W.numpy())
    if not zero_w:
        assert np.array_equal(u8_to_np(w.packed), ref["packed"]), "packed NF4 codes differ"
    An, Bn = bf16_to_np(case.A), bf16_to_np(case.B)
    for T in (1, 16):
        X = case.X[:T].contiguous()
        Y, U = qn.qlora_linear_fwd(w, X.cuda(), A, B, case.scale)
        torch.cuda.synchronize()
        H, Uo = oracle.lora_forward(bf16_to_np(X), ref["wd"], An, Bn, case.scale)
        eh, eu = normwise_rel_err(bf16_to_np(Y), H), normwise_rel_err(f32_to_np(U), Uo)
        print("T=%d H %.2e U %.2e" % (T, eh, eu), flush=True)
        assert eh <= TOL and eu <= TOL, (T, eh, eu)
        if zero_w:
            # nothing but the adapter term: fp32 sums of bf16 products, one bf16 rounding
            assert eh < 1e-2
