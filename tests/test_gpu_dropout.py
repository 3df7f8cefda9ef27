"""GPU parity of the LoRA layer with dropout on the adapter input (the keep
mask and p passed in) against the fp64 oracle's lora_forward_dropout /
lora_backward_dropout, through the C ABI; the normwise tolerance of the
plain layer."""

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


def _run(qn, case, p, seed, dq=True, save_u=True, tol=TOL):
    W = case.W
    T, K = case.X.shape
    keep = workloads.keep_mask(T, K, p, seed)
    bits = workloads.pack_keep_bits(keep).cuda()
    w = qn.quantize_weight(W.contiguous().cuda(), double_quant=dq)
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    s = case.scale
    Y, U = qn.qlora_linear_fwd(w, X, A, B, s, save_u=True, keep=bits, p=p)
    dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U if save_u else None, keep=bits, p=p)
    torch.cuda.synchronize()
    ref = oracle_weight(W.numpy(), double_quant=dq)
    Xn, dYn, An, Bn = (bf16_to_np(t) for t in (case.X, case.dY, case.A, case.B))
    kn = keep.numpy().astype(np.float64)
    H, Uo = oracle.lora_forward_dropout(Xn, ref["wd"], An, Bn, s, kn, p)
    dXo, dAo, dBo, _, _ = oracle.lora_backward_dropout(Xn, dYn, ref["wd"], An, Bn, s, kn, p)
    errs = dict(
        H=normwise_rel_err(bf16_to_np(Y), H),
        U=normwise_rel_err(f32_to_np(U), Uo),
        dX=normwise_rel_err(bf16_to_np(dX), dXo),
        dA=normwise_rel_err(f32_to_np(dA), dAo),
        dB=normwise_rel_err(f32_to_np(dB), dBo),
    )
    for k, v in errs.items():
        assert v <= tol, "%s: %s error %.3e > %.0e (%s)" % (case.name, k, v, tol, errs)
    return errs


@pytest.mark.parametrize("T", [1, 5, 16, 17, 300])
@pytest.mark.parametrize("p", [0.05, 0.5])
def test_dropout_matches_oracle_across_token_counts(qn, T, p):
    W = workloads.normal_weight(256, 320, 0.02, seed=T)
    _run(qn, workloads.lora_case("T%d" % T, W, T, 8, 16.0, 1 / 320, 0.05, seed=T), p, seed=T + 1)


@pytest.mark.parametrize("N,K,T,r", [(136, 192, 40, 1), (256, 512, 96, 33), (512, 384, 200, 128), (64, 64, 7, 16)])
def test_dropout_ragged_shapes_and_ranks(qn, N, K, T, r):
    W = workloads.normal_weight(N, K, 0.02, seed=N + K)
    case = workloads.lora_case("drop_%d_%d_%d_%d" % (N, K, T, r), W, T, r, 2.0 * r, 1 / K, 0.05, seed=r)
    _run(qn, case, 0.1, seed=N + r)


@pytest.mark.parametrize("T", [4, 96])
def test_dropout_zero_base_isolates_the_masked_branch(qn, T):
    # W = 0: H = s U B^T and dX = c (G A) * keep exactly in the oracle
    W = torch.zeros(256, 256)
    case = workloads.lora_case("zeroW", W, T, 8, 16.0, 1 / 16, 0.5, seed=21)
    errs = _run(qn, case, 0.3, seed=22)
    assert errs["H"] < 1e-2 and errs["dX"] < 1e-2


def test_dropout_without_saved_u_and_without_double_quant(qn):
    W = workloads.normal_weight(384, 512, 0.02, seed=23)
    case = workloads.lora_case("recompute_u", W, 150, 16, 32.0, 1 / 512, 0.05, seed=23)
    _run(qn, case, 0.05, seed=24, save_u=False)
    _run(qn, case, 0.05, seed=25, dq=False)


def test_everything_kept_at_p0_equals_the_plain_layer(qn):
    # same operands through the dropout route: H and dA bit for bit, dX up to
    # the one extra bf16 rounding of the adapter term
    W = workloads.normal_weight(256, 512, 0.02, seed=26)
    case = workloads.lora_case("keep_all", W, 100, 16, 32.0, 1 / 512, 0.05, seed=26)
    w = qn.quantize_weight(W.cuda())
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    bits = workloads.pack_keep_bits(torch.ones(100, 512, dtype=torch.bool)).cuda()
    Y0, U0 = qn.qlora_linear_fwd(w, X, A, B, case.scale)
    Y1, U1 = qn.qlora_linear_fwd(w, X, A, B, case.scale, keep=bits, p=0.0)
    assert torch.equal(Y0, Y1) and torch.equal(U0, U1)
    dX0, dA0, dB0 = qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, U=U0)
    dX1, dA1, dB1 = qn.qlora_linear_bwd(w, X, dY, A, B, case.scale, U=U1, keep=bits, p=0.0)
    assert torch.equal(dA0, dA1) and torch.equal(dB0, dB1)
    assert normwise_rel_err(bf16_to_np(dX1), bf16_to_np(dX0)) < 1e-2


def test_full_size_mlp_gate_with_dropout(qn):
    # the 7B MLP gate projection at T = 1024, r = 16, p = 0.05
    case = workloads.mlp_7b("gate", T=1024)
    _run(qn, case, 0.05, seed=27)


def test_autograd_function_with_dropout(qn):
    W = workloads.normal_weight(256, 256, 0.02, seed=28)
    case = workloads.lora_case("autograd", W, 64, 8, 16.0, 1 / 256, 0.05, seed=28)
    w = qn.quantize_weight(W.cuda())
    keep = workloads.keep_mask(64, 256, 0.2, seed=29)
    bits = workloads.pack_keep_bits(keep).cuda()
    X = case.X.cuda().requires_grad_(True)
    A = case.A.cuda().requires_grad_(True)
    B = case.B.cuda().requires_grad_(True)
    Y = qn.QLoRALinearFunction.apply(X, A, B, w, case.scale, bits, 0.2)
    Y.backward(case.dY.cuda())
    ref = oracle_weight(W.numpy())
    Xn, dYn, An, Bn = (bf16_to_np(t) for t in (case.X, case.dY, case.A, case.B))
    dXo, dAo, dBo, _, _ = oracle.lora_backward_dropout(Xn, dYn, ref["wd"], An, Bn, case.scale,
                                                       keep.numpy().astype(np.float64), 0.2)
    assert normwise_rel_err(bf16_to_np(X.grad), dXo) <= TOL
    assert normwise_rel_err(bf16_to_np(A.grad.float()), dAo) <= TOL
    assert normwise_rel_err(bf16_to_np(B.grad.float()), dBo) <= TOL
