"""GPU parity of the adapter merge (qlora_merge) against the oracle's
lora_merge, through the C ABI: bf16(fl32(w' + s B A)). The kernel sums B A
in fp32 and the oracle in fp64, so a result may sit one bf16 step away where
the exact value lies next to a rounding point; everything else is equal bit
for bit, and without an adapter the output is the bf16 dequantization
exactly."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bf16_bits_np, oracle_constants, oracle_weight, sample_indices

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import bit_nf4_quantized_16_amd as qn

    assert torch.cuda.is_available()
    return qn


def _adapter(N, K, r, seed, a_std=0.02, b_std=0.02):
    A = workloads.bf16_normal((r, K), a_std, seed)
    B = workloads.bf16_normal((N, r), b_std, seed + 1)
    return A, B


def _compare(got_bits, want_bits, A, B, scale, min_exact=0.999):
    """|got - want| <= one bf16 step at the larger of the two plus the bound
    on the fp32 accumulation of s B A (r + 2 roundings of at most 2^-24 of
    s |B| |A|), and equal bit for bit almost everywhere."""
    g = oracle.bf16_bits_to_f32(got_bits).astype(np.float64)
    w = oracle.bf16_bits_to_f32(want_bits).astype(np.float64)
    assert np.all(np.isfinite(g))
    r = A.shape[0]
    big = np.maximum(np.maximum(np.abs(g), np.abs(w)), 1e-38)
    step = np.ldexp(1.0, np.frexp(big)[1] - 8)  # bf16 spacing in the binade of big
    acc = abs(scale) * (np.abs(np.asarray(B, np.float64)) @ np.abs(np.asarray(A, np.float64))) * (r + 2) * 2.0 ** -24
    bad = np.abs(g - w) > step + acc
    assert not bad.any(), "%d outputs out of bound, first at %s" % (bad.sum(), np.argwhere(bad)[:5])
    exact = np.mean(got_bits == want_bits)
    assert exact >= min_exact, "only %.5f of outputs equal the oracle's" % exact


def _check(qn, N, K, r, scale, seed, dq=True, std=0.02):
    W = workloads.normal_weight(N, K, std, seed=seed)
    ow = oracle_weight(W.numpy(), double_quant=dq)
    w = qn.quantize_weight(W.cuda(), double_quant=dq)
    wd32 = oracle.dequantize(ow["packed"], ow["a_eff"], N * K, out="f32").reshape(N, K)
    if r == 0:
        got = qn.qlora_merge(w)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits_np(got), ow["wd_bits"])
        return
    A, B = _adapter(N, K, r, seed + 7)
    got = qn.qlora_merge(w, A.cuda(), B.cuda(), scale)
    torch.cuda.synchronize()
    An, Bn = A.float().numpy(), B.float().numpy()
    _compare(bf16_bits_np(got), oracle.lora_merge(wd32, An, Bn, scale), An, Bn, scale)


CASES = [
    (64, 64, 1),        # one partial tile, rank 1
    (256, 512, 16),     # whole tiles
    (40, 320, 5),       # ragged rows and columns, rank not a multiple of 8
    (96, 1088, 33),     # rank just over one MFMA step
    (128, 256, 64),
    (32, 768, 128),     # the largest rank
    (8, 64, 3),
]


@pytest.mark.parametrize("N,K,r", CASES)
def test_merge_matches_oracle(qn, N, K, r):
    _check(qn, N, K, r, scale=2.0, seed=N * 7 + K + r)


@pytest.mark.parametrize("N,K", [(64, 64), (40, 320), (256, 1024)])
def test_merge_without_adapter_is_the_dequant(qn, N, K):
    _check(qn, N, K, 0, scale=2.0, seed=N + K)
    W = workloads.normal_weight(N, K, 0.02, seed=3)
    w = qn.quantize_weight(W.cuda())
    assert torch.equal(qn.qlora_merge(w), qn.nf4_dequantize(w))


def test_merge_without_double_quant(qn):
    _check(qn, 128, 640, 16, scale=0.5, seed=11, dq=False)


def test_merge_negative_scale_and_large_update(qn):
    # s B A as large as the weight itself, and of either sign
    _check(qn, 96, 512, 8, scale=-4.0, seed=12, std=0.01)
    _check(qn, 96, 512, 24, scale=16.0, seed=13)


def test_merge_then_unmerge_by_negated_adapter(qn):
    # the 4-bit weight is never changed, so "unmerging" is the bf16
    # dequantization itself; merging s B A and then -s B A on top of the
    # merged copy returns to it up to the two roundings
    N, K, r = 128, 512, 16
    W = workloads.normal_weight(N, K, 0.02, seed=14)
    w = qn.quantize_weight(W.cuda())
    before = bytes(w.packed.cpu().numpy())
    A, B = _adapter(N, K, r, 15)
    m = qn.qlora_merge(w, A.cuda(), B.cuda(), 2.0)
    torch.cuda.synchronize()
    assert bytes(w.packed.cpu().numpy()) == before
    back = m.float() - 2.0 * (B.cuda().float() @ A.cuda().float())
    base = qn.nf4_dequantize(w).float()
    assert torch.max(torch.abs(back - base)).item() <= 2 * 2.0 ** -8 * torch.max(torch.abs(m.float())).item()


def test_merged_weight_reproduces_the_forward(qn):
    # one bf16 matmul with the merged copy against the library's forward with
    # the adapter branch, on the same inputs (within the forward's tolerance)
    N, K, r, T = 256, 512, 16, 64
    W = workloads.normal_weight(N, K, 0.02, seed=16)
    w = qn.quantize_weight(W.cuda())
    A, B = _adapter(N, K, r, 17, b_std=0.05)
    X = workloads.bf16_normal((T, K), 1.0, 18).cuda()
    Y, _ = qn.qlora_linear_fwd(w, X, A.cuda(), B.cuda(), 2.0)
    M = qn.qlora_merge(w, A.cuda(), B.cuda(), 2.0)
    Ym = X.float() @ M.float().T
    err = torch.max(torch.abs(Y.float() - Ym)).item() / torch.max(torch.abs(Ym)).item()
    assert err < 2e-2


def _check_sampled(qn, N, K, r, scale, seed, count=48):
    W = workloads.normal_weight(N, K, 0.02, seed=seed)
    w = qn.quantize_weight(W.cuda())
    A, B = _adapter(N, K, r, seed + 17)
    got = bf16_bits_np(qn.qlora_merge(w, A.cuda(), B.cuda(), scale))
    Wn = W.numpy()
    consts = oracle_constants(Wn)
    rows = sample_indices(N, count, seed=seed + 18)
    kb = K // oracle.BLOCKSIZE
    blocks = (rows[:, None] * kb + np.arange(kb)[None, :]).ravel()
    codes = oracle.nf4_codes(Wn[rows].ravel(), consts["absmax"][blocks])
    wd32 = oracle.dequantize(oracle.pack_nibbles(codes), consts["a_eff"][blocks], len(rows) * K, out="f32")
    An, Bn = A.float().numpy(), B.float().numpy()[rows]
    _compare(got[rows], oracle.lora_merge(wd32.reshape(len(rows), K), An, Bn, scale), An, Bn, scale)


def test_merge_full_size_sampled_rows(qn):
    # the 7B MLP gate projection (11008 x 4096) at rank 64, rows sampled
    _check_sampled(qn, 11008, 4096, 64, 0.25, seed=2)


@pytest.mark.parametrize("N,K,r", [(4104, 16384, 16), (2056, 8192, 100)])
def test_merge_many_row_blocks_per_workgroup(qn, N, K, r):
    # wide weights: few row blocks per column window run in each workgroup,
    # with a half-filled last 16-row block (N % 16 == 8)
    _check_sampled(qn, N, K, r, 1.5, seed=N + r)
