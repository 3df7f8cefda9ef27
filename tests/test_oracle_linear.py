"""Pins for the oracle's forward and backward (no GPU): brute-force loops on
tiny shapes, gradients derived by torch.autograd (fp64) and by central
differences, and closed forms for the special cases B = 0, A = 0 and W = 0."""

import numpy as np
import torch

import oracle


def _case(T=3, N=5, K=8, r=2, seed=0, b_std=0.5):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, K))
    W = rng.standard_normal((N, K)) * 0.1
    A = rng.standard_normal((r, K)) * 0.3
    B = rng.standard_normal((N, r)) * b_std
    dY = rng.standard_normal((T, N))
    return X, W, A, B, dY


def test_forward_matches_brute_force_loops():
    X, W, A, B, _ = _case(T=3, N=7, K=16, r=3, seed=1)
    s = 1.75
    H, U = oracle.lora_forward(X, W, A, B, s)
    T_, K = X.shape
    N, r = B.shape
    for t in range(T_):
        for j in range(r):
            u = 0.0
            for k in range(K):
                u += X[t, k] * A[j, k]
            assert abs(u - U[t, j]) < 1e-12
        for n in range(N):
            h = 0.0
            for k in range(K):
                h += X[t, k] * W[n, k]
            lora = 0.0
            for j in range(r):
                ba = 0.0
                for k in range(K):
                    ba += B[n, j] * A[j, k] * X[t, k]
                lora += ba
            assert abs(h + s * lora - H[t, n]) < 1e-12


def test_backward_matches_autograd_fp64():
    X, W, A, B, dY = _case(T=4, N=6, K=12, r=3, seed=2)
    s = 2.0
    tX = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    tA = torch.tensor(A, dtype=torch.float64, requires_grad=True)
    tB = torch.tensor(B, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(W, dtype=torch.float64)
    H = tX @ tW.T + s * ((tX @ tA.T) @ tB.T)
    H.backward(torch.tensor(dY, dtype=torch.float64))
    dX, dA, dB, G, U = oracle.lora_backward(X, dY, W, A, B, s)
    assert np.allclose(dX, tX.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dA, tA.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dB, tB.grad.numpy(), rtol=0, atol=1e-12)
    Href, _ = oracle.lora_forward(X, W, A, B, s)
    assert np.allclose(Href, H.detach().numpy(), rtol=0, atol=1e-12)


def test_backward_matches_central_differences():
    X, W, A, B, dY = _case(T=2, N=4, K=6, r=2, seed=3)
    s = 0.5
    dX, dA, dB, _, _ = oracle.lora_backward(X, dY, W, A, B, s)

    def loss(X_, A_, B_):
        H, _ = oracle.lora_forward(X_, W, A_, B_, s)
        return float(np.sum(H * dY))

    h = 1e-6
    for arr, grad, which in ((X, dX, 0), (A, dA, 1), (B, dB, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy()
            m = arr.copy()
            p[idx] += h
            m[idx] -= h
            args_p = [X, A, B]
            args_m = [X, A, B]
            args_p[which] = p
            args_m[which] = m
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.allclose(num, grad, rtol=1e-6, atol=1e-8)


def test_special_case_B_zero():
    X, W, A, B, dY = _case(seed=4)
    B = np.zeros_like(B)
    H, _ = oracle.lora_forward(X, W, A, B, 2.0)
    assert np.array_equal(H, X @ W.T)
    dX, dA, dB, _, _ = oracle.lora_backward(X, dY, W, A, B, 2.0)
    assert np.all(dA == 0)
    assert np.allclose(dX, dY @ W, rtol=0, atol=1e-14)


def test_special_case_A_zero():
    X, W, A, B, dY = _case(seed=5)
    A = np.zeros_like(A)
    H, U = oracle.lora_forward(X, W, A, B, 2.0)
    assert np.all(U == 0) and np.array_equal(H, X @ W.T)
    _, _, dB, _, _ = oracle.lora_backward(X, dY, W, A, B, 2.0)
    assert np.all(dB == 0)


def test_special_case_W_zero():
    X, W, A, B, dY = _case(seed=6)
    W = np.zeros_like(W)
    s = 3.0
    H, _ = oracle.lora_forward(X, W, A, B, s)
    assert np.allclose(H, s * X @ A.T @ B.T, rtol=0, atol=1e-13)
    dX, _, _, G, _ = oracle.lora_backward(X, dY, W, A, B, s)
    assert np.allclose(dX, (s * dY @ B) @ A, rtol=0, atol=1e-13)
    assert np.allclose(G, s * dY @ B, rtol=0, atol=1e-14)


def test_quantized_all_zero_weight_gives_zero_base():
    # an all-zero weight quantizes to code 7 everywhere and dequantizes to 0,
    # which is how the GPU tests isolate the LoRA branch
    w = np.zeros((8, 128), dtype=np.float32)
    packed, a = oracle.quantize(w)
    assert np.all(packed == 0x77) and np.all(a == 0)
    c8, S, mu = oracle.double_quant(a)
    ar = oracle.dequant_absmax(c8, S, mu)
    assert np.all(ar == 0)
    wd = oracle.dequantize(packed, ar, w.size, out="f32")
    assert np.all(wd == 0)


# ---- adapter merge ---------------------------------------------------------


def _bf16_bits_torch(v):
    """Independent bf16 rounding (torch's fp32 -> bf16 cast, nearest even)."""
    t = torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_merge_matches_brute_force_loops():
    _, W, A, B, _ = _case(N=5, K=7, r=3, seed=7)
    W = W.astype(np.float32)
    s = 1.5
    got = oracle.lora_merge(W, A, B, s)
    N, K = W.shape
    want = np.empty((N, K), dtype=np.float32)
    for n in range(N):
        for k in range(K):
            d = 0.0
            for j in range(B.shape[1]):
                d += B[n, j] * A[j, k]
            want[n, k] = np.float32(float(W[n, k]) + s * d)
    assert np.array_equal(got, _bf16_bits_torch(want))


def test_merge_rank_one_zero_base_is_scaled_outer_product():
    rng = np.random.default_rng(8)
    a = rng.standard_normal(9)
    b = rng.standard_normal(4)
    s = 0.25
    got = oracle.lora_merge(np.zeros((4, 9), dtype=np.float32), a[None, :], b[:, None], s)
    assert np.array_equal(got, _bf16_bits_torch(s * np.multiply.outer(b, a)))


def test_merge_without_adapter_is_the_bf16_dequant():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((8, 128)) * 0.05).astype(np.float32)
    packed, a = oracle.quantize(w)
    c8, S, mu = oracle.double_quant(a)
    ar = oracle.dequant_absmax(c8, S, mu)
    wd = oracle.dequantize(packed, ar, w.size, out="f32").reshape(8, 128)
    bits = oracle.dequantize(packed, ar, w.size, out="bf16").reshape(8, 128)
    A = rng.standard_normal((4, 128))
    assert np.array_equal(oracle.lora_merge(wd, A, np.zeros((8, 4)), 2.0), bits)
    assert np.array_equal(oracle.lora_merge(wd, np.zeros((4, 128)), rng.standard_normal((8, 4)), 2.0), bits)


def test_merged_weight_reproduces_the_adapter_branch():
    # the point of merging: X M^T equals X W'^T + s (X A^T) B^T up to the one
    # bf16 rounding of M (relative 2^-9 per element)
    X, W, A, B, _ = _case(T=6, N=11, K=24, r=4, seed=10)
    s = 3.0
    M = oracle.bf16_bits_to_f32(oracle.lora_merge(W.astype(np.float32), A, B, s)).astype(np.float64)
    H, _ = oracle.lora_forward(X, W.astype(np.float32), A, B, s)
    exact = W.astype(np.float32).astype(np.float64) + s * (B @ A)
    bound = np.abs(X) @ (np.abs(exact) * 2.0 ** -8).T + 1e-12
    assert np.all(np.abs(X @ M.T - H) <= bound)
    # a dropped scale would be far outside the bound
    M1 = oracle.bf16_bits_to_f32(oracle.lora_merge(W.astype(np.float32), A, B, 1.0)).astype(np.float64)
    assert not np.all(np.abs(X @ M1.T - H) <= bound)


# ---- dropout on the adapter input --------------------------------------------


def test_dropout_with_everything_kept_and_p0_is_the_plain_layer():
    X, W, A, B, dY = _case(T=4, N=6, K=16, r=3, seed=11)
    keep = np.ones_like(X)
    H0, U0 = oracle.lora_forward(X, W, A, B, 1.5)
    H1, U1 = oracle.lora_forward_dropout(X, W, A, B, 1.5, keep, 0.0)
    assert np.array_equal(H0, H1) and np.array_equal(U0, U1)
    for a, b in zip(oracle.lora_backward(X, dY, W, A, B, 1.5), oracle.lora_backward_dropout(X, dY, W, A, B, 1.5, keep, 0.0)):
        assert np.array_equal(a, b)


def test_dropout_backward_matches_autograd_fp64():
    X, W, A, B, dY = _case(T=5, N=7, K=24, r=3, seed=12)
    rng = np.random.default_rng(13)
    keep = (rng.random(X.shape) >= 0.3).astype(np.float64)
    p, s = 0.3, 2.0
    tX = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    tA = torch.tensor(A, dtype=torch.float64, requires_grad=True)
    tB = torch.tensor(B, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(W, dtype=torch.float64)
    tk = torch.tensor(keep)
    H = tX @ tW.T + s * (((tX * tk) / (1 - p)) @ tA.T) @ tB.T
    H.backward(torch.tensor(dY, dtype=torch.float64))
    Href, _ = oracle.lora_forward_dropout(X, W, A, B, s, keep, p)
    dX, dA, dB, _, _ = oracle.lora_backward_dropout(X, dY, W, A, B, s, keep, p)
    assert np.allclose(Href, H.detach().numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dX, tX.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dA, tA.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dB, tB.grad.numpy(), rtol=0, atol=1e-12)


def test_dropout_forward_matches_brute_force_loops():
    X, W, A, B, _ = _case(T=2, N=3, K=8, r=2, seed=14)
    keep = np.array([[1, 0, 1, 1, 0, 1, 1, 1], [0, 0, 1, 0, 1, 1, 0, 1]], dtype=np.float64)
    p, s = 0.25, 3.0
    H, U = oracle.lora_forward_dropout(X, W, A, B, s, keep, p)
    for t in range(2):
        for j in range(2):
            u = sum(X[t, k] * keep[t, k] * A[j, k] for k in range(8)) / (1 - p)
            assert abs(u - U[t, j]) < 1e-12
        for n in range(3):
            h = sum(X[t, k] * W[n, k] for k in range(8)) + s * sum(U[t, j] * B[n, j] for j in range(2))
            assert abs(h - H[t, n]) < 1e-12


def test_dropout_with_nothing_kept_leaves_only_the_base():
    X, W, A, B, dY = _case(T=3, N=5, K=8, r=2, seed=15)
    keep = np.zeros_like(X)
    H, U = oracle.lora_forward_dropout(X, W, A, B, 2.0, keep, 0.5)
    assert np.all(U == 0) and np.array_equal(H, X @ W.T)
    dX, dA, dB, _, _ = oracle.lora_backward_dropout(X, dY, W, A, B, 2.0, keep, 0.5)
    assert np.all(dA == 0) and np.all(dB == 0) and np.array_equal(dX, dY @ W)


def test_keep_bit_packing_layout():
    import workloads

    keep = torch.zeros(2, 16, dtype=torch.bool)
    keep[0, 0] = keep[0, 9] = keep[1, 7] = keep[1, 15] = True
    bits = workloads.pack_keep_bits(keep)
    assert bits.tolist() == [[1, 2], [128, 128]]
