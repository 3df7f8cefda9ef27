"""Helpers shared by the GPU parity tests: conversions and the oracle's view of
a weight. Everything here calls the oracle or torch only; nothing from the
HIP path feeds an expected value."""

import numpy as np
import torch

import oracle


def bf16_to_np(t):
    """bf16 tensor (any device) -> fp32 numpy with the same values."""
    return t.detach().to("cpu").float().numpy()


def f32_to_np(t):
    return t.detach().to("cpu").numpy().astype(np.float32)


def u8_to_np(t):
    return t.detach().to("cpu").numpy().astype(np.uint8)


def bf16_bits_np(t):
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_weight(W, double_quant=True):
    """The oracle's quantization of fp32 numpy W: dict with packed, absmax,
    c8, scale, mean, the effective absmax and the dequantized bf16 weight
    (as fp32 values) and its bit patterns."""
    W = np.asarray(W, dtype=np.float32)
    packed, absmax = oracle.quantize(W)
    out = dict(packed=packed, absmax=absmax)
    if double_quant:
        c8, scale, mean = oracle.double_quant(absmax)
        a_eff = oracle.dequant_absmax(c8, scale, mean)
        out.update(c8=c8, scale=scale, mean=mean)
    else:
        a_eff = absmax
    bits = oracle.dequantize(packed, a_eff, W.size, out="bf16")
    out["a_eff"] = a_eff
    out["wd_bits"] = bits.reshape(W.shape)
    out["wd"] = oracle.bf16_bits_to_f32(bits).reshape(W.shape)
    return out


def normwise_rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.max(np.abs(want))
    if den == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - want)) / den)


# The tolerance the forward and backward outputs are held to: bf16 inputs,
# fp32 accumulation on the GPU vs fp64 in the oracle, normwise (max |error|
# over max |reference|).
TOL = 2e-2


def oracle_constants(W, double_quant=True):
    """The oracle's block constants of the whole fp32 numpy W: absmax of
    every 64-block and the effective constants a' (after double
    quantization when asked)."""
    W = np.asarray(W, dtype=np.float32)
    absmax = oracle.blockwise_absmax(W)
    out = dict(absmax=absmax)
    if double_quant:
        c8, scale, mean = oracle.double_quant(absmax)
        out.update(c8=c8, scale=scale, mean=mean, a_eff=oracle.dequant_absmax(c8, scale, mean))
    else:
        out["a_eff"] = absmax
    return out


def oracle_rows(W, rows, consts):
    """Packed codes [len(rows), K/2] and dequantized bf16 values (fp32)
    [len(rows), K] of whole rows of W (K a multiple of 64), by the oracle's
    steps applied to those rows' blocks."""
    W = np.asarray(W, dtype=np.float32)
    K = W.shape[1]
    kb = K // oracle.BLOCKSIZE
    rows = np.asarray(rows)
    w = W[rows].ravel()
    blocks = (rows[:, None] * kb + np.arange(kb)[None, :]).ravel()
    codes = oracle.nf4_codes(w, consts["absmax"][blocks])
    packed = oracle.pack_nibbles(codes)
    wd = oracle.bf16_bits_to_f32(oracle.dequantize(packed, consts["a_eff"][blocks], w.size))
    return packed.reshape(len(rows), K // 2), wd.reshape(len(rows), K)


def oracle_cols(W, cols, consts):
    """Dequantized bf16 values (fp32) [N, len(cols)] of whole columns of W:
    every element with its own block's constants (the oracle's steps with a
    block of one element and that element's block constant)."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    cols = np.asarray(cols)
    w = W[:, cols].ravel()
    blk = ((np.arange(N)[:, None] * K + cols[None, :]) // oracle.BLOCKSIZE).ravel()
    codes = oracle.nf4_codes(w, consts["absmax"][blk], blocksize=1)
    packed = oracle.pack_nibbles(codes)
    wd = oracle.bf16_bits_to_f32(oracle.dequantize(packed, consts["a_eff"][blk], w.size, blocksize=1))
    return wd.reshape(N, len(cols))


def sample_indices(n, count, seed):
    """Sorted distinct indices in [0, n): both ends, the 256- and 128-tile
    edges near the start and the end, and seeded random ones."""
    fixed = {0, 1, n - 1, n - 2, min(127, n - 1), min(128, n - 1), min(255, n - 1), min(256, n - 1),
             max(0, n - 129), max(0, n - 257)}
    rng = np.random.default_rng(seed)
    rest = rng.choice(n, size=min(n, count), replace=False)
    return np.array(sorted(fixed | set(int(x) for x in rest)))
