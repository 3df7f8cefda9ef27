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
