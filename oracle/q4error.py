"""Error of blockwise-absmax 4-bit quantization on a sixteen-value grid (CPU
oracle). Test infrastructure only (see the package docstring).

ai-reference-codex "QLoRA 与 PEFT 全家", §3.2: the naive 4-bit grid puts its
sixteen values at equal spacing; NF4 spaces them by the normal density
(dense near zero, sparse in the tails), which is said to distort less for the
same four bits. §5 of the same page: the advantage shrinks for weight
distributions that are not normal. The page gives no error figures; this
module computes them.

Readings: the uniform grid is the sixteen values -1 + 2i/15 (i = 0..15),
each rounded to fp32, so that it spans the same [-1, 1] as NF4 after the
same blockwise absmax normalisation; everything else (normalisation, nearest
value with ties to the lower code, w' = fl32(T[c] * absmax)) is the NF4
quantizer's rule with the other table.
"""

import numpy as np

from .nf4 import BLOCKSIZE, NF4_PRINTED, blockwise_absmax, nf4_codes

# Sixteen equally spaced values on [-1, 1] (fp64 values rounded to fp32).
UNIFORM4 = ((2.0 * np.arange(16) - 15.0) / 15.0).astype(np.float32)

GRIDS = {"nf4": NF4_PRINTED, "uniform": UNIFORM4}


def quantize_dequantize(w, table, blocksize=BLOCKSIZE):
    """w' = fl32(T[code] * absmax) for every weight of ``w`` (row-major
    flattening, blocks of ``blocksize``, a shorter last block)."""
    w = np.asarray(w, dtype=np.float32).ravel()
    a = blockwise_absmax(w, blocksize)
    codes = nf4_codes(w, a, blocksize, table=table)
    t = np.asarray(table, dtype=np.float32)
    return (t[codes] * a[np.arange(w.size) // blocksize]).astype(np.float32)


def quant_error(w, table, blocksize=BLOCKSIZE):
    """(sum (w - w')^2, sum w^2, max |w - w'|), all in fp64 (w - w' of two
    fp32 values is exact in fp64). Zeros for an empty input."""
    w = np.asarray(w, dtype=np.float32).ravel()
    if w.size == 0:
        return 0.0, 0.0, 0.0
    err = w.astype(np.float64) - quantize_dequantize(w, table, blocksize).astype(np.float64)
    w64 = w.astype(np.float64)
    return float(np.sum(err * err)), float(np.sum(w64 * w64)), float(np.max(np.abs(err)))
