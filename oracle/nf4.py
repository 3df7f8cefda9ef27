"""Blockwise NF4 quantization, double quantization and dequantization (CPU oracle).

Test infrastructure only (see the package docstring). Plain, slow NumPy: each
function follows one step of the method as the pages state it, with no
blocking or fusion beyond what the step itself says.
"""

import numpy as np

# Weights per first-level block (aivaro.ru "Как работает QLoRA", §5: blocks of
# usually 64 weights; tqpw.cn QLoRA notes, "Double Quantization": NF4 at g64).
BLOCKSIZE = 64
# Absmax constants per second-level group (tqpw.cn QLoRA notes,
# "Double Quantization": FP8 at g256).
DQ_BLOCKSIZE = 256

# The sixteen NF4 values as printed, in the printed ascending order, on the
# tqpw.cn QLoRA notes, "NormalFloat Quantization (NF4)". A code is the
# position in this list: 0 is -1.0, 7 is 0.0, 15 is +1.0.
NF4_PRINTED = np.array(
    [
        -1.0,
        -0.6961928009986877,
        -0.5250730514526367,
        -0.39491748809814453,
        -0.28444138169288635,
        -0.18477343022823334,
        -0.09105003625154495,
        0.0,
        0.07958029955625534,
        0.16093020141124725,
        0.24611230194568634,
        0.33791524171829224,
        0.44070982933044434,
        0.5626170039176941,
        0.7229568362236023,
        1.0,
    ],
    dtype=np.float32,
)

_CHUNK = 1 << 20


def nf4_from_quantiles(k=4, delta=1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)):
    """Build the k-bit NormalFloat grid from standard-normal quantiles (fp64).

    tqpw.cn QLoRA notes, "NormalFloat Quantization (NF4)": the grid comes from
    the quantile function of the standard normal at equally spaced
    probabilities; the non-negative half takes 2^(k-1)+1 points (one of them
    +0), the non-positive half 2^(k-1) points (one of them -0); the halves are
    merged with one zero dropped, which leaves the grid asymmetric, and the
    result is normalised to [-1, 1].

    Reading: the pages do not give the outermost probability (the quantiles at
    0 and 1 are infinite); ``delta`` is that probability. The printed table is
    canonical; this construction is a check on it.
    """
    from scipy.special import ndtri  # standard-normal quantile function

    nonneg = ndtri(np.linspace(delta, 0.5, 2 ** (k - 1) + 1))  # ends at +0
    nonpos = -ndtri(np.linspace(delta, 0.5, 2 ** (k - 1)))  # ends at -0
    merged = np.sort(np.concatenate([nonneg, nonpos[:-1]]))  # one zero dropped
    return merged / np.max(np.abs(merged))


# ----------------------------------------------------------------------------
# Number formats: bf16 (the compute dtype) and OCP FP8 E4M3FN (the 8-bit code
# of the second-level constants).
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16, to nearest with ties to even; returns the
    16-bit patterns as uint16. apxml.com "量化 LoRA (QLoRA) 与 4 位训练": the
    compute dtype of the temporary dequantization is bfloat16."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    out = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b):
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def e4m3fn_value_table():
    """fp64 value of each of the 256 E4M3FN codes: 1 sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits, subnormals at exponent 0, no infinities, NaN at
    0x7F and 0xFF."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def e4m3fn_encode(y):
    """Encode fp32 values as E4M3FN: the nearest finite value, ties to the
    code with an even mantissa, the sign kept (so a negative value that rounds
    to zero gives 0x80). Magnitudes above 448 go to 448 (nearest finite).

    Reading (tqpw.cn QLoRA notes, "Double Quantization" says FP8 without a
    variant): OCP E4M3FN, round to nearest even."""
    y = np.asarray(y, dtype=np.float32).ravel()
    table = e4m3fn_value_table()
    mags = table[0:0x7F]  # codes 0x00..0x7E: the non-negative finite values, ascending
    out = np.empty(y.size, dtype=np.uint8)
    for s in range(0, y.size, _CHUNK):
        yy = y[s : s + _CHUNK].astype(np.float64)
        mag = np.abs(yy)
        dist = np.abs(mag[:, None] - mags[None, :])
        best = np.argmin(dist, axis=1)  # lowest code among the nearest
        dbest = dist[np.arange(best.size), best]
        nxt = np.minimum(best + 1, mags.size - 1)
        tie = (dist[np.arange(best.size), nxt] == dbest) & (nxt != best)
        best = np.where(tie & (best % 2 == 1), nxt, best)  # ties to even mantissa
        sign = np.signbit(yy).astype(np.uint8) << 7
        out[s : s + _CHUNK] = best.astype(np.uint8) | sign
    return out


def e4m3fn_decode(c):
    """fp32 value of E4M3FN codes (exact)."""
    return e4m3fn_value_table()[np.asarray(c, dtype=np.uint8)].astype(np.float32)


# ----------------------------------------------------------------------------
# First level: blockwise absmax + nearest NF4 code + 4-bit packing.
# ----------------------------------------------------------------------------


def blockwise_absmax(w, blocksize=BLOCKSIZE):
    """Per-block max |w| (fp32) over the row-major flattening of ``w``; the
    last block may be shorter. aivaro.ru "Как работает QLoRA", §5: one
    constant per block of (usually) 64 weights."""
    w = np.asarray(w, dtype=np.float32).ravel()
    nb = -(-w.size // blocksize)
    padded = np.zeros(nb * blocksize, dtype=np.float32)
    padded[: w.size] = np.abs(w)
    return padded.reshape(nb, blocksize).max(axis=1)


def nf4_codes(w, absmax, blocksize=BLOCKSIZE, table=NF4_PRINTED):
    """4-bit code of every weight: normalise the block to [-1, 1] by its
    absmax, then take the nearest of the sixteen NF4 values.

    tqpw.cn QLoRA notes, "NormalFloat Quantization (NF4)": the weights are
    first normalised to [-1, 1] and then quantized; ai-reference-codex
    "QLoRA 与 PEFT 全家", §3.1: each number is recorded as the nearest of the
    sixteen allowed values.

    Readings: the normalisation is x = fl32(w * fl32(1/absmax)); a tie
    between two nearest values goes to the lower code; a block whose absmax
    is 0 gets code 7 (the value 0) throughout. "Nearest, ties to the lower
    code" is decided exactly as "code = number of midpoints below x": the
    midpoint of two neighbouring fp32 table values is exact in fp64, and so
    is the comparison with the fp32 x (a distance argmin in fp64 cannot
    resolve an x within 1e-17 of a midpoint at zero, as the uniform grid has).
    """
    w = np.asarray(w, dtype=np.float32).ravel()
    absmax = np.asarray(absmax, dtype=np.float32)
    t64 = np.asarray(table, dtype=np.float32).astype(np.float64)
    mids = (t64[:-1] + t64[1:]) * 0.5  # ascending, exact
    codes = np.empty(w.size, dtype=np.uint8)
    for s in range(0, w.size, _CHUNK):
        ww = w[s : s + _CHUNK]
        a = absmax[(np.arange(s, s + ww.size)) // blocksize]
        with np.errstate(divide="ignore", invalid="ignore"):
            inv = np.float32(1.0) / a
            x = ww * inv
        x = np.where(a == 0, np.float32(0.0), x).astype(np.float32)
        # number of midpoints strictly below x (x on a midpoint: the lower code)
        codes[s : s + ww.size] = np.searchsorted(mids, x.astype(np.float64), side="left")
    return codes


def pack_nibbles(codes):
    """Two 4-bit codes per byte, the earlier element in the high nibble; an
    odd count pads the last low nibble with code 7. apxml.com page: the base
    stays in memory as 4-bit data (the byte layout is a reading)."""
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    if codes.size % 2:
        codes = np.concatenate([codes, np.array([7], dtype=np.uint8)])
    pairs = codes.reshape(-1, 2)
    return ((pairs[:, 0] << 4) | pairs[:, 1]).astype(np.uint8)


def unpack_nibbles(packed, n):
    """Inverse of :func:`pack_nibbles` for ``n`` codes."""
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    codes = np.empty(packed.size * 2, dtype=np.uint8)
    codes[0::2] = packed >> 4
    codes[1::2] = packed & 0xF
    return codes[:n]


def quantize(w, blocksize=BLOCKSIZE):
    """First-level NF4 quantization of ``w`` (fp32 values; bf16 input is
    widened exactly before it comes here). Returns (packed uint8, absmax fp32)."""
    w = np.asarray(w, dtype=np.float32)
    absmax = blockwise_absmax(w, blocksize)
    return pack_nibbles(nf4_codes(w, absmax, blocksize)), absmax


# ----------------------------------------------------------------------------
# Second level: double quantization of the absmax constants.
# ----------------------------------------------------------------------------


def pairwise_tree_sum(values):
    """fp64 sum over a contiguous pairwise tree: zero-pad to a power of two,
    then add neighbours (2j, 2j+1) level by level.

    Reading: the pages ask for the mean of the constants but fix no order of
    summation; this order sets the fp32 rounding of the mean bit for bit."""
    v = np.asarray(values, dtype=np.float64).ravel()
    p = 1
    while p < v.size:
        p *= 2
    buf = np.zeros(p, dtype=np.float64)
    buf[: v.size] = v
    while buf.size > 1:
        buf = buf[0::2] + buf[1::2]
    return buf[0]


def double_quant(absmax, dq_blocksize=DQ_BLOCKSIZE):
    """Quantize the fp32 absmax constants to 8 bits.

    tqpw.cn QLoRA notes, "Double Quantization": the first-level constants are
    quantized again with FP8 at group size 256; since they are all positive,
    their mean is subtracted first and the rest is quantized symmetrically.
    apxml.com page ("双重量化"): this takes the constants from 32 to 8 bits.

    Readings: one mean per tensor, mu = fl32(tree_sum_fp64 / n1); d = fl32(a -
    mu); per group s = max|d| and scale S = fl32(s / 448) (448 being the
    largest E4M3FN value); code = E4M3FN(fl32(d / S)); a group with S = 0 gets
    codes 0x00. Returns (c8 uint8 [n1], scale fp32 [ceil(n1/256)], mean fp32).
    """
    a = np.asarray(absmax, dtype=np.float32).ravel()
    n1 = a.size
    mean = np.float32(pairwise_tree_sum(a) / np.float64(n1))
    d = (a - mean).astype(np.float32)
    ng = -(-n1 // dq_blocksize)
    padded = np.zeros(ng * dq_blocksize, dtype=np.float32)
    padded[:n1] = np.abs(d)
    smax = padded.reshape(ng, dq_blocksize).max(axis=1)
    scale = (smax / np.float32(448.0)).astype(np.float32)
    g = np.arange(n1) // dq_blocksize
    sg = scale[g]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (d / sg).astype(np.float32)
    y = np.where(sg == 0, np.float32(0.0), y)
    c8 = e4m3fn_encode(y)
    c8 = np.where(sg == 0, np.uint8(0), c8).astype(np.uint8)
    return c8, scale, mean


def dequant_absmax(c8, scale, mean, dq_blocksize=DQ_BLOCKSIZE):
    """Recover the first-level constants: a' = fl32(fl32(E(c8) * S) + mu),
    with no fused multiply-add (a reading)."""
    c8 = np.asarray(c8, dtype=np.uint8).ravel()
    scale = np.asarray(scale, dtype=np.float32)
    g = np.arange(c8.size) // dq_blocksize
    prod = (e4m3fn_decode(c8) * scale[g]).astype(np.float32)
    return (prod + np.float32(mean)).astype(np.float32)


def dequantize(packed, absmax_eff, n, blocksize=BLOCKSIZE, out="bf16", table=NF4_PRINTED):
    """Dequantize ``n`` weights: w' = fl32(T[code] * a'), then (for the bf16
    output) rounded to bf16 to nearest even. apxml.com page: the 4-bit weight
    is temporarily dequantized to the compute dtype (bfloat16) for the
    matmul. Returns uint16 bf16 bit patterns, or fp32 values for out='f32'."""
    codes = unpack_nibbles(packed, n)
    a = np.asarray(absmax_eff, dtype=np.float32)[np.arange(n) // blocksize]
    w = (np.asarray(table, dtype=np.float32)[codes] * a).astype(np.float32)
    if out == "f32":
        return w
    return f32_to_bf16_bits(w)


def dq_bits_per_param(blocksize=BLOCKSIZE, dq_blocksize=DQ_BLOCKSIZE):
    """Storage overhead of the quantization constants, in bits per weight:
    8 bits per first-level block plus 32 bits per second-level group
    (the mean, one per tensor, is not counted)."""
    return 8.0 / blocksize + 32.0 / (blocksize * dq_blocksize)
