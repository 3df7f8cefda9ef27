"""Forward and backward of the frozen-base LoRA linear layer (CPU oracle, fp64).

Test infrastructure only (see the package docstring).

Notation (aivaro.ru "Как работает QLoRA", §2): W in R^{d x k} (here N x K, the
frozen base, already dequantized), B in R^{d x r}, A in R^{r x k}, h = Wx + BAx.
apxml.com "量化 LoRA (QLoRA) 与 4 位训练": in QLoRA the base enters as
dequant(W_NF4). With a batch of row vectors X [T, K] the layer is

    U = X A^T          [T, r]
    H = X W'^T + s U B^T   [T, N],  s = alpha / r

(the scale s is the reading of the "lora_alpha" scaling factor; the printed
equations omit it). aivaro.ru §7: gradients flow through the dequantized
4-bit weight, which is never updated; only A and B are trained.
"""

import numpy as np

from .nf4 import f32_to_bf16_bits


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def lora_forward(X, Wd, A, B, scale):
    """Return (H, U) in fp64 from bf16-valued inputs X [T,K], dequantized
    W' [N,K], A [r,K], B [N,r]."""
    X, Wd, A, B = _f64(X), _f64(Wd), _f64(A), _f64(B)
    U = X @ A.T
    H = X @ Wd.T + float(scale) * (U @ B.T)
    return H, U


def lora_backward(X, dY, Wd, A, B, scale):
    """Return (dX, dA, dB, G, U) in fp64 for the upstream gradient dY [T,N]:

        G  = s dY B        [T, r]
        dX = dY W' + G A   [T, K]
        dA = G^T X         [r, K]
        dB = s dY^T U      [N, r]
    """
    X, dY, Wd, A, B = _f64(X), _f64(dY), _f64(Wd), _f64(A), _f64(B)
    s = float(scale)
    U = X @ A.T
    G = s * (dY @ B)
    dX = dY @ Wd + G @ A
    dA = G.T @ X
    dB = s * (dY.T @ U)
    return dX, dA, dB, G, U


def lora_merge(Wd, A, B, scale):
    """Merged 16-bit weight after training (ai-reference-codex "QLoRA 与 PEFT
    全家", §3.6: the adapter product is added back into the base weight, so
    inference needs no adapter branch; aivaro.ru §7, step 5; tqpw.cn notes,
    "Introduction": the adapters are 16-bit and cannot be folded into the
    4-bit weight, so the merged weight is 16-bit).

    Wd is the dequantized base w' as fp32 values [N, K] (before its bf16
    rounding), A [r, K], B [N, r]. Returns bf16 bit patterns of
    bf16(fl32(w' + s B A)), the product and the sum taken in fp64."""
    Wd, A, B = _f64(Wd), _f64(A), _f64(B)
    merged = Wd + float(scale) * (B @ A)
    return f32_to_bf16_bits(merged.astype(np.float32))


def lora_forward_dropout(X, Wd, A, B, scale, keep, p):
    """Forward with dropout on the adapter input (ai-reference-codex "QLoRA 与
    PEFT 全家", §3.4: dropout, 0.05-0.1 on the adapters for small data;
    aivaro.ru §11: lora_dropout = 0.05). Reading: inverted dropout of the
    adapter branch's input only, the keep mask ``keep`` [T, K] (0/1) given:

        U = X_d A^T / (1 - p),  X_d = X * keep
        H = X W'^T + s U B^T

    Returns (H, U) in fp64."""
    X, Wd, A, B, keep = _f64(X), _f64(Wd), _f64(A), _f64(B), _f64(keep)
    c = 1.0 / (1.0 - float(p))
    U = c * ((X * keep) @ A.T)
    H = X @ Wd.T + float(scale) * (U @ B.T)
    return H, U


def lora_backward_dropout(X, dY, Wd, A, B, scale, keep, p):
    """Backward of :func:`lora_forward_dropout` (fp64): the dropout's
    derivative passes the kept entries scaled by 1/(1 - p).

        G  = s dY B
        dX = dY W' + (G A) * keep / (1 - p)
        dA = G^T X_d / (1 - p)
        dB = s dY^T U

    Returns (dX, dA, dB, G, U)."""
    X, dY, Wd, A, B, keep = _f64(X), _f64(dY), _f64(Wd), _f64(A), _f64(B), _f64(keep)
    s = float(scale)
    c = 1.0 / (1.0 - float(p))
    Xd = X * keep
    U = c * (Xd @ A.T)
    G = s * (dY @ B)
    dX = dY @ Wd + c * ((G @ A) * keep)
    dA = c * (G.T @ Xd)
    dB = s * (dY.T @ U)
    return dX, dA, dB, G, U
