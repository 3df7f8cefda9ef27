"""Seeded synthetic inputs shaped like the QLoRA workloads (7B / 65B linears).

This module only draws random numbers and fixes shapes; it holds none of the
method's arithmetic. Both the CPU oracle's tests and the HIP path take their
inputs from here, so the two are fed identical tensors.

Every tensor is drawn on the CPU with ``torch.Generator`` seeded as stated, so
it is identical on every machine with this torch build. "N(0, s)" means a
normal with standard deviation s.
"""

from dataclasses import dataclass

import torch


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal_weight(rows, cols, std, seed, outlier_frac=0.0, outlier_scale=20.0):
    """fp32 [rows, cols] ~ N(0, std); a Bernoulli(outlier_frac) mask of the
    entries is scaled by ``outlier_scale`` (large-magnitude outliers)."""
    g = _gen(seed)
    w = torch.randn(rows, cols, generator=g, dtype=torch.float32) * std
    if outlier_frac > 0:
        mask = torch.rand(rows, cols, generator=g) < outlier_frac
        w = torch.where(mask, w * outlier_scale, w)
    return w


def student_t_weight(rows, cols, df, scale, seed):
    """fp32 [rows, cols] ~ scale * Student-t(df), drawn as Z / sqrt(V/df) with
    V a sum of df squared standard normals (heavy-tailed weights)."""
    g = _gen(seed)
    z = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    v = torch.zeros(rows, cols, dtype=torch.float32)
    for _ in range(int(df)):
        e = torch.randn(rows, cols, generator=g, dtype=torch.float32)
        v += e * e
    return (z / torch.sqrt(v / df) * scale).to(torch.float32)


def keep_mask(rows, cols, p, seed):
    """bool [rows, cols]: each entry kept (True) with probability 1 - p (the
    dropout draws, made here and passed to both sides as an input)."""
    g = _gen(seed)
    return torch.rand(rows, cols, generator=g) >= p


def pack_keep_bits(keep):
    """bool [T, K] (K a multiple of 8) -> uint8 [T, K / 8], element 8i + j of a
    row in bit j (least significant first) of byte i: the layout the library
    takes the keep mask in."""
    k = keep.to(torch.uint8).reshape(keep.shape[0], -1, 8)
    weights = torch.tensor([1, 2, 4, 8, 16, 32, 64, 128], dtype=torch.int32)
    return (k.to(torch.int32) * weights).sum(dim=2).to(torch.uint8).contiguous()


def bf16_normal(shape, std, seed):
    """bf16 tensor ~ N(0, std) (drawn in fp32, rounded by torch's cast)."""
    g = _gen(seed)
    return (torch.randn(*shape, generator=g, dtype=torch.float32) * std).to(torch.bfloat16)


@dataclass
class LinearCase:
    """One linear layer's inputs: W fp32 [N, K]; X bf16 [T, K]; dY bf16 [T, N];
    A bf16 [r, K]; B bf16 [N, r]; scale = alpha / r."""

    name: str
    W: torch.Tensor
    X: torch.Tensor
    dY: torch.Tensor
    A: torch.Tensor
    B: torch.Tensor
    r: int
    alpha: float

    @property
    def scale(self):
        return self.alpha / self.r


def lora_case(name, W, T, r, alpha, a_std, b_std, seed):
    """Activations, upstream gradient and adapters for weight W."""
    N, K = W.shape
    X = bf16_normal((T, K), 1.0, seed * 7 + 1)
    dY = bf16_normal((T, N), 1.0, seed * 7 + 2)
    A = bf16_normal((r, K), a_std, seed * 7 + 3)
    B = bf16_normal((N, r), b_std, seed * 7 + 4)
    return LinearCase(name, W, X, dY, A, B, r, alpha)


def tiny_256(seed=0):
    """Single 256x256 linear: W ~ N(0, 0.02) seed 0; x bf16 [4, 256] ~ N(0,1);
    LoRA r=8, alpha=16, A ~ N(0, 1/256), B ~ N(0, 0.01)."""
    W = normal_weight(256, 256, 0.02, seed)
    return lora_case("tiny_256x256", W, 4, 8, 16.0, 1.0 / 256, 0.01, seed)


def attn_proj_7b(T=16, seed=1):
    """Llama-7B-shaped attention projection 4096x4096: W ~ N(0, 0.02) with 0.1%
    of entries scaled x20; decode token counts T in {1, 16}; r=16, alpha=32,
    A ~ N(0, 1/4096), B ~ N(0, 0.01)."""
    W = normal_weight(4096, 4096, 0.02, seed, outlier_frac=1e-3, outlier_scale=20.0)
    return lora_case("attn_proj_4096x4096", W, T, 16, 32.0, 1.0 / 4096, 0.01, seed)


def mlp_7b(which, T=1024, seed=2):
    """7B MLP linears: gate/up [11008, 4096], down [4096, 11008]; W ~ 0.02 *
    Student-t(5); x bf16 [1024, K]; r=16, alpha=32."""
    shapes = {"gate": (11008, 4096, 0), "up": (11008, 4096, 1), "down": (4096, 11008, 2)}
    n, k, off = shapes[which]
    W = student_t_weight(n, k, 5, 0.02, seed * 10 + off)
    return lora_case("mlp_%s_%dx%d" % (which, n, k), W, T, 16, 32.0, 1.0 / k, 0.01, seed * 10 + off)


LLAMA7B_LAYER = [
    ("q", 4096, 4096),
    ("k", 4096, 4096),
    ("v", 4096, 4096),
    ("o", 4096, 4096),
    ("gate", 11008, 4096),
    ("up", 11008, 4096),
    ("down", 4096, 11008),
]

LLAMA65B_SHAPES = [("sq", 8192, 8192), ("up", 22016, 8192), ("down", 8192, 22016)]


def llama7b_layer_linear(which, T=4096, seed=3):
    """One linear of the 32-layer 7B-shaped stack at T = 4096 tokens, LoRA
    r = 64, alpha = 16 on all linears. The stack's weight distribution is not
    stated: attention shapes take the 4096x4096 recipe (N(0, 0.02), 0.1 %
    outliers x20), MLP shapes the 0.02 Student-t(5) recipe."""
    shapes = {name: (n, k, i) for i, (name, n, k) in enumerate(LLAMA7B_LAYER)}
    n, k, off = shapes[which]
    s = seed * 10 + off
    if which in ("gate", "up", "down"):
        W = student_t_weight(n, k, 5, 0.02, s)
    else:
        W = normal_weight(n, k, 0.02, s, outlier_frac=1e-3, outlier_scale=20.0)
    return lora_case("llama7b_%s_%dx%d" % (which, n, k), W, T, 64, 16.0, 1.0 / k, 0.01, s)


def llama65b_linear(which, T=4096, seed=4):
    """65B-shaped linears 8192x8192, 22016x8192, 8192x22016: W ~ N(0, 0.015);
    x bf16 [4096, K]; LoRA r = 64, alpha = 16."""
    shapes = {name: (n, k, i) for i, (name, n, k) in enumerate(LLAMA65B_SHAPES)}
    n, k, off = shapes[which]
    s = seed * 10 + off
    W = normal_weight(n, k, 0.015, s)
    return lora_case("llama65b_%s_%dx%d" % (which, n, k), W, T, 64, 16.0, 1.0 / k, 0.01, s)
