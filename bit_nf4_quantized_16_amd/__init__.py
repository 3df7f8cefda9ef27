"""MI355X (gfx950) QLoRA frozen-base linear layer: blockwise NF4 quantization
with double quantization, and the LoRA forward / backward on the 4-bit base.

The functions below carry the names of the C ABI (include/qlora_nf4.h) and do
argument marshalling only: every step runs in the HIP library
libqlora_nf4.so. torch supplies device memory and the current stream.
Importing this package fails if the library has not been built.
"""

import ctypes
from dataclasses import dataclass

import torch

from . import _lib

lib = _lib.load()

__all__ = [
    "NF4Weight",
    "QLoraError",
    "nf4_quantize",
    "nf4_double_quant",
    "nf4_dequantize",
    "qlora_merge",
    "q4_quant_error",
    "qlora_linear_fwd",
    "qlora_linear_fwd_group",
    "qlora_linear_bwd",
    "qlora_linear_bwd_group",
    "quantize_weight",
    "QLoRALinearFunction",
    "QLoRAGroupFunction",
    "KernelTimer",
    "lib",
]

BLOCKSIZE = 64
DQ_BLOCKSIZE = 256


class QLoraError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (%d): %s" % (lib.qlora_status_string(status).decode(), status, message))
        self.status = status


def _check(status):
    if status != _lib.QL_OK:
        raise QLoraError(status, lib.qlora_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _bits(t):
    """bf16 tensor -> its storage (the library takes bf16 as raw 16-bit)."""
    if t is None:
        return None
    assert t.dtype == torch.bfloat16 and t.is_contiguous(), "expected a contiguous bf16 tensor"
    return t


def _workspace(nbytes, device):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


@dataclass
class NF4Weight:
    """A frozen weight in NF4 (+ double-quantized constants) on the device."""

    rows: int
    cols: int
    packed: torch.Tensor
    absmax: torch.Tensor = None  # fp32 [nblocks]; kept when double_quant=False
    c8: torch.Tensor = None  # uint8 [nblocks]
    dq_scale: torch.Tensor = None  # fp32 [ngroups]
    dq_mean: torch.Tensor = None  # fp32 [1]

    @property
    def double_quant(self):
        return self.c8 is not None

    @property
    def shape(self):
        return (self.rows, self.cols)

    def nbytes(self):
        n = self.packed.numel()
        if self.double_quant:
            n += self.c8.numel() + 4 * self.dq_scale.numel() + 4
        else:
            n += 4 * self.absmax.numel()
        return n

    def descriptor(self):
        d = _lib.QlNf4Weight()
        d.rows = self.rows
        d.cols = self.cols
        d.blocksize = BLOCKSIZE
        d.dq_blocksize = DQ_BLOCKSIZE if self.double_quant else 0
        d.packed = self.packed.data_ptr()
        d.absmax = self.absmax.data_ptr() if self.absmax is not None else None
        d.c8 = self.c8.data_ptr() if self.double_quant else None
        d.dq_scale = self.dq_scale.data_ptr() if self.double_quant else None
        d.dq_mean = self.dq_mean.data_ptr() if self.double_quant else None
        return d


def nf4_quantize(W, packed=None, absmax=None):
    """First-level NF4 quantization of a 2-D fp32/bf16 device tensor.
    Returns (packed uint8 [ceil(n/2)], absmax fp32 [ceil(n/64)])."""
    assert W.is_cuda and W.dim() == 2 and W.is_contiguous()
    rows, cols = W.shape
    dtype = {torch.float32: _lib.QL_F32, torch.bfloat16: _lib.QL_BF16}[W.dtype]
    if packed is None:
        packed = torch.empty(lib.nf4_packed_bytes(rows, cols), dtype=torch.uint8, device=W.device)
    if absmax is None:
        absmax = torch.empty(lib.nf4_num_blocks(rows, cols, BLOCKSIZE), dtype=torch.float32, device=W.device)
    _check(lib.nf4_quantize(_ptr(W), dtype, rows, cols, BLOCKSIZE, _ptr(packed), _ptr(absmax), _stream()))
    return packed, absmax


def nf4_double_quant(absmax):
    """Second-level quantization of the fp32 absmax constants.
    Returns (c8 uint8 [n1], scale fp32 [ceil(n1/256)], mean fp32 [1])."""
    n1 = absmax.numel()
    dev = absmax.device
    c8 = torch.empty(n1, dtype=torch.uint8, device=dev)
    scale = torch.empty(lib.nf4_dq_num_groups(n1, DQ_BLOCKSIZE), dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(lib.nf4_double_quant_workspace(n1), dev)
    _check(
        lib.nf4_double_quant(_ptr(absmax), n1, DQ_BLOCKSIZE, _ptr(c8), _ptr(scale), _ptr(mean), _ptr(ws), wsb, _stream())
    )
    return c8, scale, mean


def nf4_quantize_dq(W):
    """nf4_quantize and nf4_double_quant in one call (two launches where the
    size allows). Returns (packed, absmax, c8, scale, mean)."""
    assert W.is_cuda and W.dim() == 2 and W.is_contiguous()
    rows, cols = W.shape
    dtype = {torch.float32: _lib.QL_F32, torch.bfloat16: _lib.QL_BF16}[W.dtype]
    dev = W.device
    n1 = lib.nf4_num_blocks(rows, cols, BLOCKSIZE)
    packed = torch.empty(lib.nf4_packed_bytes(rows, cols), dtype=torch.uint8, device=dev)
    absmax = torch.empty(n1, dtype=torch.float32, device=dev)
    c8 = torch.empty(n1, dtype=torch.uint8, device=dev)
    scale = torch.empty(lib.nf4_dq_num_groups(n1, DQ_BLOCKSIZE), dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(lib.nf4_quantize_dq_workspace(rows, cols, dtype), dev)
    _check(lib.nf4_quantize_dq(_ptr(W), dtype, rows, cols, BLOCKSIZE, _ptr(packed), _ptr(absmax), DQ_BLOCKSIZE,
                               _ptr(c8), _ptr(scale), _ptr(mean), _ptr(ws), wsb, _stream()))
    return packed, absmax, c8, scale, mean


def quantize_weight(W, double_quant=True, keep_absmax=False):
    """nf4_quantize_dq (or nf4_quantize alone) into an NF4Weight."""
    if not double_quant:
        packed, absmax = nf4_quantize(W)
        return NF4Weight(W.shape[0], W.shape[1], packed, absmax=absmax)
    packed, absmax, c8, scale, mean = nf4_quantize_dq(W)
    return NF4Weight(W.shape[0], W.shape[1], packed, absmax=absmax if keep_absmax else None, c8=c8, dq_scale=scale,
                     dq_mean=mean)


def nf4_dequantize(w, dtype=torch.bfloat16, out=None):
    """Expand an NF4Weight to a [rows, cols] bf16 (or fp32) device tensor."""
    od = {torch.float32: _lib.QL_F32, torch.bfloat16: _lib.QL_BF16}[dtype]
    if out is None:
        out = torch.empty(w.rows, w.cols, dtype=dtype, device=w.packed.device)
    d = w.descriptor()
    _check(lib.nf4_dequantize(ctypes.byref(d), _ptr(out), od, _stream()))
    return out


def qlora_merge(w, A=None, B=None, scale=1.0, out=None):
    """bf16 [rows, cols] = dequant(W) + scale * B @ A (one rounding to bf16)."""
    r = 0 if A is None else A.shape[0]
    if out is None:
        out = torch.empty(w.rows, w.cols, dtype=torch.bfloat16, device=w.packed.device)
    d = w.descriptor()
    _check(lib.qlora_merge(ctypes.byref(d), _ptr(_bits(A)), _ptr(_bits(B)), r, float(scale), _ptr(out), _stream()))
    return out


def q4_quant_error(W, grid="nf4", stats=None):
    """Blockwise-absmax 4-bit quantization error of W (fp32 or bf16, 2-D) on
    the NF4 or the uniform grid: fp64 device tensor [sum (w-w')^2, sum w^2,
    max |w-w'|]."""
    dt = {torch.float32: _lib.QL_F32, torch.bfloat16: _lib.QL_BF16}[W.dtype]
    g = {"nf4": _lib.QL_GRID_NF4, "uniform": _lib.QL_GRID_UNIFORM}[grid]
    assert W.is_contiguous()
    rows, cols = (W.shape[0], W.numel() // W.shape[0]) if W.dim() >= 1 and W.shape[0] > 0 else (0, 0)
    if stats is None:
        stats = torch.empty(3, dtype=torch.float64, device=W.device)
    ws, wsb = _workspace(lib.q4_quant_error_workspace(rows, cols, dt), W.device)
    _check(lib.q4_quant_error(_ptr(W), dt, rows, cols, BLOCKSIZE, g, _ptr(stats), _ptr(ws), wsb, _stream()))
    return stats


def _keep(keep, T, K):
    assert keep.dtype == torch.uint8 and keep.is_contiguous() and keep.numel() == T * (K // 8), \
        "keep: bit-packed uint8 [T, K/8]"
    return keep


def qlora_linear_fwd(w, X, A=None, B=None, scale=1.0, save_u=True, out=None, keep=None, p=0.0):
    """Y = X W'^T + scale (X A^T) B^T. Returns (Y bf16 [T, N], U fp32 [T, r] or None).
    With ``keep`` (bit-packed uint8 [T, K/8]) and ``p``: dropout on the
    adapter input, U = (X * keep) A^T / (1 - p)."""
    T = X.shape[0]
    r = 0 if A is None else A.shape[0]
    dev = X.device
    Y = out if out is not None else torch.empty(T, w.rows, dtype=torch.bfloat16, device=dev)
    U = torch.empty(T, r, dtype=torch.float32, device=dev) if (save_u and r > 0) else None
    d = w.descriptor()
    if keep is None:
        ws, wsb = _workspace(lib.qlora_linear_fwd_workspace(w.rows, w.cols, max(T, 1), r), dev)
        _check(
            lib.qlora_linear_fwd(ctypes.byref(d), _ptr(_bits(X)), T, _ptr(_bits(A)), _ptr(_bits(B)), r, float(scale),
                                 _ptr(Y), _ptr(U), _ptr(ws), wsb, _stream())
        )
    else:
        ws, wsb = _workspace(lib.qlora_linear_fwd_dropout_workspace(w.rows, w.cols, max(T, 1), r), dev)
        _check(
            lib.qlora_linear_fwd_dropout(ctypes.byref(d), _ptr(_bits(X)), T, _ptr(_bits(A)), _ptr(_bits(B)), r,
                                         float(scale), _ptr(_keep(keep, T, w.cols)), float(p), _ptr(Y), _ptr(U),
                                         _ptr(ws), wsb, _stream())
        )
    return Y, U


def qlora_linear_fwd_noalloc(w, X, A=None, B=None, scale=1.0, save_u=True, out=None, U_out=None):
    """qlora_linear_fwd through the entry point that allocates nothing (its
    scratch is a device array of the library, shared by every call on a GPU).
    Pass ``out`` (and ``U_out``) to keep this function from allocating the
    outputs as well. Returns (Y, U or None)."""
    T = X.shape[0]
    r = 0 if A is None else A.shape[0]
    dev = X.device
    Y = out if out is not None else torch.empty(T, w.rows, dtype=torch.bfloat16, device=dev)
    U = U_out
    if U is None and save_u and r > 0:
        U = torch.empty(T, r, dtype=torch.float32, device=dev)
    d = w.descriptor()
    _check(lib.qlora_linear_fwd_noalloc(ctypes.byref(d), _ptr(_bits(X)), T, _ptr(_bits(A)), _ptr(_bits(B)), r,
                                        float(scale), _ptr(Y), _ptr(U), _stream()))
    return Y, U


def qlora_linear_fwd_group(ws, X, As=None, Bs=None, scale=1.0, save_u=True):
    """qlora_linear_fwd for up to four layers that read the same X (q/k/v,
    gate/up): one launch when T <= 16. ``ws`` NF4Weights sharing ``cols``;
    ``As``/``Bs`` lists of adapters (None for r = 0). Returns a list of
    (Y, U) pairs, as qlora_linear_fwd."""
    nw = len(ws)
    T = X.shape[0]
    r = 0 if As is None else As[0].shape[0]
    dev = X.device
    Ys = [torch.empty(T, w.rows, dtype=torch.bfloat16, device=dev) for w in ws]
    Us = [torch.empty(T, r, dtype=torch.float32, device=dev) if (save_u and r > 0) else None for _ in ws]
    descs = [w.descriptor() for w in ws]
    arr = lambda ts: (ctypes.c_void_p * max(nw, 1))(*[_ptr(t) for t in ts])
    wp = (ctypes.c_void_p * max(nw, 1))(*[ctypes.addressof(d) for d in descs])
    rows = (ctypes.c_int64 * max(nw, 1))(*[w.rows for w in ws])
    cols = ws[0].cols if nw else 0
    ws_, wsb = _workspace(lib.qlora_linear_fwd_group_workspace(rows, nw, cols, max(T, 1), r), dev)
    As_ = arr([_bits(a) for a in As]) if As is not None else None
    Bs_ = arr([_bits(b) for b in Bs]) if Bs is not None else None
    _check(
        lib.qlora_linear_fwd_group(wp, nw, _ptr(_bits(X)), T, As_, Bs_, r, float(scale), arr(Ys), arr(Us), _ptr(ws_),
                                   wsb, _stream())
    )
    return list(zip(Ys, Us))


def qlora_linear_bwd(w, X, dY, A=None, B=None, scale=1.0, U=None, need_dx=True, need_da=True, need_db=True, dA=None,
                     dB=None, accumulate=False, keep=None, p=0.0):
    """Returns (dX bf16 [T, K] or None, dA fp32 [r, K] or None, dB fp32 [N, r] or None).
    ``keep`` / ``p``: the forward's dropout mask and probability."""
    T = dY.shape[0]
    r = 0 if A is None else A.shape[0]
    dev = dY.device
    dX = torch.empty(T, w.cols, dtype=torch.bfloat16, device=dev) if need_dx else None
    if r > 0 and need_da and dA is None:
        dA = (torch.zeros if accumulate else torch.empty)(r, w.cols, dtype=torch.float32, device=dev)
    if r > 0 and need_db and dB is None:
        dB = (torch.zeros if accumulate else torch.empty)(w.rows, r, dtype=torch.float32, device=dev)
    if not need_da:
        dA = None
    if not need_db:
        dB = None
    d = w.descriptor()
    if keep is None:
        ws, wsb = _workspace(lib.qlora_linear_bwd_workspace(w.rows, w.cols, max(T, 1), r), dev)
        _check(
            lib.qlora_linear_bwd(ctypes.byref(d), _ptr(_bits(X)), _ptr(_bits(dY)), T, _ptr(_bits(A)), _ptr(_bits(B)),
                                 r, float(scale), _ptr(U), _ptr(dX), _ptr(dA), _ptr(dB), 1 if accumulate else 0,
                                 _ptr(ws), wsb, _stream())
        )
    else:
        ws, wsb = _workspace(lib.qlora_linear_bwd_dropout_workspace(w.rows, w.cols, max(T, 1), r), dev)
        _check(
            lib.qlora_linear_bwd_dropout(ctypes.byref(d), _ptr(_bits(X)), _ptr(_bits(dY)), T, _ptr(_bits(A)),
                                         _ptr(_bits(B)), r, float(scale), _ptr(_keep(keep, T, w.cols)), float(p),
                                         _ptr(U), _ptr(dX), _ptr(dA), _ptr(dB), 1 if accumulate else 0, _ptr(ws), wsb,
                                         _stream())
        )
    return dX, dA, dB


def qlora_linear_bwd_group(ws, X, dYs, As=None, Bs=None, scale=1.0, Us=None, need_dx=True, need_da=True,
                           need_db=True, dAs=None, dBs=None, accumulate=False):
    """qlora_linear_bwd for up to four layers that read the same X (q/k/v,
    gate/up). Returns (dX bf16 [T, K] = the sum of the layers' input
    gradients, or None; list of dA or None; list of dB or None). ``ws``
    NF4Weights sharing ``cols``; ``dYs`` their upstream gradients; ``As``,
    ``Bs``, ``Us`` lists per layer (None for r = 0 / no saved U)."""
    nw = len(ws)
    T = dYs[0].shape[0]
    r = 0 if As is None else As[0].shape[0]
    dev = dYs[0].device
    cols = ws[0].cols if nw else 0
    dX = torch.empty(T, cols, dtype=torch.bfloat16, device=dev) if need_dx else None
    new = torch.zeros if accumulate else torch.empty
    if r > 0 and need_da and dAs is None:
        dAs = [new(r, cols, dtype=torch.float32, device=dev) for _ in ws]
    if r > 0 and need_db and dBs is None:
        dBs = [new(w.rows, r, dtype=torch.float32, device=dev) for w in ws]
    if not need_da:
        dAs = None
    if not need_db:
        dBs = None
    descs = [w.descriptor() for w in ws]
    arr = lambda ts: (ctypes.c_void_p * max(nw, 1))(*[_ptr(t) for t in ts]) if ts is not None else None
    wp = (ctypes.c_void_p * max(nw, 1))(*[ctypes.addressof(d) for d in descs])
    rows = (ctypes.c_int64 * max(nw, 1))(*[w.rows for w in ws])
    ws_, wsb = _workspace(lib.qlora_linear_bwd_group_workspace(rows, nw, cols, max(T, 1), r), dev)
    _check(
        lib.qlora_linear_bwd_group(wp, nw, _ptr(_bits(X)), arr([_bits(d) for d in dYs]), T,
                                   arr([_bits(a) for a in As]) if As is not None else None,
                                   arr([_bits(b) for b in Bs]) if Bs is not None else None, r, float(scale), arr(Us),
                                   _ptr(dX), arr(dAs), arr(dBs), 1 if accumulate else 0, _ptr(ws_), wsb, _stream())
    )
    return dX, dAs, dBs


def paged_adamw_step(param, grad, exp_avg, exp_avg_sq, step, lr=2e-4, betas=(0.9, 0.999), eps=1e-8,
                     weight_decay=0.0, param_bf16=None, copy_stream=None):
    """One AdamW step (fp32 state) of a flat fp32 parameter tensor in place.
    ``exp_avg`` / ``exp_avg_sq``: fp32 tensors of the same size, both on the
    GPU or both in pinned host memory (``pin_memory=True``): paged-out state
    is read and written in place over the host link (pinned memory is mapped
    into the device's address space); with QLORA_NF4_ADAMW_PAGING=staged it
    streams through a device staging buffer instead, its copies on
    ``copy_stream`` (a torch.cuda.Stream; None runs them on the current
    stream).
    ``param_bf16``: optional bf16 tensor that receives the updated values."""
    n = param.numel()
    for t in (param, grad, exp_avg, exp_avg_sq):
        assert t.dtype == torch.float32 and t.is_contiguous() and t.numel() == n
    if param_bf16 is not None:
        assert param_bf16.dtype == torch.bfloat16 and param_bf16.is_contiguous() and param_bf16.numel() == n
    ws, wsb = (None, 0)
    if not exp_avg.is_cuda:
        ws, wsb = _workspace(lib.qlora_paged_adamw_workspace(n), param.device)
    cs = ctypes.c_void_p(copy_stream.cuda_stream) if copy_stream is not None else None
    _check(lib.qlora_paged_adamw(_ptr(param), _ptr(param_bf16), _ptr(grad), _ptr(exp_avg), _ptr(exp_avg_sq), n,
                                 int(step), float(lr), float(betas[0]), float(betas[1]), float(eps),
                                 float(weight_decay), _ptr(ws), wsb, _stream(), cs))
    return param


class QLoRALinearFunction(torch.autograd.Function):
    """autograd wrapper: forward / backward run in the HIP library; W is frozen
    (no gradient), A and B receive fp32 gradients cast to their dtype."""

    @staticmethod
    def forward(ctx, X, A, B, w, scale, keep=None, p=0.0):
        Y, U = qlora_linear_fwd(w, X.contiguous(), A.contiguous(), B.contiguous(), scale, save_u=True, keep=keep, p=p)
        ctx.save_for_backward(X, A, B, U)
        ctx.w = w
        ctx.scale = scale
        ctx.keep = keep
        ctx.p = p
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, A, B, U = ctx.saved_tensors
        dX, dA, dB = qlora_linear_bwd(ctx.w, X, dY.contiguous().to(torch.bfloat16), A, B, ctx.scale, U=U,
                                      need_dx=ctx.needs_input_grad[0], keep=ctx.keep, p=ctx.p)
        return dX, dA.to(A.dtype), dB.to(B.dtype), None, None, None, None


class QLoRAGroupFunction(torch.autograd.Function):
    """autograd wrapper for up to four layers that read the same X (q/k/v,
    gate/up): apply(X, scale, ws, A_0, B_0, A_1, B_1, ...) returns the
    layers' Y; the forward is one qlora_linear_fwd_group call, the backward
    one qlora_linear_bwd_group call (X receives the summed input gradient;
    the weights in ``ws`` are frozen)."""

    @staticmethod
    def forward(ctx, X, scale, ws, *adapters):
        As, Bs = [a.contiguous() for a in adapters[0::2]], [b.contiguous() for b in adapters[1::2]]
        outs = qlora_linear_fwd_group(ws, X.contiguous(), As, Bs, scale)
        ctx.save_for_backward(X, *As, *Bs, *[U for _, U in outs])
        ctx.ws = ws
        ctx.scale = scale
        return tuple(Y for Y, _ in outs)

    @staticmethod
    def backward(ctx, *dYs):
        n = len(ctx.ws)
        saved = ctx.saved_tensors
        X, As, Bs, Us = saved[0], list(saved[1:1 + n]), list(saved[1 + n:1 + 2 * n]), list(saved[1 + 2 * n:])
        dYs = [(d if d is not None else torch.zeros(X.shape[0], w.rows, device=X.device)).contiguous()
               .to(torch.bfloat16) for d, w in zip(dYs, ctx.ws)]
        dX, dAs, dBs = qlora_linear_bwd_group(ctx.ws, X, dYs, As, Bs, ctx.scale, Us=Us,
                                              need_dx=ctx.needs_input_grad[0])
        grads = []
        for i in range(n):
            grads += [dAs[i].to(As[i].dtype), dBs[i].to(Bs[i].dtype)]
        return (dX, None, None, *grads)


class KernelTimer:
    """HIP-event timer of one library kernel (QL_KERNEL_* id): arm(), run the
    work, read() -> (launches, total milliseconds)."""

    def __init__(self, kernel_id):
        self.kid = kernel_id

    def arm(self):
        _check(lib.qlora_timer_arm(self.kid))

    def read(self):
        n = ctypes.c_int64(0)
        ms = ctypes.c_double(0.0)
        _check(lib.qlora_timer_read(self.kid, ctypes.byref(n), ctypes.byref(ms)))
        return n.value, ms.value

    def disarm(self):
        _check(lib.qlora_timer_disarm(self.kid))
