"""ctypes loader of libqlora_nf4.so and the C declarations of include/qlora_nf4.h.

Loading fails loudly (ImportError) when the built library is missing: the
package has no fallback path of any kind.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqlora_nf4.so")

QL_OK = 0
QL_ERR_NULL = -1
QL_ERR_SHAPE = -2
QL_ERR_UNSUPPORTED = -3
QL_ERR_ALIGN = -4
QL_ERR_WORKSPACE = -5
QL_ERR_HIP = -6

QL_F32 = 0
QL_BF16 = 1

QL_KERNEL_QUANTIZE = 1
QL_KERNEL_DQ_ENCODE = 2
QL_KERNEL_DEQUANTIZE = 3
QL_KERNEL_GEMV = 4
QL_KERNEL_GEMM_FWD = 5
QL_KERNEL_GEMM_DX = 6
QL_KERNEL_LORA_GRAD = 7
QL_KERNEL_MERGE = 8
QL_KERNEL_QERROR = 9
QL_KERNEL_KEEP_APPLY = 10
QL_KERNEL_DX_KEEP = 11
QL_KERNEL_ADAMW = 12
QL_NOALLOC_SCRATCH_BYTES = 96 << 20  # include/qlora_nf4.h
QL_GRID_NF4 = 0
QL_GRID_UNIFORM = 1


class QlNf4Weight(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("blocksize", ctypes.c_int32),
        ("dq_blocksize", ctypes.c_int32),
        ("packed", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("c8", ctypes.c_void_p),
        ("dq_scale", ctypes.c_void_p),
        ("dq_mean", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_WP = ctypes.POINTER(QlNf4Weight)

# name -> (restype, argtypes); the exported surface of include/qlora_nf4.h
SIGNATURES = {
    "nf4_packed_bytes": (_SZ, [_I64, _I64]),
    "nf4_num_blocks": (_I64, [_I64, _I64, _I32]),
    "nf4_dq_num_groups": (_I64, [_I64, _I32]),
    "nf4_quantize": (_I, [_P, _I, _I64, _I64, _I32, _P, _P, _P]),
    "nf4_double_quant_workspace": (_SZ, [_I64]),
    "nf4_double_quant": (_I, [_P, _I64, _I32, _P, _P, _P, _P, _SZ, _P]),
    "nf4_quantize_dq_workspace": (_SZ, [_I64, _I64, _I]),
    "nf4_quantize_dq": (_I, [_P, _I, _I64, _I64, _I32, _P, _P, _I32, _P, _P, _P, _P, _SZ, _P]),
    "nf4_dequantize": (_I, [_WP, _P, _I, _P]),
    "qlora_merge": (_I, [_WP, _P, _P, _I32, _F, _P, _P]),
    "q4_quant_error_workspace": (_SZ, [_I64, _I64, _I]),
    "q4_quant_error": (_I, [_P, _I, _I64, _I64, _I32, _I32, _P, _P, _SZ, _P]),
    "qlora_linear_fwd_workspace": (_SZ, [_I64, _I64, _I64, _I32]),
    "qlora_linear_fwd_u_in_launch": (_I32, [_I64, _I64, _I64, _I32]),
    "qlora_linear_bwd_g_in_launch": (_I32, [_I64, _I64, _I64, _I32]),
    "qlora_linear_fwd": (_I, [_WP, _P, _I64, _P, _P, _I32, _F, _P, _P, _P, _SZ, _P]),
    "qlora_linear_fwd_noalloc": (_I, [_WP, _P, _I64, _P, _P, _I32, _F, _P, _P, _P]),
    "qlora_linear_fwd_group_workspace": (_SZ, [_P, _I32, _I64, _I64, _I32]),
    "qlora_linear_fwd_group_one_launch": (_I32, [_P, _I32, _I64, _I64, _I32]),
    "qlora_linear_fwd_group": (_I, [_P, _I32, _P, _I64, _P, _P, _I32, _F, _P, _P, _P, _SZ, _P]),
    "qlora_linear_fwd_dropout_workspace": (_SZ, [_I64, _I64, _I64, _I32]),
    "qlora_linear_fwd_dropout": (_I, [_WP, _P, _I64, _P, _P, _I32, _F, _P, _F, _P, _P, _P, _SZ, _P]),
    "qlora_linear_bwd_workspace": (_SZ, [_I64, _I64, _I64, _I32]),
    "qlora_linear_bwd": (_I, [_WP, _P, _P, _I64, _P, _P, _I32, _F, _P, _P, _P, _P, _I, _P, _SZ, _P]),
    "qlora_linear_bwd_group_workspace": (_SZ, [_P, _I32, _I64, _I64, _I32]),
    "qlora_linear_bwd_group": (_I, [_P, _I32, _P, _P, _I64, _P, _P, _I32, _F, _P, _P, _P, _P, _I, _P, _SZ, _P]),
    "qlora_linear_bwd_dropout_workspace": (_SZ, [_I64, _I64, _I64, _I32]),
    "qlora_linear_bwd_dropout": (_I, [_WP, _P, _P, _I64, _P, _P, _I32, _F, _P, _F, _P, _P, _P, _P, _I, _P, _SZ, _P]),
    "qlora_paged_adamw_workspace": (_SZ, [_I64]),
    "qlora_paged_adamw": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _F, _F, _F, _F, _F, _P, _SZ, _P, _P]),
    "qlora_status_string": (ctypes.c_char_p, [_I]),
    "qlora_last_error": (ctypes.c_char_p, []),
    "qlora_timer_arm": (_I, [_I]),
    "qlora_timer_read": (_I, [_I, ctypes.POINTER(_I64), ctypes.POINTER(ctypes.c_double)]),
    "qlora_timer_disarm": (_I, [_I]),
}


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            "libqlora_nf4.so is not built (%s); run `python bit_nf4_quantized_16_amd/build.py` "
            "or __graft_entry__.build()" % path
        )
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib
