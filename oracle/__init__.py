"""Plain CPU oracle for the QLoRA frozen-base linear layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or calls
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code, table or
constant with the HIP library in ``bit_nf4_quantized_16_amd/``; the two meet
only through the seeded input generators in ``workloads/``.

Sources (web pages on QLoRA; cited by title and section):
  * tqpw.cn QLoRA notes, "Method" > "NormalFloat Quantization (NF4)" and
    "Double Quantization"
  * aivaro.ru "Как работает QLoRA (Quantized LoRA) для training?", §2, §5, §7
  * apxml.com "量化 LoRA (QLoRA) 与 4 位训练" (the h = dequant(W_NF4)x + BAx
    equation and the four configuration knobs)
  * ai-reference-codex "QLoRA 与 PEFT 全家", §3.1-§3.3, §3.4 (dropout), §3.6
    (merge), §3.2 and §5 (the uniform 4-bit grid, for the quantization-error
    comparison), §3.3 and §4 (the paged AdamW optimizer of the adapters)
  * apxml.com, the paged-optimizer paragraph; aivaro.ru §6 (Adam's two
    moments per trained parameter, paged between GPU and CPU memory)

Precision: the quantization steps take their integer decisions (codes) in
fp32, as the kernels do; sums that set a bit-exact value (the mean of the
absmax constants) are fp64; the forward and backward matmuls are fp64.

Readings the pages leave open: the outermost
quantile probability of the NF4 construction, the tie rule at a code
midpoint (lower index), the nibble order (first element in the high
nibble), the 8-bit format of the second-level constants (OCP E4M3FN, round to
nearest even), a per-tensor mean with an fp64 pairwise-tree sum, and
x = w * fl32(1/absmax) as the normalisation. These readings are pinned only
oracle <-> GPU, not by the pages ("parity unpinned" against the pages for
the choice itself; every function is still pinned by invariants, closed
forms, library routines or brute force in tests/test_oracle_*.py).
"""

from .nf4 import (  # noqa: F401
    BLOCKSIZE,
    DQ_BLOCKSIZE,
    NF4_PRINTED,
    nf4_from_quantiles,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    e4m3fn_value_table,
    e4m3fn_encode,
    e4m3fn_decode,
    blockwise_absmax,
    nf4_codes,
    pack_nibbles,
    unpack_nibbles,
    quantize,
    pairwise_tree_sum,
    double_quant,
    dequant_absmax,
    dequantize,
    dq_bits_per_param,
)
from .linear import lora_forward, lora_backward, lora_merge, lora_forward_dropout, lora_backward_dropout  # noqa: F401
from .q4error import UNIFORM4, GRIDS, quantize_dequantize, quant_error  # noqa: F401
from .optim import adamw_step  # noqa: F401
