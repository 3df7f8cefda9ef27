/*
 * qlora_nf4.h — C ABI of the MI355X (gfx950) QLoRA frozen-base linear layer.
 *
 * The library quantizes a frozen weight to blockwise 4-bit NormalFloat (NF4)
 * with double quantization of its absmax constants, and runs the LoRA linear
 * layer on it:
 *
 *     forward   H  = X * dequant(W)^T + s * (X * A^T) * B^T,   s = alpha / r
 *     backward  G  = s * dY * B
 *               dX = dY * dequant(W) + G * A
 *               dA = G^T * X
 *               dB = s * dY^T * (X * A^T)
 *
 * Sources (web pages on QLoRA, cited by title and section):
 *   [tqpw]   tqpw.cn QLoRA notes, "Method" > "NormalFloat Quantization (NF4)"
 *            and "Double Quantization"
 *   [aivaro] aivaro.ru "Как работает QLoRA (Quantized LoRA) для training?"
 *   [apxml]  apxml.com "量化 LoRA (QLoRA) 与 4 位训练"
 *   [codex]  ai-reference-codex "QLoRA 与 PEFT 全家"
 *
 * Conventions shared by every call:
 *   - Matrices are row-major. W is [rows = N, cols = K] (out x in features,
 *     aivaro §2: W in R^{d x k}); X is [T, K]; A is [r, K]; B is [N, r];
 *     H and dY are [T, N].
 *   - bf16 values travel as uint16_t bit patterns.
 *   - Every pointer except the ql_nf4_weight descriptor itself is a device
 *     pointer. The caller owns all buffers; the library never allocates,
 *     frees or keeps a pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call is
 *     asynchronous on it; buffers must stay alive until the work completes.
 *     Calls are re-entrant; calls that share output or workspace buffers on
 *     different streams race.
 *   - Workspace buffers need no initialisation and may hold anything between
 *     calls (the arrival counters and handed-over words kept in them are
 *     tagged with a token that is new for every launch, and a launch leaves
 *     its counters clear).
 *   - Calls may be captured into a HIP graph and replayed: they issue only
 *     kernel launches (no memset or copy nodes, no host synchronisation). A
 *     replayed launch reusing its token finds its counters clear, and the
 *     launches that hand words between workgroups (the decode GEMV, the GEMM
 *     forward with U inside its launch) record a one-thread kernel before
 *     them that advances an epoch word in the workspace, which their tags mix
 *     in, so a replay never takes the previous replay's words.
 *   - Some kernels hand partial results from one workgroup to another inside
 *     a launch (device-scope stores and loads). Where a workgroup waits for
 *     another, the wait is bounded; if it runs out, the workgroup computes
 *     the result itself (the decode GEMV in the same order, same bits; the
 *     GEMM forward's tiles with plain fp32 sums, equal up to rounding). Such
 *     kernels rely on no other work writing their workspace during the
 *     launch.
 *   - Device pointers must be 16-byte aligned (QL_ERR_ALIGN otherwise).
 *   - All arguments are validated before anything is launched; on an error
 *     nothing is written. No C++ exception crosses this interface.
 *     qlora_last_error() gives a message for the calling thread.
 *   - Results are bitwise reproducible run to run (no floating-point
 *     atomics).
 *   - Environment overrides, for tuning and tests only: QLORA_NF4_GEMM_TILE
 *     (128 or 256) and QLORA_NF4_GEMM_SPLITS (split count of the 256 tile) for
 *     the T > 16 GEMMs, QLORA_NF4_PROJ_SPLITS for the rank-r projections, and
 *     QLORA_NF4_GEMV_SPIN (loads of the shared U before a decode workgroup
 *     computes U itself; 0 forces that path), QLORA_NF4_GEMM_SPIN (the same
 *     for a GEMM tile waiting on U or G; -1 forces it), QLORA_NF4_FWD_U=prepass
 *     (U, and the backward's G, in a separate launch before the GEMM) and
 *     QLORA_NF4_ADAMW_PAGING=staged (qlora_paged_adamw). Results stay within
 *     the stated tolerances under any of them.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define QL_OK 0
#define QL_ERR_NULL (-1)        /* a required pointer is NULL             */
#define QL_ERR_SHAPE (-2)       /* a size is out of range                 */
#define QL_ERR_UNSUPPORTED (-3) /* blocksize, dtype or option not offered */
#define QL_ERR_ALIGN (-4)       /* a device pointer is not 16-B aligned   */
#define QL_ERR_WORKSPACE (-5)   /* workspace missing or too small         */
#define QL_ERR_HIP (-6)         /* the HIP runtime reported an error      */

/* ---- element types ----------------------------------------------------- */
#define QL_F32 0
#define QL_BF16 1

/* First-level block size: 64 weights share one absmax constant
 * ([aivaro] §5; [tqpw] "Double Quantization": NF4 at g64). */
#define QL_NF4_BLOCKSIZE 64
/* Second-level group size: 256 absmax constants share one fp32 scale
 * ([tqpw] "Double Quantization": FP8 at g256). */
#define QL_DQ_BLOCKSIZE 256
/* Largest LoRA rank the kernels take ([aivaro] §10 uses r = 8..64). */
#define QL_MAX_RANK 128

/*
 * A quantized frozen weight. The struct itself is host memory; its pointers
 * are device pointers.
 *   packed   [ceil(rows*cols/2)] bytes: the NF4 code of element e of the
 *            row-major flattening sits in byte e/2, high nibble for even e.
 *            Code c means the c-th of the sixteen NF4 values in ascending
 *            order ([tqpw] NF4: the printed list).
 *   Without double quantization (dq_blocksize == 0):
 *     absmax [ceil(rows*cols/64)] fp32, one per block of 64 elements.
 *   With double quantization (dq_blocksize == 256):
 *     c8       [nblocks] OCP FP8 E4M3FN codes of (absmax - mean) / scale
 *     dq_scale [ceil(nblocks/256)] fp32
 *     dq_mean  [1] fp32
 */
typedef struct ql_nf4_weight {
    int64_t rows;
    int64_t cols;
    int32_t blocksize;    /* must be 64 */
    int32_t dq_blocksize; /* 256, or 0 for no double quantization */
    const uint8_t* packed;
    const float* absmax;
    const uint8_t* c8;
    const float* dq_scale;
    const float* dq_mean;
} ql_nf4_weight;

/* ---- sizes ------------------------------------------------------------- */
/* Bytes of the packed codes for rows x cols weights. */
size_t nf4_packed_bytes(int64_t rows, int64_t cols);
/* Number of first-level blocks (= absmax constants = c8 codes). */
int64_t nf4_num_blocks(int64_t rows, int64_t cols, int32_t blocksize);
/* Number of second-level groups (= dq_scale entries) for n1 constants. */
int64_t nf4_dq_num_groups(int64_t n1, int32_t dq_blocksize);

/*
 * nf4_quantize — first-level blockwise NF4 quantization ([tqpw] NF4: weights
 * are normalised to [-1, 1] per block and mapped to the nearest NF4 value;
 * [aivaro] §5: blocks of 64 weights, fp32 constants).
 *
 *   W        [rows, cols] row-major, fp32 (w_dtype QL_F32) or bf16 (QL_BF16)
 *   packed   out, nf4_packed_bytes(rows, cols) bytes
 *   absmax   out, nf4_num_blocks(rows, cols, 64) fp32
 *
 * Per block of 64 consecutive elements of the row-major flattening (the last
 * block may be shorter): a = max|w|; x = fl32(w * fl32(1/a)); code = the
 * index of the nearest NF4 value to x, the lower index on an exact tie; a
 * block with a = 0 gets code 7 (the value 0). An odd element count pads the
 * last low nibble with 7. Inputs must be finite; a block whose absmax is
 * subnormal gets unspecified codes (no crash).
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (rows or cols <= 0), QL_ERR_UNSUPPORTED
 * (blocksize != 64, unknown dtype), QL_ERR_ALIGN, QL_ERR_HIP.
 */
int nf4_quantize(const void* W, int w_dtype, int64_t rows, int64_t cols, int32_t blocksize,
                 uint8_t* packed, float* absmax, void* stream);

/*
 * nf4_double_quant — second-level quantization of the fp32 absmax constants
 * ([tqpw] "Double Quantization": FP8 at group size 256 after subtracting the
 * mean, then symmetric; [apxml]: constants go from 32 to 8 bits).
 *
 *   absmax   [n1] fp32 (from nf4_quantize)
 *   c8       out [n1] E4M3FN codes
 *   scale    out [ceil(n1/256)] fp32
 *   mean     out [1] fp32
 *   ws       workspace of nf4_double_quant_workspace(n1) bytes
 *
 * mean = fl32(S / n1), S the fp64 sum of the constants over a contiguous
 * pairwise tree (zero-padded to a power of two, neighbours added level by
 * level); d = fl32(a - mean); per group s = max|d|, scale = fl32(s / 448);
 * c8 = E4M3FN(fl32(d / scale)) rounded to nearest even with the sign kept; a
 * group with scale 0 gets codes 0x00.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (n1 <= 0), QL_ERR_UNSUPPORTED
 * (dq_blocksize != 256), QL_ERR_ALIGN, QL_ERR_WORKSPACE, QL_ERR_HIP.
 */
size_t nf4_double_quant_workspace(int64_t n1);
int nf4_double_quant(const float* absmax, int64_t n1, int32_t dq_blocksize, uint8_t* c8,
                     float* scale, float* mean, void* ws, size_t ws_bytes, void* stream);

/*
 * nf4_quantize_dq — nf4_quantize followed by nf4_double_quant of its
 * constants ([tqpw] NF4 and "Double Quantization"), in one call: the same
 * packed, absmax, c8, scale and mean bit for bit, arguments as the two calls.
 * When rows x cols is a multiple of 256 (fp32 input) or 512 (bf16) and at
 * most 2^24 (fp32) or 2^25 (bf16), it takes two launches instead of three:
 * the quantize launch also adds each workgroup's 64 (fp32) or 128 (bf16)
 * constants as one node of the mean's pairwise tree, stored in the
 * workspace, and the encoder adds the (at most 4096) nodes before it
 * encodes; the separate tree-level launch is gone. Other sizes run the two
 * calls' kernels.
 *   ws   workspace of nf4_quantize_dq_workspace(rows, cols, w_dtype) bytes
 *        (0 for invalid arguments); two calls that overlap in time must not
 *        share one.
 * Errors: those of the two calls.
 */
size_t nf4_quantize_dq_workspace(int64_t rows, int64_t cols, int w_dtype);
int nf4_quantize_dq(const void* W, int w_dtype, int64_t rows, int64_t cols, int32_t blocksize,
                    uint8_t* packed, float* absmax, int32_t dq_blocksize, uint8_t* c8, float* scale,
                    float* mean, void* ws, size_t ws_bytes, void* stream);

/*
 * nf4_dequantize — expand the quantized weight to the compute dtype ([apxml]:
 * the 4-bit weight is temporarily dequantized to bfloat16 for the matmul).
 *
 *   out   [rows, cols] row-major, bf16 (out_dtype QL_BF16) or fp32 (QL_F32)
 *
 * a' = fl32(fl32(E4M3(c8) * scale) + mean) with double quantization, else
 * a' = absmax; w' = fl32(NF4[code] * a'), then rounded to bf16 to nearest
 * even for the bf16 output.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_UNSUPPORTED, QL_ERR_ALIGN,
 * QL_ERR_HIP.
 */
int nf4_dequantize(const ql_nf4_weight* w, void* out, int out_dtype, void* stream);

/*
 * q4_quant_error — error of blockwise-absmax 4-bit quantization of a weight
 * on one of two sixteen-value grids, measured in one pass ([codex] §3.2: the
 * naive grid spaces sixteen values equally, NF4 by the normal density, and
 * NF4 distorts less; §5: its edge shrinks for non-normal weights; the page
 * gives no figures).
 *
 *   W      [rows, cols] row-major, fp32 (w_dtype QL_F32) or bf16 (QL_BF16)
 *   grid   QL_GRID_NF4 (the NF4 table) or QL_GRID_UNIFORM (fl32(-1 + 2i/15),
 *          i = 0..15)
 *   stats  device, 3 fp64: sum (w - w')^2, sum w^2, max |w - w'|
 *   ws     workspace of q4_quant_error_workspace(rows, cols, w_dtype) bytes,
 *          16-B aligned (may be NULL when that is 0)
 *
 * Per block of 64 consecutive elements (a shorter last block): a = max |w|,
 * x = fl32(w * fl32(1/a)), c = the nearest grid value with ties to the lower
 * code (for NF4 the code nf4_quantize writes), w' = fl32(T[c] * a). The sums
 * are fp64 in an order fixed by the size, so equal inputs give equal bits.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (rows or cols <= 0), QL_ERR_UNSUPPORTED
 * (blocksize != 64, dtype, grid), QL_ERR_ALIGN, QL_ERR_WORKSPACE, QL_ERR_HIP.
 */
#define QL_GRID_NF4 0
#define QL_GRID_UNIFORM 1
size_t q4_quant_error_workspace(int64_t rows, int64_t cols, int w_dtype);
int q4_quant_error(const void* W, int w_dtype, int64_t rows, int64_t cols, int32_t blocksize, int32_t grid,
                   double* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * qlora_merge — fold the trained adapter into a 16-bit copy of the base
 * weight ([codex] §3.6: after training the product of the two adapter
 * matrices is added to the base weight, so inference needs no adapter branch;
 * [aivaro] §7 step 5: adapters merged with the 4-bit model for inference;
 * [tqpw] "Introduction": the adapter weights are 16-bit, so the merged weight
 * is a 16-bit one). The quantized weight is left unchanged.
 *
 *   A    [r, K] bf16 row-major      B  [N, r] bf16 row-major
 *   out  [N, K] bf16 row-major (caller-owned, 16-B aligned):
 *        out[n][k] = bf16(fl32(w'[n][k] + scale * D[n][k])),  D = B A
 *   w' = fl32(NF4[code] * a') as in nf4_dequantize; D is accumulated in fp32
 *   (order unspecified); the sum takes one fused multiply-add in fp32 and
 *   bf16 rounding is to nearest even. With r == 0, A and B are not read and
 *   out is exactly nf4_dequantize's bf16 output.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (K % 64 != 0, N % 8 != 0, r < 0 or
 * r > QL_MAX_RANK), QL_ERR_UNSUPPORTED, QL_ERR_ALIGN, QL_ERR_HIP.
 */
int qlora_merge(const ql_nf4_weight* w, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                uint16_t* out, void* stream);

/*
 * qlora_linear_fwd — forward of the frozen-base LoRA linear layer ([apxml]:
 * h = dequant(W_NF4) x + B A x; [aivaro] §2: B in R^{d x r}, A in R^{r x k};
 * the scale s = alpha / r is the LoRA scaling factor).
 *
 *   X      [T, K] bf16        A  [r, K] bf16      B  [N, r] bf16
 *   Y      out [T, N] bf16:   Y = X W'^T + s (X A^T) B^T, fp32 accumulation
 *   U_out  optional out [T, r] fp32 = X A^T (saved for the backward), or NULL
 *   ws     workspace of qlora_linear_fwd_workspace(...) bytes (may be NULL
 *          when that size is 0)
 *
 * r == 0 (A and B may then be NULL) runs the base matmul alone. T <= 16 takes
 * the dequant-GEMV kernel: one launch, the adapter branch included (its
 * first workgroups compute U for the others; the workspace holds U's
 * partial sums and their flags, size 0 when r == 0); larger T the
 * dequant-in-LDS MFMA GEMM, after a projection launch for U or, where
 * qlora_linear_fwd_u_in_launch says so, with U computed inside its launch.
 * K must be a multiple of 64 and N a multiple of 8. Y must not alias any
 * input.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (T < 0, K % 64 != 0, N % 8 != 0, r < 0
 * or r > QL_MAX_RANK), QL_ERR_UNSUPPORTED, QL_ERR_ALIGN, QL_ERR_WORKSPACE,
 * QL_ERR_HIP. T == 0 is a no-op.
 */
size_t qlora_linear_fwd_workspace(int64_t rows, int64_t cols, int64_t T, int32_t r);
/*
 * qlora_linear_fwd_u_in_launch — 1 when qlora_linear_fwd (and _noalloc)
 * with these sizes computes U = X A^T inside the dequant GEMM launch (its
 * first workgroups, one per 16 tokens, run on CUs the GEMM's tiles leave
 * free and hand U to the tiles through words tagged for the launch in the
 * workspace), 0 when a separate projection launch precedes the GEMM or
 * T <= 16 (the decode GEMV computes U inside its own launch). It applies to
 * ranks 8 and 16 without dropout when the GEMM runs unsplit 256 x 256 tiles
 * and the projection is unsplit; QLORA_NF4_FWD_U=prepass turns it off.
 * Either way Y and U_out are the same bits (should a tile's bounded wait
 * for the words run out, it forms its U values itself: equal up to fp32
 * rounding). No errors: invalid sizes give 0.
 */
int qlora_linear_fwd_u_in_launch(int64_t rows, int64_t cols, int64_t T, int32_t r);
/*
 * qlora_linear_bwd_g_in_launch — 1 when qlora_linear_bwd with these sizes,
 * asked for dX without dropout, computes G = s dY B inside the dX GEMM
 * launch (its first workgroups, one per 16 tokens, also write G^T and U^T
 * for the gradient kernel), 0 when a separate projection launch precedes
 * the dX GEMM. The same conditions as qlora_linear_fwd_u_in_launch, for the
 * dX GEMM's plan (output K, reduction N); QLORA_NF4_FWD_U=prepass turns it
 * off. Either way dX, dA and dB are the same bits (unless a tile's bounded
 * wait for the words runs out: then equal up to fp32 rounding). No errors.
 */
int qlora_linear_bwd_g_in_launch(int64_t rows, int64_t cols, int64_t T, int32_t r);
int qlora_linear_fwd(const ql_nf4_weight* w, const uint16_t* X, int64_t T, const uint16_t* A,
                     const uint16_t* B, int32_t r, float scale, uint16_t* Y, float* U_out,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * qlora_linear_fwd_noalloc — qlora_linear_fwd without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. The call
 * allocates nothing; the kernels' scratch (what qlora_linear_fwd_workspace
 * reports for the same sizes) lives in a device array of the library of
 * QL_NOALLOC_SCRATCH_BYTES, one copy per GPU, held until the process ends.
 *
 * Arguments, layouts and results as qlora_linear_fwd (the same kernels and
 * launch plan). A call whose scratch need exceeds QL_NOALLOC_SCRATCH_BYTES
 * returns QL_ERR_WORKSPACE before anything is launched. The first call on a
 * GPU looks up that GPU's copy of the array (hipGetSymbolAddress); make it
 * outside graph capture. Every call on a GPU shares its one array: calls
 * that overlap on one GPU (other streams, other threads) race and give
 * undefined results; calls ordered on one stream, or captured in one graph
 * and replayed in order, do not. The array keeps the last call's contents;
 * nothing in it needs clearing (its counters and flags are tagged per
 * launch, as in a workspace).
 * Errors: as qlora_linear_fwd.
 */
#define QL_NOALLOC_SCRATCH_BYTES (96u << 20)
int qlora_linear_fwd_noalloc(const ql_nf4_weight* w, const uint16_t* X, int64_t T, const uint16_t* A,
                             const uint16_t* B, int32_t r, float scale, uint16_t* Y, float* U_out, void* stream);

/*
 * qlora_linear_fwd_group — qlora_linear_fwd for up to four layers that read
 * the same input X (adapters sit on every attention projection, q/k/v among
 * them, and sometimes on the MLP: [aivaro] §10), e.g. q/k/v or gate/up.
 *
 *   w[i], A[i], B[i], Y[i], U_out[i]   per layer i < nw, as qlora_linear_fwd;
 *          w, A, B, Y and U_out are host arrays of nw pointers (A and B may
 *          be NULL when r == 0, U_out NULL or U_out[i] NULL to skip U)
 *   nw     1..4 layers; all share K = w[i]->cols, r and scale
 *   ws     workspace of qlora_linear_fwd_group_workspace(rows, nw, K, T, r)
 *          bytes, rows = the nw values w[i]->rows (enough for either path
 *          below, whatever the layers' formats)
 *
 * T <= 16 runs all layers in one dequant-GEMV launch (each layer's U and
 * outputs bitwise equal to qlora_linear_fwd's). Larger T runs one dequant
 * GEMM launch over all layers' 256-row tiles, after each layer's U
 * projection, when r is a multiple of 8, the layers share the format and
 * the tile plan favours it (e.g. q/k/v at T = 1024, whose single GEMMs
 * would split their reduction): U bitwise qlora_linear_fwd's, Y the same up
 * to fp32 summation order; otherwise the layers run one after another
 * through qlora_linear_fwd on the one workspace. Each Y[i] and U_out[i]
 * must not alias an input or another output.
 * Errors: as qlora_linear_fwd, plus QL_ERR_SHAPE for nw outside 1..4 or
 * layers of different K; the workspace query returns 0 for invalid sizes.
 */
size_t qlora_linear_fwd_group_workspace(const int64_t* rows, int32_t nw, int64_t cols, int64_t T, int32_t r);
/*
 * qlora_linear_fwd_group_one_launch — 1 when qlora_linear_fwd_group with
 * these sizes (T > 16) runs one GEMM launch over all layers' row tiles
 * (given layers of one format), 0 when it runs them one after another or
 * T <= 16 (the one GEMV launch). No errors: invalid sizes give 0.
 */
int qlora_linear_fwd_group_one_launch(const int64_t* rows, int32_t nw, int64_t cols, int64_t T, int32_t r);
int qlora_linear_fwd_group(const ql_nf4_weight* const* w, int32_t nw, const uint16_t* X, int64_t T,
                           const uint16_t* const* A, const uint16_t* const* B, int32_t r, float scale,
                           uint16_t* const* Y, float* const* U_out, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * qlora_linear_fwd_dropout — the forward with dropout on the adapter input
 * ([codex] §3.4: dropout on the adapters, 0.05-0.1 for small data; [aivaro]
 * §11: lora_dropout = 0.05). Inverted dropout of the adapter branch only, the
 * random draws passed in as a keep mask:
 *
 *   keep   device, bit-packed [T, K/8] u8: element (t, 8i + j) in bit j of
 *          byte t K/8 + i, 1 = kept; 16-B aligned
 *   p      the dropout probability, 0 <= p < 1; c = fl32(1 / (1 - p))
 *   U_out  c (X * keep) A^T (fp32), the U the backward needs
 *   Y      X W'^T + s U B^T (the base sees X unmasked)
 *
 * Other arguments, layouts and errors as qlora_linear_fwd (QL_ERR_NULL for a
 * NULL keep, QL_ERR_UNSUPPORTED for p outside [0, 1)); the workspace is
 * qlora_linear_fwd_dropout_workspace(...) bytes. Every T takes the GEMM path.
 */
size_t qlora_linear_fwd_dropout_workspace(int64_t rows, int64_t cols, int64_t T, int32_t r);
int qlora_linear_fwd_dropout(const ql_nf4_weight* w, const uint16_t* X, int64_t T, const uint16_t* A,
                             const uint16_t* B, int32_t r, float scale, const uint8_t* keep, float p,
                             uint16_t* Y, float* U_out, void* ws, size_t ws_bytes, void* stream);

/*
 * qlora_linear_bwd — backward of the layer ([aivaro] §7: gradients flow
 * through the 4-bit weight, dequantized on the fly, and only the adapters
 * are updated).
 *
 *   dY       [T, N] bf16 upstream gradient
 *   U_saved  optional [T, r] fp32 = X A^T from the forward; NULL recomputes it
 *   dX       optional out [T, K] bf16 = dY W' + G A, G = s dY B
 *   dA       optional out [r, K] fp32 = G^T X
 *   dB       optional out [N, r] fp32 = s dY^T U
 *   accumulate  0: dA and dB are overwritten; 1: the gradients are added to
 *               their current contents (gradient accumulation)
 *
 * Any of dX, dA, dB may be NULL to skip it. X is needed for dA and when
 * U_saved is NULL. G runs in its own projection launch before the dX GEMM
 * or, where qlora_linear_bwd_g_in_launch says so, inside the GEMM launch
 * (also when the call is captured into a graph: the launch then records a
 * one-thread kernel that advances an epoch word in the workspace, which the
 * launch's tag mixes in). K must be a multiple of 64 and N a multiple of 8.
 * Outputs must not alias inputs.
 * Errors: as qlora_linear_fwd.
 */
size_t qlora_linear_bwd_workspace(int64_t rows, int64_t cols, int64_t T, int32_t r);
int qlora_linear_bwd(const ql_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t T,
                     const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                     const float* U_saved, uint16_t* dX, float* dA, float* dB, int accumulate,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * qlora_linear_bwd_group — qlora_linear_bwd for up to four layers that read
 * the same input X (q/k/v, or gate/up: [aivaro] §10 puts adapters on these
 * projections), whose input gradients add up ([aivaro] §7: the gradient
 * flows through each dequantized weight to X):
 *
 *   dX     optional out [T, K] bf16 = sum over layers i of dY_i W_i' + G_i A_i,
 *          G_i = s dY_i B_i, summed in fp32 and rounded to bf16 once
 *   dA[i]  optional out [r, K] fp32 = G_i^T X      (as qlora_linear_bwd)
 *   dB[i]  optional out [N_i, r] fp32 = s dY_i^T U_i
 *
 *   w, dY, A, B, U_saved, dA, dB  host arrays of nw pointers, per layer as in
 *          qlora_linear_bwd (A and B may be NULL when r == 0; U_saved, dA and
 *          dB may be NULL, or hold NULL entries, to skip them)
 *   nw     1..4 layers; all share K = w[i]->cols, r, scale and the format
 *          (all with double quantization or all without)
 *   ws     workspace of qlora_linear_bwd_group_workspace(rows, nw, K, T, r)
 *          bytes, rows = the nw values w[i]->rows
 *
 * dX runs as one dequant GEMM launch whose reduction walks the layers' rows
 * one after another (plus, when the plan splits that reduction, one pass
 * adding the fp32 partials): one launch and one rounding instead of nw, and
 * at T = 1024 the split reductions of gate and up share one partial set.
 * With nw == 1 dX is bitwise qlora_linear_bwd's. Each layer's G runs in a
 * projection launch before it; dA[i] and dB[i] are bitwise those of
 * qlora_linear_bwd for layer i. K must be a multiple of 64 and each N_i a
 * multiple of 8. Outputs must not alias inputs or one another.
 * Errors: as qlora_linear_bwd, plus QL_ERR_SHAPE for nw outside 1..4 or
 * layers of different K, QL_ERR_UNSUPPORTED for a group mixing formats; the
 * workspace query returns 0 for invalid sizes.
 */
size_t qlora_linear_bwd_group_workspace(const int64_t* rows, int32_t nw, int64_t cols, int64_t T, int32_t r);
int qlora_linear_bwd_group(const ql_nf4_weight* const* w, int32_t nw, const uint16_t* X,
                           const uint16_t* const* dY, int64_t T, const uint16_t* const* A,
                           const uint16_t* const* B, int32_t r, float scale, const float* const* U_saved,
                           uint16_t* dX, float* const* dA, float* const* dB, int accumulate, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * qlora_linear_bwd_dropout — the backward of qlora_linear_fwd_dropout with
 * the same keep mask and p ([codex] §3.4):
 *
 *   dX = dY W' + c (G A) * keep,  dA = c G^T (X * keep),  dB = s dY^T U
 *
 * with G = s dY B and U = c (X * keep) A^T (U_saved from the forward, or
 * recomputed from X and keep when NULL). dX is dY W' rounded to bf16, then
 * the kept entries get fl32(c (G A)) added and are rounded again. Other
 * arguments, layouts and errors as qlora_linear_bwd (QL_ERR_NULL for a NULL
 * keep, QL_ERR_UNSUPPORTED for p outside [0, 1)); the workspace is
 * qlora_linear_bwd_dropout_workspace(...) bytes.
 */
size_t qlora_linear_bwd_dropout_workspace(int64_t rows, int64_t cols, int64_t T, int32_t r);
int qlora_linear_bwd_dropout(const ql_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t T,
                             const uint16_t* A, const uint16_t* B, int32_t r, float scale, const uint8_t* keep,
                             float p, const float* U_saved, uint16_t* dX, float* dA, float* dB, int accumulate,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * qlora_paged_adamw — one AdamW step of the trained adapter parameters with
 * 32-bit optimizer state that lives in device memory or, paged out, in host
 * memory ([apxml], the paged-optimizer paragraph: optimizer state moves
 * between GPU memory and CPU memory when GPU memory runs short; [codex] §3.3
 * and §4: paged_adamw_32bit, learning rate 2e-4; [aivaro] §6: Adam keeps the
 * first and second moment of every trained parameter, paged out to the CPU
 * and back as needed). The pages give no update formula; this is AdamW as
 * published (bias-corrected moments, weight decay decoupled from the
 * gradient), in fp32, for step number t = step >= 1:
 *
 *   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2
 *   p = p - lr wd p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
 *
 *   param       [n] fp32, device, updated in place (e.g. every layer's A and
 *               B laid end to end)
 *   param_bf16  optional out [n] bf16, device: the updated parameters
 *               rounded to nearest even (what the layer kernels read), or NULL
 *   grad        [n] fp32, device (dA and dB from qlora_linear_bwd)
 *   exp_avg, exp_avg_sq   [n] fp32 m and v, updated in place: both device
 *               memory, or both pinned host memory (hipHostMalloc); pageable
 *               or managed memory is refused (QL_ERR_UNSUPPORTED)
 *   ws          device workspace of qlora_paged_adamw_workspace(n) bytes
 *               when the state is in host memory (unused, may be NULL, when
 *               it is in device memory)
 *   copy_stream hipStream_t for the copies of host-resident state in the
 *               staged mode below (NULL, or stream itself: on stream)
 *
 * Host-resident state is by default updated in place over the host link
 * (pinned memory is mapped into the device's address space): one kernel
 * launch on stream, as for device-resident state (ws and copy_stream are
 * not used). With the environment variable QLORA_NF4_ADAMW_PAGING=staged it
 * instead streams through ws in chunks: host-to-device copies on copy_stream,
 * updates and copies back on stream, event hand-offs both ways; the library
 * keeps a few events per device for this, and paged calls from several
 * threads are serialised while they are queued. Either way the call behaves
 * as one operation on stream: it starts after the work already queued there,
 * and work queued there afterwards (and a synchronisation of stream) sees m
 * and v updated in host memory. A one-launch call may be captured into a
 * graph. All device pointers 16-byte aligned.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (n <= 0, step < 1), QL_ERR_UNSUPPORTED
 * (state memory, beta outside [0, 1), eps or lr or weight_decay negative),
 * QL_ERR_ALIGN, QL_ERR_WORKSPACE, QL_ERR_HIP.
 */
size_t qlora_paged_adamw_workspace(int64_t n);
int qlora_paged_adamw(float* param, uint16_t* param_bf16, const float* grad, float* exp_avg, float* exp_avg_sq,
                      int64_t n, int64_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                      void* ws, size_t ws_bytes, void* stream, void* copy_stream);

/* ---- diagnostics ------------------------------------------------------- */
/* Static text for a status code. */
const char* qlora_status_string(int status);
/* Message of the last failed call on this thread ("" if none). */
const char* qlora_last_error(void);

/*
 * Kernel timers (a profiling aid). While a timer is armed for a kernel, the
 * library records a pair of HIP events on the launch stream around every
 * launch of that kernel. qlora_timer_read() waits for the recorded events and
 * returns the number of launches and their summed duration. Kernel ids are
 * the QL_KERNEL_* values. Not meant to be armed from several threads at once,
 * nor while launches are captured into a HIP graph (events recorded inside a
 * replayed graph give no elapsed times: qlora_timer_read returns QL_ERR_HIP).
 */
#define QL_KERNEL_QUANTIZE 1
#define QL_KERNEL_DQ_ENCODE 2
#define QL_KERNEL_DEQUANTIZE 3
#define QL_KERNEL_GEMV 4
#define QL_KERNEL_GEMM_FWD 5
#define QL_KERNEL_GEMM_DX 6
#define QL_KERNEL_LORA_GRAD 7
#define QL_KERNEL_MERGE 8
#define QL_KERNEL_QERROR 9
#define QL_KERNEL_KEEP_APPLY 10
#define QL_KERNEL_DX_KEEP 11
#define QL_KERNEL_ADAMW 12
#define QL_KERNEL_COUNT 13
int qlora_timer_arm(int kernel_id);
int qlora_timer_read(int kernel_id, int64_t* launches, double* total_ms);
int qlora_timer_disarm(int kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
