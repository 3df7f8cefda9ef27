// Launchers shared between the kernel files and the C-ABI layer (api.cpp).
// Every launcher takes already-validated arguments and returns a status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora_nf4.h"

namespace qlnf4 {

// Device view of a quantized weight (all pointers device memory).
struct NF4Dev {
    const uint8_t* packed;
    const float* absmax;  // no double quantization
    const uint8_t* c8;    // double quantization
    const float* scale;
    const float* mean;
    int dq;
};

int launch_quantize(const void* W, bool bf16, int64_t n, uint8_t* packed, float* absmax, hipStream_t stream);
size_t dq_workspace_bytes(int64_t n1);
int launch_double_quant(const float* absmax, int64_t n1, uint8_t* c8, float* scale, float* mean, double* ws,
                        hipStream_t stream);
int launch_dequantize(const ql_nf4_weight& w, void* out, bool bf16_out, hipStream_t stream);

// out_f[t][j] = alpha_f * sum_k P[t][k] Q[j][k]   (j < ncols_f)
// out_b[t][j] = bf16(alpha_b * same)              (j < ld_b; zero for j >= qrows)
// out_bt[j][t] = the same bf16 values transposed   (j < rows_bt)
struct SkinnyArgs {
    const uint16_t* P;
    int64_t ldp;
    const uint16_t* Q;
    int64_t ldq;
    int qrows;
    int64_t T;
    int64_t kred;
    float alpha_f;
    float* out_f;
    int64_t ld_f;
    int ncols_f;
    float alpha_b;
    uint16_t* out_b;
    int64_t ld_b;
    uint16_t* out_bt;  // optional: out_bt[j * ld_bt + t] = bf16(alpha_b * sum), j < rows_bt
    int rows_bt;
    int64_t ld_bt;
};
// part: fp32 workspace of skinny_workspace_bytes(T, kred, qrows) bytes
size_t skinny_workspace_bytes(int64_t T, int64_t kred, int qrows);
int launch_skinny(const SkinnyArgs& a, float* part, hipStream_t stream);

// dst[i][j] = src[i][j] for j < cols, 0 for cols <= j < ldd.
int launch_pad_copy(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst, int64_t ldd, hipStream_t stream);
// dst[c][r] = src[r][c] for r < R, 0 for R <= r < ldd.
int launch_transpose_pad(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst, int64_t ldd, hipStream_t stream);

// Y[t][n] = sum_k X[t][k] W'[n][k] + scale sum_j U[t][j] B[n][j] for T <= 16.
int launch_gemv(const NF4Dev& w, const uint16_t* X, int64_t T, int64_t N, int64_t K, const float* U,
                const uint16_t* B, int r, float scale, uint16_t* Y, hipStream_t stream);

// Tile / split-K plan of the dequant GEMMs for an MA x T output with a
// reduction of RED, and the fp32 workspace its split partials need.
struct GemmPlan {
    int tile;
    int splits;
};
GemmPlan plan_gemm(int64_t MA, int64_t T, int64_t RED);
size_t gemm_split_bytes(int64_t MA, int64_t T, int64_t RED);

// Forward: Y = X W'^T + Us Bsrc^T over the padded rank rp (Us [T, rp] bf16 =
// bf16(s U), zero beyond r; Bsrc [N, r_b] with row stride ld_b, 16-B rows).
int launch_gemm_fwd(const NF4Dev& w, const uint16_t* X, const uint16_t* Us, const uint16_t* Bsrc, int64_t ld_b,
                    int r_b, int rp, uint16_t* Y, int64_t T, int64_t N, int64_t K, float* split_ws,
                    hipStream_t stream);
// dX = dY W' + Gp A over the padded rank rp (Gp [T, rp] bf16, A [r, K]).
int launch_gemm_dx(const NF4Dev& w, const uint16_t* dY, const uint16_t* Gp, const uint16_t* A, int r, int rp,
                   uint16_t* dX, int64_t T, int64_t N, int64_t K, float* split_ws, hipStream_t stream);

int lora_grad_rp(int r);  // rank rounded up to 16
int64_t lora_vt_ld(int64_t T);  // row stride of the transposed [rp16, T] operands
int lora_grad_splits(int64_t T, int64_t cols);
// part[ts][j][c] = sum_{t in split ts} Vt[j][t] * M[t][c] (Vt bf16 [rp16, T])
int launch_lora_grad_partial(const uint16_t* M, int64_t ldm, int64_t cols, const uint16_t* Vt, int rp16, int64_t T,
                             int splits, float* part, hipStream_t stream);
// Vt[j][t] = bf16(U[t][j]), zero rows from r to rows
int launch_transpose_f32_bf16(const float* U, int64_t T, int r, int rows, uint16_t* Vt, hipStream_t stream);
// out[j][c] (layout_jc) or out[c][j] = (acc ? out : 0) + scale * sum_ts part[ts][j][c]
int launch_lora_grad_final(const float* part, int splits, int rp, int r, int64_t cols, float scale, bool layout_jc,
                           float* out, int accumulate, hipStream_t stream);

}  // namespace qlnf4
