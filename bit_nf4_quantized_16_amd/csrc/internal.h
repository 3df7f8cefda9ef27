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
// Quantize and double quant in two launches: the quantize launch also forms
// one node of the constants' mean tree per workgroup (whole 512- /
// 256-element segments and at most 4096 nodes; otherwise the three-launch
// path), the encoder adds them.
size_t quantize_dq_workspace_bytes(bool bf16, int64_t n);
int launch_quantize_dq(const void* W, bool bf16, int64_t n, uint8_t* packed, float* absmax, uint8_t* c8,
                       float* scale, float* mean, void* ws, hipStream_t stream);
int launch_double_quant(const float* absmax, int64_t n1, uint8_t* c8, float* scale, float* mean, double* ws,
                        hipStream_t stream);
int launch_dequantize(const ql_nf4_weight& w, void* out, bool bf16_out, hipStream_t stream);

// Adapter merge: out[n][k] = bf16(fl32(w'[n][k] + scale sum_j B[n][j] A[j][k]))
// for 1 <= r <= QL_MAX_RANK, K % 64 == 0. Dynamic LDS merge_lds_bytes(r).
// LoRA dropout with a bit-packed keep mask [T, K/8] (element 8i + j in bit
// j of byte i): X_d = X * keep; dX[t][k] += fl32(c sum_j G[t][j] A[j][k]) for
// kept (t, k) (G bf16 with row stride ldg, A [r, K]).
int launch_keep_apply(const uint16_t* X, const uint8_t* keep, int64_t T, int64_t K, uint16_t* Xd, hipStream_t stream);
int launch_lora_dx_keep(const uint16_t* G, int64_t ldg, const uint16_t* A, int r, const uint8_t* keep, float c,
                        int64_t T, int64_t K, uint16_t* dX, hipStream_t stream);

// Quantization error on a 4-bit grid (QL_GRID_*): fp64 partials in ws.
size_t q4_error_ws_bytes(bool bf16, int64_t n);
int launch_q4_error(const void* W, bool bf16, int64_t n, int grid, double* stats, void* ws, hipStream_t stream);

size_t merge_lds_bytes(int r);
int launch_merge(const NF4Dev& w, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int r, float scale,
                 uint16_t* out, hipStream_t stream);

// LoRA projection V[t][j] = sum_k P[t][k] Q[j][k] (j < rq), one launch:
//   out_f[t][j]  = alpha_f V[t][j]                      (fp32, j < rq)
//   out_b[t][j]  = bf16(alpha_b V[t][j]), 0 for j >= rq  (j < ld_b)
//   out_bt[j][t] = the same bf16 values transposed       (j < rows_bt)
// Q is A-like (q_cols false: Q[j][k] at Q + j ldq + k) or B-like (q_cols
// true: Q[j][n] = B[n][j], B [kred, rq] row-major). Side job, done whatever
// proj says: Ut[j][t] = bf16(Usrc[t][j]) for j < ru, 0 for ru <= j < rows_ut.
struct ProjArgs {
    int proj;  // 0: only the side job
    const uint16_t* P;
    int64_t ldp;
    const uint16_t* Q;
    int64_t ldq;
    int rq;
    int64_t T;
    int64_t kred;  // multiple of 8
    float alpha_f;
    float* out_f;
    int64_t ld_f;
    float alpha_b;
    uint16_t* out_b;
    int ld_b;
    uint16_t* out_bt;
    int rows_bt;
    int64_t ld_bt;
    const float* Usrc;
    int ru;
    uint16_t* Ut;
    int rows_ut;
    int64_t ld_ut;
    // set by the launcher: fp32 partials and per-token-block counters when
    // the reduction is split over several workgroups, and the launch token
    float* part;
    uint64_t* cnt;
    uint64_t token;
    // optional: the raw sums v (before alpha_f / alpha_b) as tagged words
    // uword[t][j] = tag << 32 | fp32 bits, j < rq, device-scope stores (the
    // GEMM forward's tiles read them inside the same launch)
    uint64_t* uword;
    uint32_t tag;
};
// Workspace of a projection over T tokens, rank rq, reduction kred (0 when
// its reduction is not split); ws must hold that many bytes, 16-B aligned.
size_t lora_proj_ws_bytes(int64_t T, int rq, int64_t kred, bool q_cols);
// Workgroups per 16-token block of that projection (1: unsplit).
int lora_proj_splits(int64_t T, int rq, int64_t kred, bool q_cols);

// A fresh 56-bit token per launch for the counters that kernels keep in a
// workspace (a counter carrying another token counts as zero).
uint64_t next_token();
int launch_lora_proj(const ProjArgs& a, bool q_cols, void* ws, hipStream_t stream);

// dst[i][j] = src[i][j] for j < cols, 0 for cols <= j < ldd.
int launch_pad_copy(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst, int64_t ldd, hipStream_t stream);

// Y[t][n] = sum_k X[t][k] W'[n][k] + scale sum_j U[t][j] B[n][j] for T <= 16,
// U = X A^T computed first (fp32, into U_out or the workspace) when r > 0;
// ws holds gemv_ws_bytes(T, K, r) bytes, 16-B aligned.
size_t gemv_ws_bytes(int64_t T, int64_t K, int r);
int launch_gemv(const NF4Dev& w, const uint16_t* X, int64_t T, int64_t N, int64_t K, const uint16_t* A,
                const uint16_t* B, int r, float scale, uint16_t* Y, float* U_out, void* ws, hipStream_t stream);
// Up to four such weights that share X (the same K, T, rank and scale) in
// one launch; weight i uses gemv_ws_bytes(T, K, r) bytes of ws from i times
// that size on (a multiple of 256).
struct GemvCall {
    NF4Dev w;
    int64_t N;
    const uint16_t* A;
    const uint16_t* B;
    uint16_t* Y;
    float* U_out;
};
constexpr int kGemvMaxGroup = 4;
int launch_gemv_group(const GemvCall* calls, int nw, const uint16_t* X, int64_t T, int64_t K, int r, float scale,
                      void* ws, hipStream_t stream);

// Tile / split-K plan of the dequant GEMMs for an MA x T output with a
// reduction of RED, and the fp32 workspace its split partials need.
struct GemmPlan {
    int tile;
    int splits;
    double cost;  // rounds of the chip x steps per round (+ the split penalty), in 256-tile step units
};
GemmPlan plan_gemm(int64_t MA, int64_t T, int64_t RED);
size_t gemm_split_bytes(int64_t MA, int64_t T, int64_t RED);

// Forward: Y = X W'^T + Us Bsrc^T over the padded rank rp (Us [T, rp] bf16 =
// bf16(s U), zero beyond r; Bsrc [N, r_b] with row stride ld_b, 16-B rows).
int launch_gemm_fwd(const NF4Dev& w, const uint16_t* X, const uint16_t* Us, const uint16_t* Bsrc, int64_t ld_b,
                    int r_b, int rp, uint16_t* Y, int64_t T, int64_t N, int64_t K, float* split_ws,
                    hipStream_t stream);
// dX = dY W' + Gp A over the padded rank rp (Gp [T, rp] bf16, A [r, K]).
// The forward with U = X A^T computed inside the GEMM launch (its first
// workgroups; no separate projection launch): whether it applies to a
// forward without dropout (rank 8 or 16, the 256 tile, no reduction split,
// an unsplit projection; QLORA_NF4_FWD_U=prepass turns it off), and the
// workspace words it needs (U as tagged words, 8 bytes each). Launches
// being captured into a graph take the separate projection.
bool gemm_fwd_u_in_launch(int64_t N, int64_t K, int64_t T, int r);
size_t gemm_fwd_u_words(int64_t T, int r);
// The same for dX: G = s dY B computed by the dX GEMM launch's first
// workgroups (rank 8 or 16, the dX plan's unsplit 256 tile, an unsplit
// projection; QLORA_NF4_FWD_U=prepass turns it off); its workspace words are
// gemm_fwd_u_words(T, r).
bool gemm_dx_g_in_launch(int64_t N, int64_t K, int64_t T, int r);
// dX = dY W' + G A with G from projection g (its G^T and U^T outputs as the
// caller set them; out_b unused), one launch.
int launch_gemm_dx_g(const NF4Dev& w, const uint16_t* dY, const uint16_t* A, int r, uint16_t* dX, int64_t T,
                     int64_t N, int64_t K, const ProjArgs& g, uint64_t* words, hipStream_t stream);
// Y = X W'^T + s (X A^T) B^T with U_out = X A^T (optional), one launch.
int launch_gemm_fwd_u(const NF4Dev& w, const uint16_t* X, const uint16_t* A, const uint16_t* B, int r, float scale,
                      uint16_t* Y, float* U_out, int64_t T, int64_t N, int64_t K, uint64_t* words, hipStream_t stream);
int launch_gemm_dx(const NF4Dev& w, const uint16_t* dY, const uint16_t* Gp, const uint16_t* A, int r, int rp,
                   uint16_t* dX, int64_t T, int64_t N, int64_t K, float* split_ws, hipStream_t stream);
// dX = sum over ng layers that read the same X of dY_L W_L' + G_L A_L, one
// GEMM launch (+ the split reduce): the layers' rows are one reduction of
// gemm_group_steps(N, ng) 64-row steps, planned as plan_gemm(K, T, 64 x
// steps) plans one layer's. Every layer has the same format (double
// quantization or not), rank r and padded rank rp.
constexpr int kGemmMaxGroup = 4;
// One layer of a grouped launch. dX: its weight, dY [T, N] (act, row stride
// N), G [T, rp] bf16 (lt) and A [r, K] (la, row stride K). Forward: its
// weight, bf16(s U) [T, rp] (lt), B [N, r] (la, row stride r; r % 8 == 0)
// and Y [T, N] (out).
struct GemmLayer {
    NF4Dev w;
    const uint16_t* act;
    int64_t N;
    const uint16_t* lt;
    const uint16_t* la;
    uint16_t* out;
};
int64_t gemm_group_steps(const int64_t* N, int ng);
int launch_gemm_dx_group(const GemmLayer* layers, int ng, int r, int rp, uint16_t* dX, int64_t T, int64_t K,
                         float* split_ws, hipStream_t stream);
// Y_i = X W_i'^T + Us_i B_i^T for ng layers that read the same X, one GEMM
// launch over all layers' row tiles (+ one reduce pass when the plan splits
// the reduction): whether that is planned to beat the layers' own launches
// (the 256 tile, by plan_gemm's cost of rounds x steps), and the fp32 split
// workspace it needs.
bool gemm_fwd_group_pays(const int64_t* N, int ng, int64_t T, int64_t K);
size_t gemm_fwd_group_split_bytes(const int64_t* N, int ng, int64_t T, int64_t K);
int launch_gemm_fwd_group(const GemmLayer* layers, int ng, const uint16_t* X, int r, int rp, int64_t T, int64_t K,
                          float* split_ws, hipStream_t stream);

int lora_grad_rp(int r);         // rank rounded up to 16
int64_t lora_vt_ld(int64_t T);  // row stride of the transposed [rp16, T] operands

// Adapter gradients: out = (accumulate ? out : 0) + scale * Vt M, written as
// out[j][c] (layout_jc) or out[c][j], j < r, c < C; M bf16 [T, C] (row
// stride ldm), Vt bf16 [rp16, ldv]. A problem with out == NULL is skipped.
struct GradProblem {
    const uint16_t* M;
    int64_t ldm;
    int64_t C;
    const uint16_t* Vt;
    int64_t ldv;
    float* out;
    int layout_jc;
    float scale;
    float* part;  // set by the launcher
};
struct GradArgs {
    GradProblem pb[2];
    int nblk0;  // set by the launcher
    int r;
    int64_t T;
    int64_t t_per;  // set by the launcher
    int accumulate;
};
// fp32 workspace for token-split partials (0 when one split suffices);
// C0, C1: columns of the problems that will run (0 for a skipped one)
size_t lora_grads_part_bytes(int64_t T, int64_t C0, int64_t C1, int r);
int launch_lora_grads(GradArgs a, float* part, hipStream_t stream);

// AdamW step (fp32 state). paged: m and v are pinned host memory and pass
// through ws (adamw_page_ws_bytes(n) bytes of device memory) in chunks,
// copied on copy_stream (null or stream itself: everything on stream).
size_t adamw_page_ws_bytes(int64_t n);
int launch_adamw(float* p, uint16_t* p16, const float* g, float* m, float* v, int64_t n, int64_t step, float lr,
                 float b1, float b2, float eps, float wd, bool paged, float* ws, hipStream_t stream,
                 hipStream_t copy_stream);

}  // namespace qlnf4
