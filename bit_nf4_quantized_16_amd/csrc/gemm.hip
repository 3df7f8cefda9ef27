// Matmul kernels of the frozen-base LoRA linear layer (gfx950, bf16 MFMA).
//
//   forward   H  = X W'^T + s (X A^T) B^T     apxml.com "量化 LoRA (QLoRA) 与
//                                             4 位训练": h = dequant(W_NF4)x + BAx
//   backward  dX = dY W' + G A, G = s dY B    aivaro.ru "Как работает QLoRA",
//             dA = G^T X, dB = s dY^T U       §2 (shapes of A, B) and §7 (the
//                                             4-bit weight is dequantized on
//                                             the fly in the backward)
//
// W' is never materialised in HBM: the GEMMs expand NF4 tiles into LDS
// (bf16, the compute dtype) and feed them to MFMA; the dequant-GEMV for
// decode-size T expands them straight into MFMA operand registers.
// W' is the same bf16 value as nf4_dequantize produces (contraction is off
// in this file so that a' = fl(fl(E(c8) S) + mu) rounds identically).
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "mm_common.h"

namespace qlnf4 {

// ===========================================================================
// Skinny GEMM (LoRA down-projections): out[t][j] = alpha * sum_k P[t][k] Q[j][k]
// with j < 16*NT <= 128. HBM-bound (it streams P once): the grid is 64-row
// blocks of P x KS slices of the reduction, so that at least ~512 workgroups
// are in flight; each wave owns 16 rows (MFMA 16x16x32 bf16, A operand = P
// rows, B operand = Q rows) and writes fp32 partial sums; a second kernel adds
// the KS partials in order and writes every requested output form.
// ===========================================================================
constexpr int kSkinnyRows = 64;

int skinny_splits(int64_t T, int64_t kred) {
    const int64_t blocks = ceil_div(T, kSkinnyRows);
    int64_t ks = ceil_div(512, blocks);
    const int64_t max_ks = std::max<int64_t>(1, kred / 256);
    return static_cast<int>(std::min(ks, max_ks));
}

template <int NT>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs p, int ks_count, float* __restrict__ part) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kSkinnyRows + 16 * wave;
    const int ks = blockIdx.y;
    const int64_t kw = ceil_div(ceil_div(p.kred, ks_count), 32) * 32;
    const int64_t kbeg = ks * kw;
    const int64_t kend = std::min<int64_t>(kbeg + kw, p.kred);
    f32x4 acc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool trow = (t0 + li) < p.T;
    const uint16_t* prow = p.P + std::min<int64_t>(t0 + li, p.T - 1) * p.ldp;
    auto step = [&](int64_t k) {
        const int64_t kk = k + 8 * g;
        const bool kin = kk < kend;
        uint4 av = make_uint4(0, 0, 0, 0);
        if (trow && kin) av = *reinterpret_cast<const uint4*>(prow + kk);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int j = 16 * c + li;
            uint4 bv = make_uint4(0, 0, 0, 0);
            if (j < p.qrows && kin) bv = *reinterpret_cast<const uint4*>(p.Q + j * p.ldq + kk);
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc[c], 0, 0, 0);
        }
    };
    int64_t k = kbeg;
    for (; k + 64 <= kend; k += 64) {
        step(k);
        step(k + 32);
    }
    for (; k < kend; k += 32) step(k);
    // partial [ks][t][16 NT]: D[t = 4 g + r][j = 16 c + li]
    const int64_t tl = t0 + 4 * g;
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (tl + r < p.T) part[(static_cast<int64_t>(ks) * p.T + tl + r) * (16 * NT) + 16 * c + li] = acc[c][r];
}

__global__ void skinny_reduce_kernel(SkinnyArgs p, int ks_count, int width, int64_t ncols,
                                     const float* __restrict__ part) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= p.T * ncols) return;
    const int64_t t = idx / ncols;
    const int j = static_cast<int>(idx % ncols);
    float sum = 0.0f;
    if (j < width)
        for (int k = 0; k < ks_count; ++k) sum += part[(static_cast<int64_t>(k) * p.T + t) * width + j];
    if (p.out_f && j < p.ncols_f) p.out_f[t * p.ld_f + j] = p.alpha_f * sum;
    const float vb = (j < p.qrows) ? p.alpha_b * sum : 0.0f;
    const uint16_t hb = __builtin_bit_cast(uint16_t, static_cast<__bf16>(vb));
    if (p.out_b && j < p.ld_b) p.out_b[t * p.ld_b + j] = hb;
    if (p.out_bt && j < p.rows_bt) p.out_bt[j * p.ld_bt + t] = hb;
}

size_t skinny_workspace_bytes(int64_t T, int64_t kred, int qrows) {
    const int nt = (qrows + 15) / 16;
    return static_cast<size_t>(skinny_splits(T, kred)) * T * 16 * nt * sizeof(float);
}

int launch_skinny(const SkinnyArgs& a, float* part, hipStream_t stream) {
    const int nt = (a.qrows + 15) / 16;
    if (nt < 1 || nt > 8) return set_error(QL_ERR_SHAPE, "skinny GEMM: rank %d out of range", a.qrows);
    if (part == nullptr) return set_error(QL_ERR_WORKSPACE, "skinny GEMM: workspace missing");
    const int ks = skinny_splits(a.T, a.kred);
    const dim3 grid(static_cast<uint32_t>(ceil_div(a.T, kSkinnyRows)), static_cast<uint32_t>(ks));
    switch (nt) {
#define QL_SKINNY_CASE(N_)                                                               \
    case N_:                                                                             \
        hipLaunchKernelGGL(skinny_kernel<N_>, grid, dim3(256), 0, stream, a, ks, part); \
        break;
        QL_SKINNY_CASE(1)
        QL_SKINNY_CASE(2)
        QL_SKINNY_CASE(3)
        QL_SKINNY_CASE(4)
        QL_SKINNY_CASE(5)
        QL_SKINNY_CASE(6)
        QL_SKINNY_CASE(7)
        QL_SKINNY_CASE(8)
#undef QL_SKINNY_CASE
    }
    int64_t ncols = 16 * nt;
    if (a.out_b && a.ld_b > ncols) ncols = a.ld_b;
    if (a.out_bt && a.rows_bt > ncols) ncols = a.rows_bt;
    if (a.out_f && a.ncols_f > ncols) ncols = a.ncols_f;
    hipLaunchKernelGGL(skinny_reduce_kernel, dim3(static_cast<uint32_t>(ceil_div(a.T * ncols, 256))), dim3(256), 0,
                       stream, a, ks, 16 * nt, ncols, part);
    return check_launch("lora skinny GEMM");
}

// ===========================================================================
// Small layout helpers for the adapters (bf16).
// ===========================================================================
__global__ void pad_copy_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
                                uint16_t* __restrict__ dst, int64_t ldd) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= rows * ldd) return;
    const int64_t i = idx / ldd, j = idx % ldd;
    dst[idx] = (j < cols) ? src[i * cols + j] : static_cast<uint16_t>(0);
}

int launch_pad_copy(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst, int64_t ldd, hipStream_t stream) {
    hipLaunchKernelGGL(pad_copy_kernel, dim3(static_cast<uint32_t>(ceil_div(rows * ldd, 256))), dim3(256), 0, stream,
                       src, rows, cols, dst, ldd);
    return check_launch("pad copy");
}

__global__ void transpose_pad_kernel(const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                     uint16_t* __restrict__ dst, int64_t ldd) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= C * ldd) return;
    const int64_t c = idx / ldd, r = idx % ldd;
    dst[idx] = (r < R) ? src[r * C + c] : static_cast<uint16_t>(0);
}

int launch_transpose_pad(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst, int64_t ldd, hipStream_t stream) {
    hipLaunchKernelGGL(transpose_pad_kernel, dim3(static_cast<uint32_t>(ceil_div(C * ldd, 256))), dim3(256), 0, stream,
                       src, R, C, dst, ldd);
    return check_launch("transpose pad");
}

// ===========================================================================
// Dequant-GEMV for T <= 16 (decode), one kernel. A workgroup of eight waves
// owns 16 output rows; wave w covers the w-th eighth of K. Lane (i = l%16,
// g = l/16) streams 16 bytes = 32 codes of row i per 128-wide step (all of
// the wave's code loads are issued before any math) and expands them in
// registers (the v_perm lookup) into four MFMA 16x16x32 A operands; the x
// operand (lane: token l%16, the matching 8 k) is read through L2, where all
// workgroups share it. The eight partial tiles are added in a fixed order in
// LDS, then s U B^T is added and the row is rounded to bf16.
// ===========================================================================
constexpr int kGemvRows = 16;
constexpr int kGemvWaves = 8;
constexpr int kGemvMaxSteps = 8;  // 128-wide steps per wave: K <= 8 * 8 * 128 = 8192 per pass

template <bool DQ>
__global__ __launch_bounds__(512) void gemv_kernel(NF4Dev w, const uint16_t* __restrict__ X, int64_t T, int64_t N,
                                                   int64_t K, const float* __restrict__ U,
                                                   const uint16_t* __restrict__ B, int r, float scale,
                                                   uint16_t* __restrict__ Y) {
    __shared__ float red[kGemvWaves][kGemvRows][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kGemvRows;
    const int64_t row = std::min<int64_t>(n0 + li, N - 1);
    const float mu = DQ ? *w.mean : 0.0f;
    const int64_t ksteps = ceil_div(K, 128);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const bool tok = li < T;
    const uint16_t* xrow = X + std::min<int64_t>(li, T - 1) * K;
    // passes of kGemvMaxSteps steps per wave (one pass for K <= 8192)
    for (int64_t base = 0; base < ksteps; base += kGemvWaves * kGemvMaxSteps) {
        uint4 pk[kGemvMaxSteps];
        BlockConst bc[kGemvMaxSteps];
#pragma unroll
        for (int i = 0; i < kGemvMaxSteps; ++i) {
            const int64_t st = base + wave + kGemvWaves * i;
            // clamped into the row; lanes past K are zeroed below
            const int64_t k = std::min<int64_t>(std::min<int64_t>(st, ksteps - 1) * 128 + 32 * g, K - 32);
            const int64_t e = row * K + k;
            pk[i] = *reinterpret_cast<const uint4*>(w.packed + e / 2);
            if constexpr (DQ) {
                bc[i].c8 = w.c8[e / 64];
                bc[i].s = w.scale[e / 64 / QL_DQ_BLOCKSIZE];
            } else {
                bc[i].c8 = 0;
                bc[i].s = w.absmax[e / 64];
            }
        }
#pragma unroll
        for (int i = 0; i < kGemvMaxSteps; ++i) {
            const int64_t st = base + wave + kGemvWaves * i;
            if (st >= ksteps) break;
            const int64_t k = st * 128 + 32 * g;
            const bool kin = k < K;  // K % 64 == 0: a lane's 32 codes are all in or all out
            const Lut16 L = make_lut(kin ? block_value(bc[i], DQ ? 1 : 0, mu) : 0.0f);
            const uint32_t words[4] = {pk[i].x, pk[i].y, pk[i].z, pk[i].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint4 av = dequant8_lut(words[m], L);
                const uint4 bv =
                    (tok && kin) ? *reinterpret_cast<const uint4*>(xrow + k + 8 * m) : make_uint4(0, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc, 0, 0, 0);
            }
        }
    }
    // D[n = 4 g + rr][t = li]
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) red[wave][4 * g + rr][li] = acc[rr];
    __syncthreads();
    if (tid < kGemvRows * 16) {
        const int nl = tid / 16, t = tid % 16;
        const int64_t n = n0 + nl;
        if (n < N && t < T) {
            float sum = 0.0f;
#pragma unroll
            for (int ww = 0; ww < kGemvWaves; ++ww) sum += red[ww][nl][t];
            if (r > 0) {
                float lora = 0.0f;
                for (int j = 0; j < r; ++j) lora = __builtin_fmaf(U[t * r + j], bf16_to_f32(B[n * r + j]), lora);
                sum += scale * lora;
            }
            Y[t * N + n] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(sum));
        }
    }
}

int launch_gemv(const NF4Dev& w, const uint16_t* X, int64_t T, int64_t N, int64_t K, const float* U,
                const uint16_t* B, int r, float scale, uint16_t* Y, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(ceil_div(N, kGemvRows)));
    timer_begin(QL_KERNEL_GEMV, stream);
    if (w.dq)
        hipLaunchKernelGGL(gemv_kernel<true>, grid, dim3(64 * kGemvWaves), 0, stream, w, X, T, N, K, U, B, r, scale,
                           Y);
    else
        hipLaunchKernelGGL(gemv_kernel<false>, grid, dim3(64 * kGemvWaves), 0, stream, w, X, T, N, K, U, B, r, scale,
                           Y);
    timer_end(QL_KERNEL_GEMV, stream);
    return check_launch("dequant GEMV");
}

// ===========================================================================
// LoRA weight gradients (reductions over tokens): thread = one column c of
// M (X for dA, dY for dB), RP accumulators over the rank; the token range is
// split across workgroups and the splits are added in order afterwards.
// ===========================================================================
int lora_grad_rp(int r) { return (r + 15) / 16 * 16; }

constexpr int kGradCols = 64;  // columns of M per workgroup
constexpr int kGradRows = 32;  // token rows per MFMA step
constexpr int kGradLd = kGradCols + 8;

int lora_grad_splits(int64_t T, int64_t cols) {
    const int64_t col_blocks = ceil_div(cols, kGradCols);
    int64_t s = ceil_div(512, col_blocks);  // aim for >= 512 workgroups
    const int64_t max_s = ceil_div(T, 4 * kGradRows);
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    return static_cast<int>(s);
}

typedef short v4i16_g __attribute__((ext_vector_type(4)));
typedef short v8i16_g __attribute__((ext_vector_type(8)));

// LoRA weight gradient partials with bf16 MFMA 16x16x32 (reduction over
// tokens): part[ts][j][c] = sum_{t in split ts} Vt[j][t] * M[t][c], j < 16 RT.
// A workgroup owns 64 columns of M and one token split; its four waves take
// 32-row chunks in turn. Each wave stages its chunk in a private LDS tile and
// reads the B operand (8 consecutive tokens of one column per lane) with
// ds_read_b64_tr_b16; the A operand comes from Vt [rows, T] directly. The
// four waves' sums are added in a fixed order.
template <int RT>
__global__ __launch_bounds__(256) void lora_grad_mfma_kernel(const uint16_t* __restrict__ M, int64_t ldm, int64_t C,
                                                             const uint16_t* __restrict__ Vt, int64_t ldv,
                                                             int64_t T, int64_t t_per, float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint16_t sm[4][kGradRows * kGradLd];
    __shared__ float red[4][16][kGradCols];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kGradCols;
    const int ts = blockIdx.y;
    const int64_t tb = ts * t_per;
    const int64_t te = (tb + t_per < T) ? tb + t_per : T;
    f32x4 acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rt][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint16_t* tile = sm[wave];
    auto load_chunk = [&](int64_t t, uint4 (&v)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (lane >> 3) + 8 * i;
            const int64_t c = c0 + 8 * (lane & 7);
            v[i] = (t + row < te && c < C) ? *reinterpret_cast<const uint4*>(M + (t + row) * ldm + c)
                                           : make_uint4(0, 0, 0, 0);
        }
    };
    uint4 cur[4];
    int64_t t = tb + kGradRows * wave;
    if (t < te) load_chunk(t, cur);
    for (; t < te; t += 4 * kGradRows) {
        uint4 nxt[4];
        const int64_t tn = t + 4 * kGradRows;
        if (tn < te) load_chunk(tn, nxt);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(tile + ((lane >> 3) + 8 * i) * kGradLd + 8 * (lane & 7)) = cur[i];
        // B operands: rows 8g + 0..7 of column 16 cb + li (two transposing reads)
        bf16x8_t bv[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const uint16_t* base = tile + (8 * g + (li >> 2)) * kGradLd + 16 * cb + 4 * (li & 3);
            const v4i16_g lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16_g*)(reinterpret_cast<uintptr_t>(base)));
            const v4i16_g hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16_g*)(reinterpret_cast<uintptr_t>(base + 4 * kGradLd)));
            const v8i16_g v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            bv[cb] = __builtin_bit_cast(bf16x8_t, v);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int64_t tt = t + 8 * g;
            const uint16_t* vrow = Vt + (16 * rt + li) * ldv;
            uint4 av;
            if (tt + 8 <= te) {
                av = *reinterpret_cast<const uint4*>(vrow + tt);
            } else {  // last partial chunk of the split: element by element
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = (tt + e < te) ? vrow[tt + e] : 0u;
                av = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
            }
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                acc[rt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), bv[cb], acc[rt][cb], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
    }
    // fixed-order sum of the four waves, one 16-row tile at a time
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][4 * g + r][16 * cb + li] = acc[rt][cb][r];
        __syncthreads();
        for (int e = tid; e < 16 * kGradCols; e += 256) {
            const int j = e / kGradCols, c = e % kGradCols;
            const float v = ((red[0][j][c] + red[1][j][c]) + red[2][j][c]) + red[3][j][c];
            if (c0 + c < C) part[(static_cast<int64_t>(ts) * RT * 16 + 16 * rt + j) * C + c0 + c] = v;
        }
        __syncthreads();
    }
}

int64_t lora_vt_ld(int64_t T) { return ceil_div(T, 8) * 8; }

int launch_lora_grad_partial(const uint16_t* M, int64_t ldm, int64_t cols, const uint16_t* Vt, int rp16, int64_t T,
                             int splits, float* part, hipStream_t stream) {
    const int64_t ldv = lora_vt_ld(T);
    const int64_t t_per = ceil_div(ceil_div(T, splits), 4 * kGradRows) * 4 * kGradRows;
    const dim3 grid(static_cast<uint32_t>(ceil_div(cols, kGradCols)), static_cast<uint32_t>(splits));
    timer_begin(QL_KERNEL_LORA_GRAD, stream);
    switch (rp16 / 16) {
#define QL_GRAD_CASE(R_)                                                                                        \
    case R_:                                                                                                    \
        hipLaunchKernelGGL(lora_grad_mfma_kernel<R_>, grid, dim3(256), 0, stream, M, ldm, cols, Vt, ldv, T,      \
                           t_per, part);                                                                        \
        break;
        QL_GRAD_CASE(1)
        QL_GRAD_CASE(2)
        QL_GRAD_CASE(3)
        QL_GRAD_CASE(4)
        QL_GRAD_CASE(5)
        QL_GRAD_CASE(6)
        QL_GRAD_CASE(7)
        QL_GRAD_CASE(8)
#undef QL_GRAD_CASE
        default:
            return set_error(QL_ERR_SHAPE, "LoRA gradient: rank %d out of range", rp16);
    }
    timer_end(QL_KERNEL_LORA_GRAD, stream);
    return check_launch("LoRA gradient");
}

// Vt[j][t] = bf16(U[t][j]) for j < r, 0 for r <= j < rows (fp32 [T, r] in).
__global__ void transpose_f32_bf16_kernel(const float* __restrict__ U, int64_t T, int r, int rows, int64_t ldv,
                                          uint16_t* __restrict__ Vt) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<int64_t>(rows) * T) return;
    const int64_t j = idx / T, t = idx % T;
    const float v = (j < r) ? U[t * r + j] : 0.0f;
    Vt[j * ldv + t] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

int launch_transpose_f32_bf16(const float* U, int64_t T, int r, int rows, uint16_t* Vt, hipStream_t stream) {
    hipLaunchKernelGGL(transpose_f32_bf16_kernel, dim3(static_cast<uint32_t>(ceil_div(static_cast<int64_t>(rows) * T, 256))),
                       dim3(256), 0, stream, U, T, r, rows, lora_vt_ld(T), Vt);
    return check_launch("U transpose");
}

__global__ void lora_grad_final_kernel(const float* __restrict__ part, int splits, int rp, int r, int64_t cols,
                                       float scale, int layout_jc, float* __restrict__ out, int accumulate) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<int64_t>(r) * cols) return;
    int64_t j, c;
    if (layout_jc) {
        j = idx / cols;
        c = idx % cols;
    } else {
        c = idx / r;
        j = idx % r;
    }
    float s = 0.0f;
    for (int ts = 0; ts < splits; ++ts) s += part[(static_cast<int64_t>(ts) * rp + j) * cols + c];
    const float v = scale * s;
    out[idx] = accumulate ? out[idx] + v : v;
}

int launch_lora_grad_final(const float* part, int splits, int rp, int r, int64_t cols, float scale, bool layout_jc,
                           float* out, int accumulate, hipStream_t stream) {
    hipLaunchKernelGGL(lora_grad_final_kernel, dim3(static_cast<uint32_t>(ceil_div(static_cast<int64_t>(r) * cols, 256))),
                       dim3(256), 0, stream, part, splits, rp, r, cols, scale, layout_jc ? 1 : 0, out, accumulate);
    return check_launch("LoRA gradient reduce");
}

}  // namespace qlnf4
