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
#include "common.h"
#include "internal.h"
#include "mm_common.h"

namespace qlnf4 {

// ===========================================================================
// Skinny GEMM (LoRA down-projections): out[t][j] = alpha * sum_k P[t][k] Q[j][k]
// with j < 16*NT <= 128. One workgroup per 16 rows of P; its four waves split
// the reduction and their partial tiles are added in a fixed order.
// MFMA 16x16x32 bf16: A operand = P rows, B operand = Q rows.
// ===========================================================================
template <int NT>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs p) {
    __shared__ float red[4][16][NT * 16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int64_t kw = ((p.kred + 127) / 128) * 32;  // per-wave share, multiple of 32
    const int64_t kbeg = wave * kw;
    const int64_t kend = (kbeg + kw < p.kred) ? kbeg + kw : p.kred;
    f32x4 acc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool trow = (t0 + li) < p.T;
    const uint16_t* prow = p.P + (t0 + li) * p.ldp;
    for (int64_t k = kbeg; k < kend; k += 32) {
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
    }
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][4 * g + r][16 * c + li] = acc[c][r];
    __syncthreads();
    const int64_t ncols_b = p.out_b ? p.ld_b : 0;
    const int64_t ncols = (ncols_b > NT * 16) ? ncols_b : NT * 16;
    for (int64_t e = threadIdx.x; e < 16 * ncols; e += 256) {
        const int tl = static_cast<int>(e / ncols);
        const int j = static_cast<int>(e % ncols);
        const int64_t t = t0 + tl;
        if (t >= p.T) continue;
        float sum = 0.0f;
        if (j < NT * 16) sum = ((red[0][tl][j] + red[1][tl][j]) + red[2][tl][j]) + red[3][tl][j];
        if (p.out_f && j < p.ncols_f) p.out_f[t * p.ld_f + j] = p.alpha_f * sum;
        if (p.out_b && j < p.ld_b) {
            const float v = (j < p.qrows) ? p.alpha_b * sum : 0.0f;
            p.out_b[t * p.ld_b + j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
        }
    }
}

int launch_skinny(const SkinnyArgs& a, hipStream_t stream) {
    const int nt = (a.qrows + 15) / 16;
    const dim3 grid(static_cast<uint32_t>(ceil_div(a.T, 16)));
    switch (nt) {
#define QL_SKINNY_CASE(N_)                                                          \
    case N_:                                                                        \
        hipLaunchKernelGGL(skinny_kernel<N_>, grid, dim3(256), 0, stream, a);      \
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
        default:
            return set_error(QL_ERR_SHAPE, "skinny GEMM: rank %d out of range", a.qrows);
    }
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
// Dequant-GEMV for T <= 16 (decode). Workgroup = 64 output rows x one
// 512-wide chunk of K; each wave owns 16 rows. Lane (i = l%16, g = l/16)
// streams 16 bytes = 32 codes of row i per 128-wide step and expands them
// straight into four MFMA A operands (the k order inside the step is
// permuted identically for the x operand, which is read from LDS).
// Partial sums per chunk go to a workspace; a second kernel adds the chunks
// in order plus the LoRA term and rounds to bf16.
// ===========================================================================
constexpr int kGemvRows = 64;
constexpr int kGemvChunk = 512;
constexpr int kGemvLd = kGemvChunk + 8;

int gemv_num_chunks(int64_t K) { return static_cast<int>(ceil_div(K, kGemvChunk)); }

__global__ __launch_bounds__(256) void gemv_kernel(NF4Dev w, const uint16_t* __restrict__ X, int64_t T, int64_t N,
                                                   int64_t K, float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint16_t sx[16 * kGemvLd];
    __shared__ float tab[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kGemvRows;
    const int chunk = blockIdx.y;
    const int64_t kc0 = static_cast<int64_t>(chunk) * kGemvChunk;
    if (tid < 16) tab[tid] = c_nf4_mm[tid];
    // x chunk [16 x 512] -> LDS, zero outside [0,T) x [0,K)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i;
        const int t = idx >> 6, c = idx & 63;
        const int64_t k = kc0 + 8 * c;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (t < T && k < K) v = *reinterpret_cast<const uint4*>(X + t * K + k);
        *reinterpret_cast<uint4*>(sx + t * kGemvLd + 8 * c) = v;
    }
    // this lane's row and its four 16-byte code loads, issued up front
    const int64_t row = n0 + 16 * wave + li;
    const float mu = w.dq ? *w.mean : 0.0f;
    uint4 pk[4];
    BlockConst bc[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int64_t k = kc0 + 128 * st + 32 * g;
        if (row < N && k < K) {
            const int64_t e = row * K + k;
            pk[st] = *reinterpret_cast<const uint4*>(w.packed + e / 2);
            bc[st] = load_block_const(w, e / 64);
        } else {
            pk[st] = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
            bc[st].c8 = 0;
            bc[st].s = 0.0f;
        }
    }
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const float a = (row < N && kc0 + 128 * st + 32 * g < K) ? block_value(bc[st], w.dq, mu) : 0.0f;
        const uint32_t words[4] = {pk[st].x, pk[st].y, pk[st].z, pk[st].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint4 av = dequant8(words[m], a, tab);
            const uint4 bv = *reinterpret_cast<const uint4*>(sx + li * kGemvLd + 128 * st + 32 * g + 8 * m);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc, 0, 0, 0);
        }
    }
    // D[n = 4 g + r][t = li]
    if (li < T) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = n0 + 16 * wave + 4 * g + r;
            if (n < N) part[(static_cast<int64_t>(chunk) * T + li) * N + n] = acc[r];
        }
    }
}

int launch_gemv(const NF4Dev& w, const uint16_t* X, int64_t T, int64_t N, int64_t K, float* part,
                hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(ceil_div(N, kGemvRows)), static_cast<uint32_t>(gemv_num_chunks(K)));
    timer_begin(QL_KERNEL_GEMV, stream);
    hipLaunchKernelGGL(gemv_kernel, grid, dim3(256), 0, stream, w, X, T, N, K, part);
    timer_end(QL_KERNEL_GEMV, stream);
    return check_launch("dequant GEMV");
}

__global__ void gemv_reduce_kernel(const float* __restrict__ part, int nchunks, int64_t T, int64_t N,
                                   const float* __restrict__ U, const uint16_t* __restrict__ B, int r, float scale,
                                   uint16_t* __restrict__ Y) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= T * N) return;
    const int64_t t = idx / N, n = idx % N;
    float sum = 0.0f;
    for (int c = 0; c < nchunks; ++c) sum += part[(static_cast<int64_t>(c) * T + t) * N + n];
    if (r > 0) {
        float lora = 0.0f;
        for (int j = 0; j < r; ++j) lora = __builtin_fmaf(U[t * r + j], bf16_to_f32(B[n * r + j]), lora);
        sum += scale * lora;
    }
    Y[idx] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(sum));
}

int launch_gemv_reduce(const float* part, int nchunks, int64_t T, int64_t N, const float* U, const uint16_t* B, int r,
                       float scale, uint16_t* Y, hipStream_t stream) {
    hipLaunchKernelGGL(gemv_reduce_kernel, dim3(static_cast<uint32_t>(ceil_div(T * N, 256))), dim3(256), 0, stream,
                       part, nchunks, T, N, U, B, r, scale, Y);
    return check_launch("GEMV reduce");
}

// ===========================================================================
// LoRA weight gradients (reductions over tokens): thread = one column c of
// M (X for dA, dY for dB), RP accumulators over the rank; the token range is
// split across workgroups and the splits are added in order afterwards.
// ===========================================================================
int lora_grad_rp(int r) {
    if (r <= 16) return 16;
    if (r <= 32) return 32;
    if (r <= 64) return 64;
    return 128;
}

int lora_grad_splits(int64_t T, int64_t cols) {
    const int64_t col_tiles = ceil_div(cols, 256);
    int64_t s = ceil_div(512, col_tiles);
    const int64_t max_s = ceil_div(T, 64);
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    return static_cast<int>(s);
}

template <int RP>
__global__ __launch_bounds__(256) void lora_grad_partial_kernel(const uint16_t* __restrict__ M, int64_t ldm,
                                                                int64_t cols, const float* __restrict__ V, int64_t ldv,
                                                                int r, int64_t T, int64_t t_per,
                                                                float* __restrict__ part) {
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int ts = blockIdx.y;
    const int64_t tb = ts * t_per;
    const int64_t te = (tb + t_per < T) ? tb + t_per : T;
    float acc[RP];
#pragma unroll
    for (int j = 0; j < RP; ++j) acc[j] = 0.0f;
    const bool cin = c < cols;
    for (int64_t t = tb; t < te; ++t) {
        const float x = cin ? bf16_to_f32(M[t * ldm + c]) : 0.0f;
        const float* v = V + t * ldv;
#pragma unroll
        for (int j = 0; j < RP; ++j)
            if (j < r) acc[j] = __builtin_fmaf(v[j], x, acc[j]);
    }
    if (cin) {
#pragma unroll
        for (int j = 0; j < RP; ++j) part[(static_cast<int64_t>(ts) * RP + j) * cols + c] = acc[j];
    }
}

int launch_lora_grad_partial(const uint16_t* M, int64_t ldm, int64_t cols, const float* V, int64_t ldv, int r,
                             int64_t T, int splits, float* part, hipStream_t stream) {
    const int64_t t_per = ceil_div(T, splits);
    const dim3 grid(static_cast<uint32_t>(ceil_div(cols, 256)), static_cast<uint32_t>(splits));
    const int rp = lora_grad_rp(r);
    timer_begin(QL_KERNEL_LORA_GRAD, stream);
    switch (rp) {
        case 16:
            hipLaunchKernelGGL(lora_grad_partial_kernel<16>, grid, dim3(256), 0, stream, M, ldm, cols, V, ldv, r, T,
                               t_per, part);
            break;
        case 32:
            hipLaunchKernelGGL(lora_grad_partial_kernel<32>, grid, dim3(256), 0, stream, M, ldm, cols, V, ldv, r, T,
                               t_per, part);
            break;
        case 64:
            hipLaunchKernelGGL(lora_grad_partial_kernel<64>, grid, dim3(256), 0, stream, M, ldm, cols, V, ldv, r, T,
                               t_per, part);
            break;
        default:
            hipLaunchKernelGGL(lora_grad_partial_kernel<128>, grid, dim3(256), 0, stream, M, ldm, cols, V, ldv, r, T,
                               t_per, part);
            break;
    }
    timer_end(QL_KERNEL_LORA_GRAD, stream);
    return check_launch("LoRA gradient");
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
