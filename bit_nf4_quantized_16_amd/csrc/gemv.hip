// Dequant-GEMV of the frozen-base LoRA linear layer for decode-size T
// (gfx950, bf16 MFMA). The NF4 codes are expanded straight into MFMA operand
// registers: w' = bf16(fl32(T[c] * a')), the value nf4_dequantize produces
// (contraction is off in this file so that a' = fl(fl(E(c8) S) + mu) rounds
// identically).
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "mm_common.h"

namespace qlnf4 {

// ===========================================================================
// Dequant-GEMV for T <= 16 (decode) with the whole LoRA branch, one kernel.
// apxml.com "量化 LoRA (QLoRA) 与 4 位训练", forward pass: y = W' x + s B A x.
//
// A workgroup of eight waves owns 16 output rows n0..n0+15; wave w takes the
// 128-wide K steps w, w+8, w+16, ... In a step, lane (i = l%16, g = l/16):
//  - reads 16 bytes = 32 codes of row n0+i at k = 128 st + 32 g .. +32 and
//    expands them in registers (v_perm lookup) into four MFMA A operands;
//  - reads x of token i at the same 32 k: four B operands (16-byte loads that
//    every workgroup shares through L2);
//  - reads row i of each 16-row tile of the LoRA A at the same 32 k, the A
//    operands of U^T = A x^T on the same B operands. The k order inside one
//    MFMA is immaterial as long as both operands share it.
// Every load of a pass is issued before any arithmetic. The eight waves'
// partial tiles are added in a fixed order in LDS, then y = W'x + s U B^T is
// rounded to bf16. Every workgroup computes the same U bit for bit (same
// operands, same order); workgroup 0 stores it when the caller wants it.
// Lanes of tokens >= T carry zero x and their outputs are dropped.
// ===========================================================================
constexpr int kGemvRows = 16;
constexpr int kGemvWaves = 8;

// 128-wide steps per wave per pass: fewer when the LoRA rank needs more
// operand registers
template <int RT>
constexpr int gemv_steps() {
    return RT <= 1 ? 4 : (RT == 2 ? 2 : 1);
}

template <bool DQ, int RT>
__global__ __launch_bounds__(512) void gemv_kernel(NF4Dev w, const uint16_t* __restrict__ X, int64_t T, int64_t N,
                                                   int64_t K, const uint16_t* __restrict__ A,
                                                   const uint16_t* __restrict__ B, int r, float scale,
                                                   uint16_t* __restrict__ Y, float* __restrict__ U_out) {
    constexpr int S = gemv_steps<RT>();
    constexpr int RMAX = RT > 0 ? 16 * RT : 1;
    __shared__ float red[kGemvWaves][kGemvRows][16];
    __shared__ float ured[kGemvWaves][16][16];
    __shared__ float Us[16][RMAX];
    __shared__ uint16_t sB[kGemvRows * RMAX];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar step loop
    const int li = lane & 15, g = lane >> 4;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kGemvRows;
    const int64_t row = std::min<int64_t>(n0 + li, N - 1);
    const int64_t ksteps = ceil_div(K, 128);
    const bool tok = li < T;
    const uint16_t* xrow = X + std::min<int64_t>(li, T - 1) * K;

    // rows n0..n0+15 of B are one contiguous run of 16 r values: fetch it now,
    // park it in LDS after the main loop
    constexpr int BQ = RT > 0 ? (kGemvRows * RMAX + 511) / 512 : 0;
    uint16_t bpre[BQ > 0 ? BQ : 1];
    if constexpr (RT > 0) {
        const int64_t nb = static_cast<int64_t>(kGemvRows) * r, last = N * r - 1;
#pragma unroll
        for (int q = 0; q < BQ; ++q) {
            const int64_t idx = tid + 512 * q;
            bpre[q] = B[std::min<int64_t>(n0 * r + std::min<int64_t>(idx, nb - 1), last)];
        }
    }

    const float mu = DQ ? *w.mean : 0.0f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    f32x4 accu[RT > 0 ? RT : 1];
#pragma unroll
    for (int t = 0; t < (RT > 0 ? RT : 1); ++t) accu[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t base = 0; base < ksteps; base += kGemvWaves * S) {
        uint4 pk[S];
        BlockConst bc[S];
        uint4 xv[S][4];
        uint4 av[S][RT > 0 ? RT : 1][4];
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const int64_t st = std::min<int64_t>(base + wave + kGemvWaves * i, ksteps - 1);
            // clamped into the row; lanes past K are zeroed below
            const int64_t k = std::min<int64_t>(st * 128 + 32 * g, K - 32);
            const int64_t e = row * K + k;
            pk[i] = *reinterpret_cast<const uint4*>(w.packed + e / 2);
            if constexpr (DQ) {
                bc[i].c8 = w.c8[e / 64];
                bc[i].s = w.scale[e / 64 / QL_DQ_BLOCKSIZE];
            } else {
                bc[i].c8 = 0;
                bc[i].s = w.absmax[e / 64];
            }
            if (tok) {  // lanes of absent tokens issue no load
#pragma unroll
                for (int m = 0; m < 4; ++m) xv[i][m] = *reinterpret_cast<const uint4*>(xrow + k + 8 * m);
            } else {
#pragma unroll
                for (int m = 0; m < 4; ++m) xv[i][m] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const uint16_t* arow = A + std::min(16 * t + li, r - 1) * K;
#pragma unroll
                for (int m = 0; m < 4; ++m) av[i][t][m] = *reinterpret_cast<const uint4*>(arow + k + 8 * m);
            }
        }
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const int64_t st = base + wave + kGemvWaves * i;
            if (st >= ksteps) break;
            const bool kin = st * 128 + 32 * g < K;  // K % 64 == 0: 32 codes all in or all out
            if (st * 128 + 128 > K) {                 // the last, half step (wave-uniform)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (!kin) xv[i][m] = make_uint4(0, 0, 0, 0);
            }
            const Lut16 L = make_lut(kin ? block_value(bc[i], DQ ? 1 : 0, mu) : 0.0f);
            const uint32_t words[4] = {pk[i].x, pk[i].y, pk[i].z, pk[i].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const bf16x8_t xb = as_bf16x8(xv[i][m]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dequant8_lut(words[m], L)), xb, acc, 0, 0,
                                                              0);
#pragma unroll
                for (int t = 0; t < RT; ++t)
                    accu[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[i][t][m]), xb, accu[t], 0, 0, 0);
            }
        }
    }
    // D[4 g + rr][li]: rows n (base) or rank index j (U^T), column token li
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) red[wave][4 * g + rr][li] = acc[rr];
    const int ol = tid >> 4, ot = tid & 15;  // output (row n0 + ol, token ot) of threads < 256
    if constexpr (RT > 0) {
#pragma unroll
        for (int q = 0; q < BQ; ++q) {
            const int idx = tid + 512 * q;
            if (idx < kGemvRows * RMAX) sB[idx] = bpre[q];
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            if (t > 0) __syncthreads();
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) ured[wave][4 * g + rr][li] = accu[t][rr];
            __syncthreads();
            if (tid < 256) {
                float u = 0.0f;
#pragma unroll
                for (int ww = 0; ww < kGemvWaves; ++ww) u += ured[ww][ol][ot];
                const int j = 16 * t + ol;
                Us[ot][j] = u;
                if (U_out != nullptr && blockIdx.x == 0 && j < r && ot < T) U_out[ot * r + j] = u;
            }
        }
    }
    __syncthreads();
    if (tid < 256) {
        const int64_t n = n0 + ol;
        if (n < N && ot < T) {
            float sum = 0.0f;
#pragma unroll
            for (int ww = 0; ww < kGemvWaves; ++ww) sum += red[ww][ol][ot];
            if constexpr (RT > 0) {
                float lora = 0.0f;
                for (int j = 0; j < r; ++j) lora = __builtin_fmaf(Us[ot][j], bf16_to_f32(sB[ol * r + j]), lora);
                sum += scale * lora;
            }
            Y[ot * N + n] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(sum));
        }
    }
}

template <bool DQ>
static void launch_gemv_rt(int rt, dim3 grid, const NF4Dev& w, const uint16_t* X, int64_t T, int64_t N, int64_t K,
                           const uint16_t* A, const uint16_t* B, int r, float scale, uint16_t* Y, float* U_out,
                           hipStream_t stream) {
    const dim3 block(64 * kGemvWaves);
    switch (rt) {
        case 0:
            hipLaunchKernelGGL((gemv_kernel<DQ, 0>), grid, block, 0, stream, w, X, T, N, K, A, B, r, scale, Y, U_out);
            break;
        case 1:
            hipLaunchKernelGGL((gemv_kernel<DQ, 1>), grid, block, 0, stream, w, X, T, N, K, A, B, r, scale, Y, U_out);
            break;
        case 2:
            hipLaunchKernelGGL((gemv_kernel<DQ, 2>), grid, block, 0, stream, w, X, T, N, K, A, B, r, scale, Y, U_out);
            break;
        case 4:
            hipLaunchKernelGGL((gemv_kernel<DQ, 4>), grid, block, 0, stream, w, X, T, N, K, A, B, r, scale, Y, U_out);
            break;
        default:
            hipLaunchKernelGGL((gemv_kernel<DQ, 8>), grid, block, 0, stream, w, X, T, N, K, A, B, r, scale, Y, U_out);
            break;
    }
}

int launch_gemv(const NF4Dev& w, const uint16_t* X, int64_t T, int64_t N, int64_t K, const uint16_t* A,
                const uint16_t* B, int r, float scale, uint16_t* Y, float* U_out, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(ceil_div(N, kGemvRows)));
    // 16-row tiles of the rank, rounded up to 0, 1, 2, 4 or 8
    const int tiles = (r + 15) / 16;
    const int rt = tiles <= 2 ? tiles : (tiles <= 4 ? 4 : 8);
    timer_begin(QL_KERNEL_GEMV, stream);
    if (w.dq)
        launch_gemv_rt<true>(rt, grid, w, X, T, N, K, A, B, r, scale, Y, U_out, stream);
    else
        launch_gemv_rt<false>(rt, grid, w, X, T, N, K, A, B, r, scale, Y, U_out, stream);
    timer_end(QL_KERNEL_GEMV, stream);
    return check_launch("dequant GEMV");
}

}  // namespace qlnf4
