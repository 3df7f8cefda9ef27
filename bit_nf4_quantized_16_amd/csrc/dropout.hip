// LoRA dropout on the adapter input, with the keep mask given (gfx950).
//
// ai-reference-codex "QLoRA 与 PEFT 全家", §3.4: dropout on the adapters
// (0.05-0.1 for small data); aivaro.ru "Как работает QLoRA", §11:
// lora_dropout = 0.05. Inverted dropout of the adapter branch's input only:
//
//   U  = (X * keep) A^T / (1 - p),   H = X W'^T + s U B^T
//   dX = dY W' + (G A) * keep / (1 - p),   dA = G^T (X * keep) / (1 - p)
//
// The mask is bit-packed: row t of the [T, K] keep mask is K / 8 bytes,
// element 8i + j in bit j of byte i (1 = kept). Two kernels serve the layer
// around the unchanged projection and GEMM kernels:
//   keep_apply_kernel    X_d = X * keep (bf16, exact: entries kept or zeroed)
//   lora_dx_keep_kernel  dX <- bf16(dX + fl32(c (G A)[t][k])) where kept
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace qlnf4 {

namespace {

// 16-bit lane masks of eight elements from their eight keep bits: word q of
// the result covers elements 2q (low half) and 2q + 1 (high half).
__device__ __forceinline__ uint4 keep_lanes(uint32_t bits) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        w[q] = ((bits >> (2 * q)) & 1u ? 0x0000FFFFu : 0u) | ((bits >> (2 * q + 1)) & 1u ? 0xFFFF0000u : 0u);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Thread i: elements 8i .. 8i + 7 of the row-major [T, K] input (K % 8 == 0,
// so they share keep byte i), 16 bytes in and out.
__global__ __launch_bounds__(256) void keep_apply_kernel(const uint16_t* __restrict__ X,
                                                         const uint8_t* __restrict__ keep, int64_t n8,
                                                         uint16_t* __restrict__ Xd) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n8) return;
    const uint4 x = *reinterpret_cast<const uint4*>(X + 8 * i);
    const uint4 m = keep_lanes(keep[i]);
    *reinterpret_cast<uint4*>(Xd + 8 * i) = make_uint4(x.x & m.x, x.y & m.y, x.z & m.z, x.w & m.w);
}

// dX[t][k] += fl32(c * sum_j G[t][j] A[j][k]) for kept (t, k), rounded to
// bf16 (fp32 products and sums). A workgroup owns 32 tokens x 128 columns:
// the rank-r slices of G (as fp32) and A are staged in LDS; thread (tt, kc)
// computes tokens tt and tt + 16 at columns 8 kc .. 8 kc + 7, whose dX values
// and keep bits it loads first, so that their latency overlaps the staging.
constexpr int kKeepTT = 32, kKeepCols = 128;
constexpr int kKeepGLd = QL_MAX_RANK + 1;  // fp32 row stride of the staged G (odd: rows in different banks)

__global__ __launch_bounds__(256) void lora_dx_keep_kernel(const uint16_t* __restrict__ G, int64_t ldg,
                                                           const uint16_t* __restrict__ A, int r,
                                                           const uint8_t* __restrict__ keep, float c, int64_t T,
                                                           int64_t K, uint16_t* __restrict__ dX) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[QL_MAX_RANK * kKeepCols];
    __shared__ float sG[kKeepTT * kKeepGLd];
    const int tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kKeepTT;  // x: tokens (any T), y: column tiles
    const int64_t k0 = static_cast<int64_t>(blockIdx.y) * kKeepCols;
    const int tt = tid >> 4, kc = tid & 15;
    const int64_t k = k0 + 8 * kc;
    uint4 xin[2];
    uint32_t kbits[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t t = t0 + tt + 16 * h;
        const bool in = t < T && k < K;
        xin[h] = in ? *reinterpret_cast<const uint4*>(dX + t * K + k) : make_uint4(0, 0, 0, 0);
        kbits[h] = in ? keep[t * (K / 8) + k / 8] : 0u;
    }
    for (int q = tid; q < r * (kKeepCols / 8); q += 256) {
        const int j = q / (kKeepCols / 8), col = 8 * (q % (kKeepCols / 8));
        const int64_t k = k0 + col;
        const uint4 v = k < K ? *reinterpret_cast<const uint4*>(A + j * K + k) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(sA + j * kKeepCols + col) = v;
    }
    for (int q = tid; q < kKeepTT * r; q += 256) {
        const int tr = q / r, j = q % r;
        const int64_t t = t0 + tr;
        sG[tr * kKeepGLd + j] = t < T ? bf16_to_f32(G[t * ldg + j]) : 0.0f;
    }
    __syncthreads();

    float acc0[8], acc1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc0[e] = acc1[e] = 0.0f;
    for (int j = 0; j < r; ++j) {
        const uint4 av = *reinterpret_cast<const uint4*>(sA + j * kKeepCols + 8 * kc);
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
        const float g0 = sG[tt * kKeepGLd + j], g1 = sG[(tt + 16) * kKeepGLd + j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float lo = __uint_as_float(aw[q] << 16), hi = __uint_as_float(aw[q] & 0xFFFF0000u);
            acc0[2 * q] = __builtin_fmaf(g0, lo, acc0[2 * q]);
            acc0[2 * q + 1] = __builtin_fmaf(g0, hi, acc0[2 * q + 1]);
            acc1[2 * q] = __builtin_fmaf(g1, lo, acc1[2 * q]);
            acc1[2 * q + 1] = __builtin_fmaf(g1, hi, acc1[2 * q + 1]);
        }
    }
    if (k >= K) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t t = t0 + tt + 16 * h;
        if (t >= T) continue;
        const float* acc = h == 0 ? acc0 : acc1;
        const uint32_t bits = kbits[h];
        uint16_t* px = dX + t * K + k;
        const uint4 xv = xin[h];
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float lo = __uint_as_float(xw[q] << 16), hi = __uint_as_float(xw[q] & 0xFFFF0000u);
            if ((bits >> (2 * q)) & 1u) lo = lo + c * acc[2 * q];
            if ((bits >> (2 * q + 1)) & 1u) hi = hi + c * acc[2 * q + 1];
            o[q] = pack_bf16x2(lo, hi);
        }
        *reinterpret_cast<uint4*>(px) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

}  // namespace

int launch_keep_apply(const uint16_t* X, const uint8_t* keep, int64_t T, int64_t K, uint16_t* Xd, hipStream_t stream) {
    const int64_t n8 = T * K / 8;
    timer_begin(QL_KERNEL_KEEP_APPLY, stream);
    hipLaunchKernelGGL(keep_apply_kernel, dim3(static_cast<uint32_t>(ceil_div(n8, 256))), dim3(256), 0, stream, X,
                       keep, n8, Xd);
    timer_end(QL_KERNEL_KEEP_APPLY, stream);
    return check_launch("dropout: keep mask on the adapter input");
}

int launch_lora_dx_keep(const uint16_t* G, int64_t ldg, const uint16_t* A, int r, const uint8_t* keep, float c,
                        int64_t T, int64_t K, uint16_t* dX, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(ceil_div(T, kKeepTT)), static_cast<uint32_t>(ceil_div(K, kKeepCols)));
    timer_begin(QL_KERNEL_DX_KEEP, stream);
    hipLaunchKernelGGL(lora_dx_keep_kernel, grid, dim3(256), 0, stream, G, ldg, A, r, keep, c, T, K, dX);
    timer_end(QL_KERNEL_DX_KEEP, stream);
    return check_launch("dropout: masked adapter term of dX");
}

}  // namespace qlnf4
