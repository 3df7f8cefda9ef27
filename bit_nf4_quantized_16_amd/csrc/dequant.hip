// Dequantization kernel (gfx950): NF4 codes + (double-quantized) absmax ->
// bf16 or fp32 weights. apxml.com "量化 LoRA (QLoRA) 与 4 位训练": the 4-bit
// weight is temporarily dequantized to the compute dtype (bfloat16).
//
// Compiled with floating-point contraction off: a' = fl(fl(E(c8) * S) + mu)
// and w' = fl(T[c] * a') round exactly as stated (compared bit for bit).
#include "common.h"
#include "internal.h"
#include "mm_common.h"

namespace qlnf4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__constant__ float c_nf4[16] = {
    kNF4Host[0], kNF4Host[1], kNF4Host[2],  kNF4Host[3],  kNF4Host[4],  kNF4Host[5],  kNF4Host[6],  kNF4Host[7],
    kNF4Host[8], kNF4Host[9], kNF4Host[10], kNF4Host[11], kNF4Host[12], kNF4Host[13], kNF4Host[14], kNF4Host[15],
};

// The absmax constant of first-level block b.
template <bool DQ>
__device__ __forceinline__ float block_absmax(const float* __restrict__ absmax, const uint8_t* __restrict__ c8,
                                              const float* __restrict__ scale, float mu, int64_t b) {
    if (!DQ) return absmax[b];
    const float prod = e4m3_decode(c8[b]) * scale[b / QL_DQ_BLOCKSIZE];
    return prod + mu;
}

// Lane u handles elements [32 u, 32 u + 32): one 16-byte load of codes (half
// a block), 32 outputs written as four 16-byte (bf16) or eight (fp32) stores.
// A last partial unit (n not a multiple of 32) is done element by element.
template <bool DQ, bool BF16_OUT>
__global__ __launch_bounds__(256) void nf4_dequantize_kernel(const uint8_t* __restrict__ packed,
                                                             const float* __restrict__ absmax,
                                                             const uint8_t* __restrict__ c8,
                                                             const float* __restrict__ scale,
                                                             const float* __restrict__ mean, int64_t n,
                                                             void* __restrict__ out) {
    __shared__ float tab[16];
    if (threadIdx.x < 16) tab[threadIdx.x] = c_nf4[threadIdx.x];
    __syncthreads();
    const int64_t u = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t e0 = u * 32;
    if (e0 >= n) return;
    const float mu = DQ ? *mean : 0.0f;
    const float a = block_absmax<DQ>(absmax, c8, scale, mu, e0 / 64);
    if (e0 + 32 <= n) {
        const uint4 p = *reinterpret_cast<const uint4*>(packed + e0 / 2);
        const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
        float w[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t byte = (pw[i] >> (8 * j)) & 0xFFu;
                w[8 * i + 2 * j] = tab[byte >> 4] * a;
                w[8 * i + 2 * j + 1] = tab[byte & 0xFu] * a;
            }
        }
        if (BF16_OUT) {
            uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + e0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint4 r;
                r.x = pack_bf16x2(w[8 * q + 0], w[8 * q + 1]);
                r.y = pack_bf16x2(w[8 * q + 2], w[8 * q + 3]);
                r.z = pack_bf16x2(w[8 * q + 4], w[8 * q + 5]);
                r.w = pack_bf16x2(w[8 * q + 6], w[8 * q + 7]);
                o[q] = r;
            }
        } else {
            float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + e0);
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = make_float4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
        }
    } else {
        for (int64_t e = e0; e < n; ++e) {
            const uint32_t byte = packed[e / 2];
            const uint32_t c = (e & 1) ? (byte & 0xFu) : (byte >> 4);
            const float w = tab[c] * a;
            if (BF16_OUT)
                static_cast<uint16_t*>(out)[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(w));
            else
                static_cast<float*>(out)[e] = w;
        }
    }
}

// bf16 output. Lane l of a wave expands block bw + l (64 codes, two 16-byte
// loads) with the register lookup of the block's sixteen bf16 products (the
// same values as bf16(fl32(T[c] * a'))) into 128 bytes. Written directly,
// each store instruction would touch 64 lines 128 bytes apart; instead the
// wave parks its 8 KiB in LDS (row stride 144 bytes) and stores it back so
// that one instruction writes 1 KiB of consecutive bytes, as streaming
// (nontemporal) stores: the output is written once and not read back here
// (measured 8-10 % faster over a pass of 28 weights than plain stores). The
// last wave of a ragged tensor stores lane by lane, a last partial block
// element by element.
template <bool DQ>
__global__ __launch_bounds__(256) void nf4_dequantize_bf16_kernel(const uint8_t* __restrict__ packed,
                                                                  const float* __restrict__ absmax,
                                                                  const uint8_t* __restrict__ c8,
                                                                  const float* __restrict__ scale,
                                                                  const float* __restrict__ mean, int64_t n,
                                                                  uint16_t* __restrict__ out) {
    __shared__ uint4 stage[4][64 * 9];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t bw = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * 64;  // first block of the wave
    const int64_t b = bw + lane;
    const int64_t nfull = n / 64;
    if (bw * 64 >= n) return;  // wave-uniform
    const float mu = DQ ? *mean : 0.0f;
    if (bw + 64 <= nfull) {
        const float a = block_absmax<DQ>(absmax, c8, scale, mu, b);
        const uint4 p0 = *reinterpret_cast<const uint4*>(packed + b * 32);
        const uint4 p1 = *reinterpret_cast<const uint4*>(packed + b * 32 + 16);
        const Lut16 L = make_lut(a);
        uint4* sl = stage[wave] + lane * 9;
        sl[0] = dequant8_lut(p0.x, L);
        sl[1] = dequant8_lut(p0.y, L);
        sl[2] = dequant8_lut(p0.z, L);
        sl[3] = dequant8_lut(p0.w, L);
        sl[4] = dequant8_lut(p1.x, L);
        sl[5] = dequant8_lut(p1.y, L);
        sl[6] = dequant8_lut(p1.z, L);
        sl[7] = dequant8_lut(p1.w, L);
        wave_lds_sync();
        u32x4* o = reinterpret_cast<u32x4*>(out + bw * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 v = stage[wave][(8 * i + (lane >> 3)) * 9 + (lane & 7)];
            __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, o + 64 * i + lane);
        }
    } else if (b < nfull) {
        const float a = block_absmax<DQ>(absmax, c8, scale, mu, b);
        const uint4 p0 = *reinterpret_cast<const uint4*>(packed + b * 32);
        const uint4 p1 = *reinterpret_cast<const uint4*>(packed + b * 32 + 16);
        const Lut16 L = make_lut(a);
        uint4* o = reinterpret_cast<uint4*>(out + b * 64);
        o[0] = dequant8_lut(p0.x, L);
        o[1] = dequant8_lut(p0.y, L);
        o[2] = dequant8_lut(p0.z, L);
        o[3] = dequant8_lut(p0.w, L);
        o[4] = dequant8_lut(p1.x, L);
        o[5] = dequant8_lut(p1.y, L);
        o[6] = dequant8_lut(p1.z, L);
        o[7] = dequant8_lut(p1.w, L);
    } else if (b * 64 < n) {
        const float a = block_absmax<DQ>(absmax, c8, scale, mu, b);
        for (int64_t e = b * 64; e < n; ++e) {
            const uint32_t byte = packed[e / 2];
            const uint32_t c = (e & 1) ? (byte & 0xFu) : (byte >> 4);
            out[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(c_nf4[c] * a));
        }
    }
}

int launch_dequantize(const ql_nf4_weight& w, void* out, bool bf16_out, hipStream_t stream) {
    const int64_t n = w.rows * w.cols;
    const int64_t units = ceil_div(n, 32);
    const dim3 grid(static_cast<uint32_t>(ceil_div(units, 256)));
    const dim3 grid64(static_cast<uint32_t>(ceil_div(ceil_div(n, 64), 256)));  // a wave per 64 blocks
    const bool dq = w.dq_blocksize != 0;
    timer_begin(QL_KERNEL_DEQUANTIZE, stream);
    if (dq && bf16_out)
        hipLaunchKernelGGL(nf4_dequantize_bf16_kernel<true>, grid64, dim3(256), 0, stream, w.packed, w.absmax, w.c8,
                           w.dq_scale, w.dq_mean, n, static_cast<uint16_t*>(out));
    else if (dq)
        hipLaunchKernelGGL((nf4_dequantize_kernel<true, false>), grid, dim3(256), 0, stream, w.packed, w.absmax, w.c8,
                           w.dq_scale, w.dq_mean, n, out);
    else if (bf16_out)
        hipLaunchKernelGGL(nf4_dequantize_bf16_kernel<false>, grid64, dim3(256), 0, stream, w.packed, w.absmax, w.c8,
                           w.dq_scale, w.dq_mean, n, static_cast<uint16_t*>(out));
    else
        hipLaunchKernelGGL((nf4_dequantize_kernel<false, false>), grid, dim3(256), 0, stream, w.packed, w.absmax,
                           w.c8, w.dq_scale, w.dq_mean, n, out);
    timer_end(QL_KERNEL_DEQUANTIZE, stream);
    return check_launch("nf4_dequantize");
}

}  // namespace qlnf4
