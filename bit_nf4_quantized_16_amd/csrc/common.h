// Shared device helpers of the gfx950 QLoRA NF4 library: the NF4 code values,
// the midpoint lookup used by the quantizer, the bf16 / FP8 E4M3FN codecs and
// sub-wave reductions. Written for CDNA4 only (64-lane waves).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora_nf4.h"

namespace qlnf4 {

// ---------------------------------------------------------------------------
// NF4 code values. The sixteen values in ascending order, as printed on the
// tqpw.cn QLoRA notes, "NormalFloat Quantization (NF4)"; code c is the c-th.
// ---------------------------------------------------------------------------
constexpr float kNF4Host[16] = {
    -1.0f,
    -0.6961928009986877f,
    -0.5250730514526367f,
    -0.39491748809814453f,
    -0.28444138169288635f,
    -0.18477343022823334f,
    -0.09105003625154495f,
    0.0f,
    0.07958029955625534f,
    0.16093020141124725f,
    0.24611230194568634f,
    0.33791524171829224f,
    0.44070982933044434f,
    0.5626170039176941f,
    0.7229568362236023f,
    1.0f,
};

// Midpoint j between codes j and j+1, rounded down to fp32. The exact
// midpoint (T_j + T_{j+1}) / 2 is an fp64 value; for an fp32 x,
// x > midpoint  <=>  x > round_down_fp32(midpoint), so the nearest-value
// search with ties to the lower code is "code = #{j : x > m_j}".
constexpr float round_down_to_f32(double v) {
    float f = static_cast<float>(v);
    if (static_cast<double>(f) > v) {
        uint32_t b = __builtin_bit_cast(uint32_t, f);
        b = (f > 0.0f) ? b - 1u : b + 1u;
        f = __builtin_bit_cast(float, b);
    }
    return f;
}

constexpr float nf4_midpoint(int j) {
    return round_down_to_f32((static_cast<double>(kNF4Host[j]) + static_cast<double>(kNF4Host[j + 1])) * 0.5);
}

// Bucketed midpoint lookup. x in [-1, 1] falls in bucket b = floor(16 x + 16)
// (33 buckets; b = 32 holds x = 1). No bucket holds more than one midpoint
// and none lies within 1e-4 of a bucket edge, so
//     code(x) = base[b] + (x > thr[b])
// holds for every x that fp32 rounding can send to bucket b. Checked below
// at compile time.
constexpr int kLutBuckets = 33;

struct LutEntry {
    float thr;     // the midpoint inside the bucket, or 2.0 if none
    uint32_t base; // number of midpoints below the bucket
};

constexpr LutEntry lut_entry(int b) {
    double lo = b / 16.0 - 1.0;
    double hi = (b + 1) / 16.0 - 1.0;
    uint32_t base = 0;
    float thr = 2.0f;
    for (int j = 0; j < 15; ++j) {
        double m = static_cast<double>(nf4_midpoint(j));
        if (m < lo) ++base;
        else if (m < hi) thr = nf4_midpoint(j);
    }
    return LutEntry{thr, base};
}

constexpr bool lut_is_sound() {
    for (int b = 0; b < kLutBuckets; ++b) {
        double lo = b / 16.0 - 1.0, hi = (b + 1) / 16.0 - 1.0;
        int inside = 0;
        for (int j = 0; j < 15; ++j) {
            double m = static_cast<double>(nf4_midpoint(j));
            if (m >= lo && m < hi) ++inside;
            double dlo = m - lo, dhi = hi - m;
            if ((dlo > -1e-4 && dlo < 1e-4) || (dhi > -1e-4 && dhi < 1e-4)) return false;
        }
        if (inside > 1) return false;
    }
    for (int j = 0; j + 1 < 15; ++j)
        if (!(nf4_midpoint(j) < nf4_midpoint(j + 1))) return false;
    return true;
}
static_assert(lut_is_sound(), "NF4 midpoint lookup: a bucket holds two midpoints or an edge is too close");

// ---------------------------------------------------------------------------
// Number formats
// ---------------------------------------------------------------------------

// bf16 (bit pattern) -> fp32, exact.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Orders a wave's LDS writes before its following LDS reads (and the reads
// before later writes) when lanes read what other lanes of the same wave
// wrote: no workgroup barrier is needed within one wave.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Two fp32 -> two bf16 packed in a u32 (lo in the low half), round to
// nearest even (v_cvt_pk_bf16_f32 on gfx950).
typedef float f32x2_cvt __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_cvt v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt));
}

// OCP FP8 E4M3FN code -> fp32 (exact). Codes 0x7F / 0xFF (NaN) never occur
// in this library's output.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    uint32_t e = (c >> 3) & 0xFu;
    uint32_t m = c & 0x7u;
    float v = (e == 0) ? static_cast<float>(m) * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -v : v;
}

// fp32 -> OCP FP8 E4M3FN, nearest value with ties to an even mantissa, the
// sign kept (a negative value that rounds to zero gives 0x80); magnitudes at
// or above 464 saturate to 448 (the library's inputs stay within 448).
__device__ __forceinline__ uint32_t e4m3_encode_rne(float y) {
    uint32_t bits = __float_as_uint(y);
    uint32_t sign = (bits >> 24) & 0x80u;
    float a = fabsf(y);
    uint32_t code;
    if (a >= 0x1p-6f) {
        uint32_t u = __float_as_uint(a);
        uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);  // round at mantissa bit 20
        uint32_t e = (r >> 23) - 120u;                // E4M3 biased exponent
        uint32_t m = (r >> 20) & 7u;
        code = (e > 15u || (e == 15u && m == 7u)) ? 0x7Eu : ((e << 3) | m);
    } else {
        // subnormal range: value = m * 2^-9, m = 8 is the smallest normal
        code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
    }
    return sign | code;
}

// ---------------------------------------------------------------------------
// Sub-wave reductions (max is exact, so the order does not matter)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over each aligned group of 16 lanes (one DPP row); every lane gets it.
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, dpp_f<0x128>(v));  // row_ror:8
    v = fmaxf(v, dpp_f<0x124>(v));  // row_ror:4
    v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
    return v;
}

// Max over each aligned group of 8 lanes; every lane gets it.
__device__ __forceinline__ float max8(float v) {
    v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0xB1>(v));
    return v;
}

// The same maxima on non-negative floats by their bit patterns (integer max
// orders non-negative floats like float max and needs no NaN canonicalising,
// so each step is one v_max_u32 with a DPP source).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t umax_(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umax16(uint32_t v) {
    v = umax_(v, dpp_u<0x128>(v));
    v = umax_(v, dpp_u<0x124>(v));
    v = umax_(v, dpp_u<0x4E>(v));
    v = umax_(v, dpp_u<0xB1>(v));
    return v;
}
__device__ __forceinline__ uint32_t umax8(uint32_t v) {
    v = umax_(v, dpp_u<0x141>(v));
    v = umax_(v, dpp_u<0x4E>(v));
    v = umax_(v, dpp_u<0xB1>(v));
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// ---------------------------------------------------------------------------
// Host side: status, messages, timers
// ---------------------------------------------------------------------------
int set_error(int code, const char* fmt, ...);
int check_launch(const char* what);

void timer_begin(int kernel_id, hipStream_t stream);
void timer_end(int kernel_id, hipStream_t stream);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace qlnf4
