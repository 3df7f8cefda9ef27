// Quantization error of blockwise-absmax 4-bit quantization on a sixteen-value
// grid, NF4 or uniform, in one pass over the weight (gfx950).
//
// ai-reference-codex "QLoRA 与 PEFT 全家", §3.2: the naive 4-bit grid spaces
// its sixteen values equally, NF4 spaces them by the normal density, and NF4
// is said to distort less; §5: the edge shrinks off the normal distribution.
// The page gives no figures; this kernel measures them:
//
//   stats[0] = sum (w - w')^2,  stats[1] = sum w^2,  stats[2] = max |w - w'|
//
// with a = block absmax (64 elements), x = fl32(w * fl32(1/a)), c = the
// nearest grid value (ties to the lower code), w' = fl32(T[c] * a): the
// quantizer's own rule (the NF4 codes equal nf4_quantize's), and the uniform
// grid T[i] = fl32(-1 + 2i/15). w - w' of two fp32 values is exact in fp64;
// the sums are fp64 in a fixed order (lane, wave butterfly, workgroup, then
// one pass over the workgroup partials), so the result is reproducible.
// A wave covers eight 1 KiB segments, all loads issued before any compute.
//
// Layout as in the quantizer: 1 KiB segments, lane l holding the 16 bytes at
// offset 16 l (4 fp32 or 8 bf16 values); a 64-element block is 16 or 8
// lanes, its absmax a DPP max on the bit patterns. Compiled with
// floating-point contraction off (w' rounds as stated).
#include "common.h"
#include "internal.h"

namespace qlnf4 {

namespace {

// ---- the uniform grid and its midpoint lookup ------------------------------
constexpr float uni_value(int i) { return static_cast<float>((2.0 * i - 15.0) / 15.0); }

constexpr float uni_midpoint(int j) {
    return round_down_to_f32((static_cast<double>(uni_value(j)) + static_cast<double>(uni_value(j + 1))) * 0.5);
}

// Bucket b = floor(16 x + 16.5) covers x in [(b - 16.5)/16, (b - 15.5)/16):
// shifted half a bucket from the NF4 lookup, because the uniform grid's
// middle midpoint is exactly 0, an NF4 bucket edge. Same contract:
// code(x) = base[b] + (x > thr[b]).
constexpr LutEntry uni_lut_entry(int b) {
    const double lo = (b - 16.5) / 16.0, hi = (b - 15.5) / 16.0;
    uint32_t base = 0;
    float thr = 2.0f;
    for (int j = 0; j < 15; ++j) {
        const double m = static_cast<double>(uni_midpoint(j));
        if (m < lo) ++base;
        else if (m < hi) thr = uni_midpoint(j);
    }
    return LutEntry{thr, base};
}

constexpr bool uni_lut_is_sound() {
    for (int b = 0; b < kLutBuckets; ++b) {
        const double lo = (b - 16.5) / 16.0, hi = (b - 15.5) / 16.0;
        int inside = 0;
        for (int j = 0; j < 15; ++j) {
            const double m = static_cast<double>(uni_midpoint(j));
            if (m >= lo && m < hi) ++inside;
            const double dlo = m - lo, dhi = hi - m;
            if ((dlo > -1e-4 && dlo < 1e-4) || (dhi > -1e-4 && dhi < 1e-4)) return false;
        }
        if (inside > 1) return false;
    }
    for (int j = 0; j + 1 < 15; ++j)
        if (!(uni_midpoint(j) < uni_midpoint(j + 1))) return false;
    return uni_value(0) == -1.0f && uni_value(15) == 1.0f && uni_midpoint(7) == 0.0f;
}
static_assert(uni_lut_is_sound(), "uniform-grid midpoint lookup");

__constant__ LutEntry c_lut_nf4[kLutBuckets] = {
    lut_entry(0),  lut_entry(1),  lut_entry(2),  lut_entry(3),  lut_entry(4),  lut_entry(5),  lut_entry(6),
    lut_entry(7),  lut_entry(8),  lut_entry(9),  lut_entry(10), lut_entry(11), lut_entry(12), lut_entry(13),
    lut_entry(14), lut_entry(15), lut_entry(16), lut_entry(17), lut_entry(18), lut_entry(19), lut_entry(20),
    lut_entry(21), lut_entry(22), lut_entry(23), lut_entry(24), lut_entry(25), lut_entry(26), lut_entry(27),
    lut_entry(28), lut_entry(29), lut_entry(30), lut_entry(31), lut_entry(32),
};
__constant__ LutEntry c_lut_uni[kLutBuckets] = {
    uni_lut_entry(0),  uni_lut_entry(1),  uni_lut_entry(2),  uni_lut_entry(3),  uni_lut_entry(4),
    uni_lut_entry(5),  uni_lut_entry(6),  uni_lut_entry(7),  uni_lut_entry(8),  uni_lut_entry(9),
    uni_lut_entry(10), uni_lut_entry(11), uni_lut_entry(12), uni_lut_entry(13), uni_lut_entry(14),
    uni_lut_entry(15), uni_lut_entry(16), uni_lut_entry(17), uni_lut_entry(18), uni_lut_entry(19),
    uni_lut_entry(20), uni_lut_entry(21), uni_lut_entry(22), uni_lut_entry(23), uni_lut_entry(24),
    uni_lut_entry(25), uni_lut_entry(26), uni_lut_entry(27), uni_lut_entry(28), uni_lut_entry(29),
    uni_lut_entry(30), uni_lut_entry(31), uni_lut_entry(32),
};
__constant__ float c_grid[2][16] = {
    {kNF4Host[0], kNF4Host[1], kNF4Host[2], kNF4Host[3], kNF4Host[4], kNF4Host[5], kNF4Host[6], kNF4Host[7],
     kNF4Host[8], kNF4Host[9], kNF4Host[10], kNF4Host[11], kNF4Host[12], kNF4Host[13], kNF4Host[14], kNF4Host[15]},
    {uni_value(0), uni_value(1), uni_value(2), uni_value(3), uni_value(4), uni_value(5), uni_value(6), uni_value(7),
     uni_value(8), uni_value(9), uni_value(10), uni_value(11), uni_value(12), uni_value(13), uni_value(14),
     uni_value(15)},
};

// Code of a normalised value x: bucket b = floor(16 x + off) by one fused
// multiply-add (16 x is exact) and v_cvt_u32_f32 (clamps below 0), then one
// comparison with the bucket's midpoint.
template <int GRID>
__device__ __forceinline__ uint32_t grid_code(float x, const LutEntry* lut) {
    uint32_t b;
    asm("v_cvt_u32_f32 %0, %1" : "=v"(b) : "v"(__builtin_fmaf(x, 16.0f, GRID == QL_GRID_NF4 ? 16.0f : 16.5f)));
    const LutEntry e = lut[b];
    return e.base + (x > e.thr ? 1u : 0u);
}

struct ErrAcc {
    double sse = 0.0, ssw = 0.0, mx = 0.0;
    __device__ __forceinline__ void add(float w, float wq) {
        const double e = static_cast<double>(w) - static_cast<double>(wq);
        const double w64 = static_cast<double>(w);
        sse = __builtin_fma(e, e, sse);
        ssw = __builtin_fma(w64, w64, ssw);
        mx = __builtin_fmax(mx, __builtin_fabs(e));
    }
};

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(u), m, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(u >> 32), m, 64);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

constexpr int kErrThreads = 256;
constexpr int kErrSegsPerWave = 8;
constexpr int kErrSegBytes = 1024;

// Workgroup partial -> part[slot], part[np + slot], part[2 np + slot] (sum of
// squared errors, sum of squares, max): lane partials, a fixed butterfly per
// wave, then the waves in order.
__device__ __forceinline__ void store_partial(ErrAcc acc, double* __restrict__ part, int64_t np, int64_t slot) {
    __shared__ double red[kErrThreads / 64][3];
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
        acc.sse += shfl_xor_f64(acc.sse, m);
        acc.ssw += shfl_xor_f64(acc.ssw, m);
        acc.mx = __builtin_fmax(acc.mx, shfl_xor_f64(acc.mx, m));
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x / 64;
    if (lane == 0) {
        red[wave][0] = acc.sse;
        red[wave][1] = acc.ssw;
        red[wave][2] = acc.mx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = red[0][0], q = red[0][1], m = red[0][2];
        for (int i = 1; i < nw; ++i) {
            s += red[i][0];
            q += red[i][1];
            m = __builtin_fmax(m, red[i][2]);
        }
        part[slot] = s;
        part[np + slot] = q;
        part[2 * np + slot] = m;
    }
}

template <bool BF16, int GRID>
__global__ __launch_bounds__(kErrThreads) void q4_error_main(const uint8_t* __restrict__ W, int64_t nseg,
                                                             double* __restrict__ part, int64_t np) {
    constexpr int kPerLane = BF16 ? 8 : 4;
    __shared__ LutEntry lut[kLutBuckets];
    __shared__ float tab[16];
    if (threadIdx.x < kLutBuckets) lut[threadIdx.x] = GRID == QL_GRID_NF4 ? c_lut_nf4[threadIdx.x] : c_lut_uni[threadIdx.x];
    if (threadIdx.x < 16) tab[threadIdx.x] = c_grid[GRID][threadIdx.x];
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kErrThreads / 64) + (threadIdx.x >> 6);
    const int64_t seg0 = wave * kErrSegsPerWave;
    ErrAcc acc;
    if (seg0 < nseg) {  // wave-uniform; every wave reaches the reduction below
        const int nsegs = static_cast<int>(nseg - seg0 < kErrSegsPerWave ? nseg - seg0 : kErrSegsPerWave);
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        u32x4 v[kErrSegsPerWave];
        const u32x4* src = reinterpret_cast<const u32x4*>(W + seg0 * kErrSegBytes) + lane;
#pragma unroll
        for (int s = 0; s < kErrSegsPerWave; ++s)
            v[s] = __builtin_nontemporal_load(src + (s < nsegs ? s : nsegs - 1) * (kErrSegBytes / 16));
#pragma unroll
        for (int s = 0; s < kErrSegsPerWave; ++s) {
            if (s >= nsegs) break;
            float e[kPerLane];
            if (BF16) {
                const uint32_t w4[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e[2 * i] = __uint_as_float(w4[i] << 16);
                    e[2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
                }
            } else {
                e[0] = __uint_as_float(v[s].x);
                e[1] = __uint_as_float(v[s].y);
                e[2] = __uint_as_float(v[s].z);
                e[3] = __uint_as_float(v[s].w);
            }
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) m = fmaxf(m, fabsf(e[i]));
            const float a = __uint_as_float(BF16 ? umax8(__float_as_uint(m)) : umax16(__float_as_uint(m)));
            const float inv = a > 0.0f ? 1.0f / a : 0.0f;
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) {
                const uint32_t c = grid_code<GRID>(e[i] * inv, lut);
                acc.add(e[i], tab[c] * a);
            }
        }
    }
    store_partial(acc, part, np, blockIdx.x);
}

// Elements after the last whole segment (fewer than 512): one wave, one
// block (possibly short) per lane; its partial goes to slot `slot`.
template <bool BF16, int GRID>
__global__ __launch_bounds__(64) void q4_error_tail(const uint8_t* __restrict__ W, int64_t start, int64_t n,
                                                    double* __restrict__ part, int64_t np, int64_t slot) {
    __shared__ LutEntry lut[kLutBuckets];
    __shared__ float tab[16];
    if (threadIdx.x < kLutBuckets) lut[threadIdx.x] = GRID == QL_GRID_NF4 ? c_lut_nf4[threadIdx.x] : c_lut_uni[threadIdx.x];
    if (threadIdx.x < 16) tab[threadIdx.x] = c_grid[GRID][threadIdx.x];
    __syncthreads();
    auto load = [&](int64_t i) -> float {
        if (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(W)[i]);
        return reinterpret_cast<const float*>(W)[i];
    };
    ErrAcc acc;
    const int64_t b0 = start + static_cast<int64_t>(threadIdx.x) * 64;
    if (b0 < n) {
        const int64_t len = (n - b0) < 64 ? (n - b0) : 64;
        float m = 0.0f;
        for (int64_t i = 0; i < len; ++i) m = fmaxf(m, fabsf(load(b0 + i)));
        const float inv = m > 0.0f ? 1.0f / m : 0.0f;
        for (int64_t i = 0; i < len; ++i) {
            const float w = load(b0 + i);
            acc.add(w, tab[grid_code<GRID>(w * inv, lut)] * m);
        }
    }
    store_partial(acc, part, np, slot);
}

// One workgroup of 1024: thread i sums partials i, i + 1024, ... in order
// (coalesced), then a fixed tree over the threads.
constexpr int kFinalThreads = 1024;
__global__ __launch_bounds__(kFinalThreads) void q4_error_final(const double* __restrict__ part, int64_t nparts,
                                                                double* __restrict__ stats) {
    ErrAcc acc;
    for (int64_t i = threadIdx.x; i < nparts; i += kFinalThreads) {
        acc.sse += part[i];
        acc.ssw += part[nparts + i];
        acc.mx = __builtin_fmax(acc.mx, part[2 * nparts + i]);
    }
    __shared__ double red[kFinalThreads][3];
    red[threadIdx.x][0] = acc.sse;
    red[threadIdx.x][1] = acc.ssw;
    red[threadIdx.x][2] = acc.mx;
    __syncthreads();
    for (int h = kFinalThreads / 2; h > 0; h >>= 1) {
        if (threadIdx.x < h) {
            red[threadIdx.x][0] += red[threadIdx.x + h][0];
            red[threadIdx.x][1] += red[threadIdx.x + h][1];
            red[threadIdx.x][2] = __builtin_fmax(red[threadIdx.x][2], red[threadIdx.x + h][2]);
        }
        __syncthreads();
    }
    if (threadIdx.x < 3) stats[threadIdx.x] = red[0][threadIdx.x];
}

struct ErrPlan {
    int64_t nseg, grid, start, nparts;
};

ErrPlan err_plan(bool bf16, int64_t n) {
    ErrPlan p;
    const int64_t seg_elems = 64 * (bf16 ? 8 : 4);
    p.nseg = n / seg_elems;
    const int64_t waves = ceil_div(p.nseg, kErrSegsPerWave);
    p.grid = ceil_div(waves, kErrThreads / 64);
    p.start = p.nseg * seg_elems;
    p.nparts = p.grid + (p.start < n ? 1 : 0);
    return p;
}

template <bool BF16, int GRID>
void launch_err(const uint8_t* W, const ErrPlan& p, int64_t n, double* part, double* stats, hipStream_t stream) {
    // the library timer spans the whole call (main pass, tail, final sum)
    timer_begin(QL_KERNEL_QERROR, stream);
    if (p.grid > 0)
        hipLaunchKernelGGL((q4_error_main<BF16, GRID>), dim3(static_cast<uint32_t>(p.grid)), dim3(kErrThreads), 0,
                           stream, W, p.nseg, part, p.nparts);
    if (p.start < n)
        hipLaunchKernelGGL((q4_error_tail<BF16, GRID>), dim3(1), dim3(64), 0, stream, W, p.start, n, part, p.nparts,
                           p.grid);
    hipLaunchKernelGGL(q4_error_final, dim3(1), dim3(kFinalThreads), 0, stream, part, p.nparts, stats);
    timer_end(QL_KERNEL_QERROR, stream);
}

}  // namespace

size_t q4_error_ws_bytes(bool bf16, int64_t n) {
    return static_cast<size_t>(err_plan(bf16, n).nparts) * 3 * sizeof(double);
}

int launch_q4_error(const void* W, bool bf16, int64_t n, int grid, double* stats, void* ws, hipStream_t stream) {
    const ErrPlan p = err_plan(bf16, n);
    const uint8_t* wb = static_cast<const uint8_t*>(W);
    double* part = static_cast<double*>(ws);
    if (grid == QL_GRID_NF4) {
        if (bf16) launch_err<true, QL_GRID_NF4>(wb, p, n, part, stats, stream);
        else launch_err<false, QL_GRID_NF4>(wb, p, n, part, stats, stream);
    } else {
        if (bf16) launch_err<true, QL_GRID_UNIFORM>(wb, p, n, part, stats, stream);
        else launch_err<false, QL_GRID_UNIFORM>(wb, p, n, part, stats, stream);
    }
    return check_launch("q4_quant_error");
}

}  // namespace qlnf4
