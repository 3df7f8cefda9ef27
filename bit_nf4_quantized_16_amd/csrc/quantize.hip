// First- and second-level quantization kernels (gfx950).
//
// nf4_quantize: blockwise absmax + nearest NF4 code + nibble packing
//   (tqpw.cn QLoRA notes, "NormalFloat Quantization (NF4)": normalise each
//   block to [-1, 1], then quantize; aivaro.ru "Как работает QLoRA", §5:
//   blocks of 64 weights with fp32 constants).
// nf4_double_quant: mean-subtracted symmetric FP8 code of the constants at
//   group size 256 (tqpw.cn QLoRA notes, "Double Quantization").
//
// Compiled with floating-point contraction off: every step here rounds
// exactly as stated (the outputs are compared bit for bit).
#include "common.h"
#include "internal.h"

namespace qlnf4 {

__constant__ LutEntry c_lut[kLutBuckets] = {
    lut_entry(0),  lut_entry(1),  lut_entry(2),  lut_entry(3),  lut_entry(4),  lut_entry(5),  lut_entry(6),
    lut_entry(7),  lut_entry(8),  lut_entry(9),  lut_entry(10), lut_entry(11), lut_entry(12), lut_entry(13),
    lut_entry(14), lut_entry(15), lut_entry(16), lut_entry(17), lut_entry(18), lut_entry(19), lut_entry(20),
    lut_entry(21), lut_entry(22), lut_entry(23), lut_entry(24), lut_entry(25), lut_entry(26), lut_entry(27),
    lut_entry(28), lut_entry(29), lut_entry(30), lut_entry(31), lut_entry(32),
};

// Code of a normalised value x (|x| <= 1 up to rounding) from the bucket
// lookup held in LDS. b = floor(16 x + 16) is taken as one fused
// multiply-add (16 x is exact, so it rounds like 16 x + 16) and
// v_cvt_u32_f32, which clamps negative values (the x = -1 - ulp case) and
// NaN to 0; x never exceeds 1 + 2^-23, so b <= 32.
__device__ __forceinline__ uint32_t nf4_code(float x, const LutEntry* lut) {
    uint32_t b;
    asm("v_cvt_u32_f32 %0, %1" : "=v"(b) : "v"(__builtin_fmaf(x, 16.0f, 16.0f)));
    LutEntry e = lut[b];
    return e.base + (x > e.thr ? 1u : 0u);
}

// ---------------------------------------------------------------------------
// Main quantize kernel. The input is cut into 1 KiB segments; within a
// segment lane l holds the 16 bytes at offset 16 l (4 fp32 or 8 bf16 values),
// so each load instruction of a wave is one contiguous 1 KiB. A 64-element
// block is then 16 lanes (fp32) or 8 lanes (bf16), reduced with DPP on the
// bit patterns. Each wave takes kSegsPerWave = 4 consecutive segments and
// issues all their loads before any compute.
// The correctly rounded reciprocal fl32(1 / absmax) costs a dozen VALU
// instructions; instead of one per segment, lane l computes it for segment
// l % 4 of its own block row and the quad broadcasts it (DPP quad_perm), so
// a wave does one division for its four segments. The same selection gives
// each of the first four lanes of a block row one segment's absmax to store,
// so the wave writes its 16 (or 32) constants in one instruction.
// ---------------------------------------------------------------------------
constexpr int kQuantThreads = 256;
constexpr int kSegsPerWave = 4;
constexpr int kSegBytes = 1024;

// The first level of the double quantization's mean, folded into the
// quantize launch: each workgroup adds its aligned blocks' absmax values as
// one node of the fp64 pairwise tree and stores it in part[workgroup]
// (the last of its waves to finish, counted in LDS, adds the wave sums: no
// barrier holds the other waves); the encoder launch adds the nodes.
// Only up to 4096 nodes (16.8 M fp32 or 33.6 M bf16 weights): every encoder
// workgroup reads all nodes, and 11008 of them took the encoder from 12 to
// 24 us at 11008 x 4096; 16-wave workgroups (a quarter of the nodes) made
// the quantize kernel 12 % slower, more than the launch saved. Counting
// arrivals to let the last workgroup of a chunk add its nodes inside this
// launch measured far slower too: up to 64 workgroups updating one
// device-scope counter serialize on it.

struct QFold {
    double* part;
};

template <bool BF16, bool FOLD>
__global__ __launch_bounds__(kQuantThreads) void nf4_quantize_main(const uint8_t* __restrict__ W, int64_t nseg,
                                                                   uint8_t* __restrict__ packed,
                                                                   float* __restrict__ absmax, QFold fold) {
    constexpr int kThreads = kQuantThreads;
    constexpr int kPerLane = BF16 ? 8 : 4;           // elements per lane per segment
    constexpr int kLanesPerBlock = 64 / kPerLane;    // 8 or 16
    constexpr int kBlocksPerSeg = 64 / kLanesPerBlock;  // 8 or 4
    constexpr int kSegElems = 64 * kPerLane;         // 512 or 256
    static_assert(kSegsPerWave == 4, "one quad of lanes per block row serves four segments");

    __shared__ LutEntry lut[kLutBuckets];
    __shared__ int s_done;  // waves that have stored their sum (the fold)
    if (threadIdx.x < kLutBuckets) lut[threadIdx.x] = c_lut[threadIdx.x];
    if (FOLD && threadIdx.x == 0) s_done = 0;
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
    const int64_t seg0 = wave * kSegsPerWave;
    uint32_t mb[kSegsPerWave] = {0u, 0u, 0u, 0u};  // block absmax, as bits
    int nsegs = 0;  // wave-uniform
    // with the fold every wave reaches the workgroup's reduction below
    if (seg0 < nseg) {
    nsegs = static_cast<int>(nseg - seg0 < kSegsPerWave ? nseg - seg0 : kSegsPerWave);

    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 v[kSegsPerWave];
    const u32x4* src = reinterpret_cast<const u32x4*>(W + seg0 * kSegBytes) + lane;
    if (nsegs == kSegsPerWave) {
#pragma unroll
        for (int s = 0; s < kSegsPerWave; ++s) v[s] = __builtin_nontemporal_load(src + s * (kSegBytes / 16));
    } else {
        // a short last wave re-reads its last segment (in bounds, results dropped)
#pragma unroll
        for (int s = 0; s < kSegsPerWave; ++s)
            v[s] = __builtin_nontemporal_load(src + (s < nsegs ? s : nsegs - 1) * (kSegBytes / 16));
    }

    float e[kSegsPerWave][kPerLane];
#pragma unroll
    for (int s = 0; s < kSegsPerWave; ++s) {
        if (BF16) {
            const uint32_t w4[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e[s][2 * i] = __uint_as_float(w4[i] << 16);
                e[s][2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
            }
        } else {
            e[s][0] = __uint_as_float(v[s].x);
            e[s][1] = __uint_as_float(v[s].y);
            e[s][2] = __uint_as_float(v[s].z);
            e[s][3] = __uint_as_float(v[s].w);
        }
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) m = fmaxf(m, fabsf(e[s][i]));
        mb[s] = BF16 ? umax8(__float_as_uint(m)) : umax16(__float_as_uint(m));
    }

    // one reciprocal per lane: segment lane % 4 of this lane's block row
    const int sel = lane & 3;
    const uint32_t mine = sel == 0 ? mb[0] : (sel == 1 ? mb[1] : (sel == 2 ? mb[2] : mb[3]));
    const float mf = __uint_as_float(mine);
    const float minv = mf > 0.0f ? 1.0f / mf : 0.0f;
    float inv[kSegsPerWave];
    inv[0] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(minv), 0x00, 0xF, 0xF, false));  // quad lane 0
    inv[1] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(minv), 0x55, 0xF, 0xF, false));  // quad lane 1
    inv[2] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(minv), 0xAA, 0xF, 0xF, false));  // quad lane 2
    inv[3] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(minv), 0xFF, 0xF, 0xF, false));  // quad lane 3

    uint8_t* pk = packed + (seg0 * kSegElems + static_cast<int64_t>(lane) * kPerLane) / 2;
#pragma unroll
    for (int s = 0; s < kSegsPerWave; ++s) {
        if (s >= nsegs) break;
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const uint32_t c = nf4_code(e[s][i] * inv[s], lut);
            // element 2j goes to the high nibble of byte j
            const int byte = i >> 1;
            const int shift = byte * 8 + ((i & 1) ? 0 : 4);
            word |= c << shift;
        }
        if (BF16)
            *reinterpret_cast<uint32_t*>(pk + s * (kSegElems / 2)) = word;
        else
            *reinterpret_cast<uint16_t*>(pk + s * (kSegElems / 2)) = static_cast<uint16_t>(word);
    }
    // absmax of block (segment sel, row lane / kLanesPerBlock), by the first
    // four lanes of each block row
    const int row = lane / kLanesPerBlock;
    if ((lane % kLanesPerBlock) < 4 && sel < nsegs)
        absmax[seg0 * kBlocksPerSeg + sel * kBlocksPerSeg + row] = mf;
    } else if (!FOLD) {
        return;
    }
    if constexpr (FOLD) {
        // The wave's blocks are [16 wave, 16 wave + 16) (fp32) or 32 (bf16),
        // block s * kBlocksPerSeg + row of the wave in lane row `row` of
        // segment s, every lane of a row holding it. Blocks past the end
        // count as zero, as in the tree's zero padding. Rows pair up by xor
        // butterflies (both partners form the same sum), then the segments
        // as (0 + 1) + (2 + 3), then the waves the same way: a subtree of
        // the contiguous pairwise tree.
        double x[kSegsPerWave];
#pragma unroll
        for (int s = 0; s < kSegsPerWave; ++s) {
            x[s] = s < nsegs ? static_cast<double>(__uint_as_float(mb[s])) : 0.0;
#pragma unroll
            for (int d = kLanesPerBlock; d < 64; d <<= 1) x[s] = x[s] + __shfl_xor(x[s], d, 64);
        }
        const double wsum = (x[0] + x[1]) + (x[2] + x[3]);
        constexpr int kWaves = kThreads / 64;
        __shared__ double s_wave[kWaves];
        if (lane == 0) {
            s_wave[threadIdx.x >> 6] = wsum;
            // release orders the sum before the count, acquire the other
            // waves' sums before the last wave's reads (LDS, workgroup scope)
            const int arrived = __hip_atomic_fetch_add(&s_done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP) + 1;
            if (arrived == kWaves) {
                double v[kWaves];
#pragma unroll
                for (int i = 0; i < kWaves; ++i) v[i] = s_wave[i];
#pragma unroll
                for (int w = kWaves / 2; w >= 1; w >>= 1)
#pragma unroll
                    for (int i = 0; i < w; ++i) v[i] = v[2 * i] + v[2 * i + 1];
                fold.part[blockIdx.x] = v[0];
            }
        }
    }
}

// Tail: the elements after the last whole segment (fewer than 512), one
// block per lane of a single wave. Handles a short last block and an odd
// element count (pad nibble 7).
template <bool BF16>
__global__ __launch_bounds__(64) void nf4_quantize_tail(const uint8_t* __restrict__ W, int64_t start, int64_t n,
                                                        uint8_t* __restrict__ packed, float* __restrict__ absmax) {
    __shared__ LutEntry lut[kLutBuckets];
    if (threadIdx.x < kLutBuckets) lut[threadIdx.x] = c_lut[threadIdx.x];
    __syncthreads();
    const int64_t b0 = start + static_cast<int64_t>(threadIdx.x) * 64;
    if (b0 >= n) return;
    const int64_t len = (n - b0) < 64 ? (n - b0) : 64;
    auto load = [&](int64_t i) -> float {
        if (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(W)[i]);
        return reinterpret_cast<const float*>(W)[i];
    };
    float m = 0.0f;
    for (int64_t i = 0; i < len; ++i) m = fmaxf(m, fabsf(load(b0 + i)));
    const float inv = m > 0.0f ? 1.0f / m : 0.0f;
    for (int64_t i = 0; i < len; i += 2) {
        uint32_t hi = nf4_code(load(b0 + i) * inv, lut);
        uint32_t lo = (i + 1 < len) ? nf4_code(load(b0 + i + 1) * inv, lut) : 7u;
        packed[(b0 + i) / 2] = static_cast<uint8_t>((hi << 4) | lo);
    }
    absmax[b0 / 64] = m;
}

int launch_quantize(const void* W, bool bf16, int64_t n, uint8_t* packed, float* absmax, hipStream_t stream) {
    const int per_lane = bf16 ? 8 : 4;
    const int64_t seg_elems = 64 * per_lane;
    const int64_t nseg = n / seg_elems;
    const uint8_t* wb = static_cast<const uint8_t*>(W);
    timer_begin(QL_KERNEL_QUANTIZE, stream);
    if (nseg > 0) {
        const int64_t waves = ceil_div(nseg, kSegsPerWave);
        const int64_t grid = ceil_div(waves, kQuantThreads / 64);
        if (bf16)
            hipLaunchKernelGGL((nf4_quantize_main<true, false>), dim3(static_cast<uint32_t>(grid)),
                               dim3(kQuantThreads), 0, stream, wb, nseg, packed, absmax, QFold{});
        else
            hipLaunchKernelGGL((nf4_quantize_main<false, false>), dim3(static_cast<uint32_t>(grid)),
                               dim3(kQuantThreads), 0, stream, wb, nseg, packed, absmax, QFold{});
    }
    timer_end(QL_KERNEL_QUANTIZE, stream);
    const int64_t start = nseg * seg_elems;
    if (start < n) {
        if (bf16)
            hipLaunchKernelGGL(nf4_quantize_tail<true>, dim3(1), dim3(64), 0, stream, wb, start, n, packed, absmax);
        else
            hipLaunchKernelGGL(nf4_quantize_tail<false>, dim3(1), dim3(64), 0, stream, wb, start, n, packed, absmax);
    }
    return check_launch("nf4_quantize");
}

// ---------------------------------------------------------------------------
// Double quantization
// ---------------------------------------------------------------------------
constexpr int kTreeThreads = 256;
constexpr int kTreePerThread = 16;
constexpr int kTreeChunk = kTreeThreads * kTreePerThread;  // 4096

// Sum of the aligned chunk [4096 c, 4096 c + 4096) of `in` (zero beyond n)
// in the order of the contiguous pairwise fp64 tree: pairs inside each
// thread's 16 values, then xor-butterfly across lanes (lane t and t^d hold
// the same sum, so the butterfly is the tree), then the four wave sums as
// (w0 + w1) + (w2 + w3). Called by all 256 threads; every thread gets the sum.
template <bool F32_IN>
__device__ double tree_chunk_sum(const void* __restrict__ in, int64_t n, int64_t c) {
    const int64_t base = c * kTreeChunk + threadIdx.x * kTreePerThread;
    double v[kTreePerThread];
#pragma unroll
    for (int i = 0; i < kTreePerThread; ++i) {
        const int64_t idx = base + i;
        double x = 0.0;
        if (idx < n) x = F32_IN ? static_cast<double>(static_cast<const float*>(in)[idx])
                                : static_cast<const double*>(in)[idx];
        v[i] = x;
    }
#pragma unroll
    for (int w = kTreePerThread / 2; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) v[i] = v[2 * i] + v[2 * i + 1];
    double s = v[0];
    for (int d = 1; d < 64; d <<= 1) s = s + __shfl_xor(s, d, 64);
    __shared__ double ws[kTreeThreads / 64];
    if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
    __syncthreads();
    const double t = (ws[0] + ws[1]) + (ws[2] + ws[3]);
    __syncthreads();  // ws may be reused by the caller
    return t;
}

// One level of the tree: workgroup g writes the sum of chunk g. With a
// single workgroup the root is the tree sum of everything and the mean is
// written.
template <bool F32_IN>
__global__ __launch_bounds__(kTreeThreads) void dq_tree_level(const void* __restrict__ in, int64_t n,
                                                              double* __restrict__ out, float* __restrict__ mean,
                                                              int64_t n_total) {
    const double t = tree_chunk_sum<F32_IN>(in, n, blockIdx.x);
    if (threadIdx.x == 0) {
        out[blockIdx.x] = t;
        if (mean != nullptr) *mean = static_cast<float>(t / static_cast<double>(n_total));
    }
}

// Symmetric E4M3FN code of (a - mean) per group of 256 constants; one wave
// per group, four waves per workgroup, groups strided over the grid. With
// `partials` (at most 4096 sums of aligned subtrees of the tree), every
// workgroup first adds them up itself, in the tree's order, instead of a
// separate launch doing it; workgroup 0 stores the mean.
__global__ __launch_bounds__(256) void dq_encode(const float* __restrict__ absmax, int64_t n1,
                                                 const float* __restrict__ mean_p, const double* __restrict__ partials,
                                                 int64_t npart, float* __restrict__ mean_out,
                                                 uint8_t* __restrict__ c8, float* __restrict__ scale) {
    float mu;
    if (partials != nullptr) {
        const double t = tree_chunk_sum<false>(partials, npart, 0);
        mu = static_cast<float>(t / static_cast<double>(n1));
        if (blockIdx.x == 0 && threadIdx.x == 0) *mean_out = mu;
    } else {
        mu = *mean_p;
    }
    const int lane = threadIdx.x & 63;
    const int64_t groups = ceil_div(n1, static_cast<int64_t>(QL_DQ_BLOCKSIZE));
    for (int64_t g = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); g < groups;
         g += static_cast<int64_t>(gridDim.x) * 4) {  // wave-uniform
        const int64_t i0 = g * QL_DQ_BLOCKSIZE + lane * 4;
        float d[4];
        bool valid[4];
        if (i0 + 3 < n1) {
            float4 a = *reinterpret_cast<const float4*>(absmax + i0);
            d[0] = a.x - mu; d[1] = a.y - mu; d[2] = a.z - mu; d[3] = a.w - mu;
            valid[0] = valid[1] = valid[2] = valid[3] = true;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                valid[i] = (i0 + i) < n1;
                d[i] = valid[i] ? absmax[i0 + i] - mu : 0.0f;
            }
        }
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, valid[i] ? fabsf(d[i]) : 0.0f);
        m = wave_max(m);
        const float S = m / 448.0f;
        uint32_t code[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) code[i] = (S > 0.0f) ? e4m3_encode_rne(d[i] / S) : 0u;
        if (i0 + 3 < n1) {
            *reinterpret_cast<uint32_t*>(c8 + i0) = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (valid[i]) c8[i0 + i] = static_cast<uint8_t>(code[i]);
        }
        if (lane == 0) scale[g] = S;
    }
}

size_t dq_workspace_bytes(int64_t n1) {
    size_t total = 0;
    int64_t c = n1;
    do {
        c = ceil_div(c, kTreeChunk);
        total += static_cast<size_t>(c);
    } while (c > 1);
    return total * sizeof(double);
}

int launch_double_quant(const float* absmax, int64_t n1, uint8_t* c8, float* scale, float* mean, double* ws,
                        hipStream_t stream) {
    // tree levels until at most one chunk (4096) of partial sums is left;
    // the encoding kernel adds that last chunk itself (one launch fewer)
    int64_t count = n1;
    const void* in = absmax;
    bool f32 = true;
    double* out = ws;
    const double* last = nullptr;  // partials the encoder reduces, or none (mean already stored)
    timer_begin(QL_KERNEL_DQ_ENCODE, stream);  // the whole double quantization: tree levels and encoder
    while (true) {
        const int64_t grid = ceil_div(count, kTreeChunk);
        float* mean_out = (grid == 1) ? mean : nullptr;
        if (f32)
            hipLaunchKernelGGL(dq_tree_level<true>, dim3(static_cast<uint32_t>(grid)), dim3(kTreeThreads), 0, stream,
                               in, count, out, mean_out, n1);
        else
            hipLaunchKernelGGL(dq_tree_level<false>, dim3(static_cast<uint32_t>(grid)), dim3(kTreeThreads), 0,
                               stream, in, count, out, mean_out, n1);
        if (grid == 1) break;
        if (grid <= kTreeChunk) {
            last = out;
            count = grid;
            break;
        }
        in = out;
        f32 = false;
        count = grid;
        out += grid;
    }
    const int64_t groups = ceil_div(n1, QL_DQ_BLOCKSIZE);
    hipLaunchKernelGGL(dq_encode, dim3(static_cast<uint32_t>(ceil_div(groups, 4))), dim3(256), 0, stream, absmax, n1,
                       mean, last, last ? count : 0, mean, c8, scale);
    timer_end(QL_KERNEL_DQ_ENCODE, stream);
    return check_launch("nf4_double_quant");
}

namespace {

// Whether quantize + double quant can fold the tree's first level into the
// quantize launch: whole segments only (no tail launch) and at most 4096
// workgroup nodes, which every encoder workgroup adds itself.
struct FoldPlan {
    bool ok;
    int64_t nseg, nwg;
};

FoldPlan fold_plan(bool bf16, int64_t n) {
    const int per_lane = bf16 ? 8 : 4;
    const int64_t seg_elems = 64 * per_lane;
    FoldPlan f{};
    f.nseg = n / seg_elems;
    f.nwg = ceil_div(ceil_div(f.nseg, kSegsPerWave), kQuantThreads / 64);
    f.ok = f.nseg > 0 && n % seg_elems == 0 && f.nwg <= kTreeChunk;
    return f;
}

}  // namespace

size_t quantize_dq_workspace_bytes(bool bf16, int64_t n) {
    const FoldPlan f = fold_plan(bf16, n);
    if (!f.ok) return dq_workspace_bytes(ceil_div(n, 64));
    return static_cast<size_t>(f.nwg) * sizeof(double);
}

int launch_quantize_dq(const void* W, bool bf16, int64_t n, uint8_t* packed, float* absmax, uint8_t* c8,
                       float* scale, float* mean, void* ws, hipStream_t stream) {
    const FoldPlan f = fold_plan(bf16, n);
    const int64_t n1 = ceil_div(n, 64);
    if (!f.ok) {
        int s = launch_quantize(W, bf16, n, packed, absmax, stream);
        if (s != QL_OK) return s;
        return launch_double_quant(absmax, n1, c8, scale, mean, static_cast<double*>(ws), stream);
    }
    QFold q;
    q.part = static_cast<double*>(ws);
    const uint8_t* wb = static_cast<const uint8_t*>(W);
    timer_begin(QL_KERNEL_QUANTIZE, stream);
    const dim3 grid_q(static_cast<uint32_t>(f.nwg));
    if (bf16)
        hipLaunchKernelGGL((nf4_quantize_main<true, true>), grid_q, dim3(kQuantThreads), 0, stream, wb, f.nseg,
                           packed, absmax, q);
    else
        hipLaunchKernelGGL((nf4_quantize_main<false, true>), grid_q, dim3(kQuantThreads), 0, stream, wb, f.nseg,
                           packed, absmax, q);
    timer_end(QL_KERNEL_QUANTIZE, stream);
    const int64_t groups = ceil_div(n1, QL_DQ_BLOCKSIZE);
    const int64_t grid = ceil_div(groups, 4);
    timer_begin(QL_KERNEL_DQ_ENCODE, stream);
    hipLaunchKernelGGL(dq_encode, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, absmax, n1, mean, q.part,
                       f.nwg, mean, c8, scale);
    timer_end(QL_KERNEL_DQ_ENCODE, stream);
    return check_launch("nf4_quantize_dq");
}

}  // namespace qlnf4
