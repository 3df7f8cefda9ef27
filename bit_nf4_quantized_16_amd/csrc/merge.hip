// Adapter merge: a 16-bit copy of the base weight with the trained low-rank
// update added,
//
//   out[n][k] = bf16( fl32( w'[n][k] + s * sum_j B[n][j] A[j][k] ) ),
//   w' = fl32(T[c] * a')  (the dequantized weight before its bf16 rounding)
//
// ai-reference-codex "QLoRA 与 PEFT 全家", §3.6: after training, the product
// of the two adapter matrices is added back into the base weight, giving a
// plain model that needs no adapter branch at inference; aivaro.ru "Как
// работает QLoRA", §7 (step 5): for inference the adapters can be merged with
// the 4-bit model through delta weights; tqpw.cn notes, "Introduction": the
// LoRA weights stay 16-bit and cannot be folded into the 4-bit weight, so the
// merged weight is a 16-bit one. The 4-bit weight itself is not changed.
//
// One workgroup (four waves) owns a window of 256 columns and 128 rows: A's
// columns of the window are staged in LDS once, and each wave walks eight
// blocks of 16 rows over its own 64 columns. The rank-r product runs on bf16
// MFMA 16x16x32 (fp32 accumulation) in transposed form, D^T = A^T B^T, so
// that each lane's accumulators end up holding 16 consecutive columns of one
// row: the transposing LDS reads of A are addressed so that MFMA row m of
// tile t is column 16 (m / 4) + 4 t + m % 4. The lane then expands the 16
// codes of those columns (8 bytes, one block constant) to fp32, adds s D with
// one fused multiply-add each and writes 32 bytes of bf16. D never leaves
// registers.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "internal.h"
#include "mm_common.h"

namespace qlnf4 {

typedef uint32_t u32x4m __attribute__((ext_vector_type(4)));

namespace {

constexpr int kMergeCols = 256;  // columns (k) per workgroup window
constexpr int kMergeThreads = 256;
constexpr int kMergeLdA = kMergeCols + 8;  // bf16 row stride of the staged A columns

// Transposing read of rows r0 .. r0+7 of the staged A tile for lane li of a
// 16-lane group. Lane L supplies the address of four consecutive columns
// starting at cl (its own choice) in row r0 + L / 4 (and r0 + 4 + L / 4);
// lane li receives, for each of those rows, element li % 4 of the four
// columns supplied by the lanes with L % 4 == li / 4.
__device__ __forceinline__ bf16x8_t lds_rows8(const uint16_t* tile, int r0, int cl, int li) {
    const uint16_t* base = tile + (r0 + (li >> 2)) * kMergeLdA + cl;
    const v4i16_l lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_l*)(base));
    const v4i16_l hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_l*)(base + 4 * kMergeLdA));
    const v8i16_l v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

// Table address (byte offset into a 16-entry fp32 table) of the NF4 code in
// byte j of x, where x holds four codes already multiplied by 4, one a byte.
__device__ __forceinline__ uint32_t code_byte(uint32_t x, int j) { return (x >> (8 * j)) & 0xFFu; }

// Codes, block constant and B operands of one 16-row block for one lane.
template <int NS>
struct MergeIn {
    uint2 codes;  // columns k .. k+15, element 2j in the high nibble of byte j
    uint32_t c8;  // E4M3 code of the block constant (double quantization)
    float s;      // its group scale, or the fp32 absmax itself
    bf16x8_t bo[NS];
};

// B[row][c .. c+8) with zeros from column r on; RAG: r is not a multiple of 8
template <bool RAG>
__device__ __forceinline__ uint4 b_cols8(const uint16_t* rowp, int c, int r) {
    if constexpr (!RAG) {
        // loaded unconditionally (from a column inside the row), then zeroed:
        // no branch around the load
        const uint4 v = *reinterpret_cast<const uint4*>(rowp + std::min(c, r - 8));
        return c < r ? v : make_uint4(0, 0, 0, 0);
    } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (c + e < r) ? rowp[c + e] : 0u;
        return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
}

template <bool DQ, bool RAG, int NS>
__device__ __forceinline__ void merge_load(MergeIn<NS>& in, const NF4Dev& w, int row, int64_t K, int64_t k,
                                           const uint16_t* __restrict__ B, int r, int g) {
    const int64_t e = static_cast<int64_t>(row) * K + k;
    in.codes = *reinterpret_cast<const uint2*>(w.packed + e / 2);
    if constexpr (DQ) {
        in.c8 = w.c8[e / 64];
        in.s = w.scale[e / (64 * QL_DQ_BLOCKSIZE)];
    } else {
        in.c8 = 0;
        in.s = w.absmax[e / 64];
    }
    const uint16_t* brow = B + static_cast<int64_t>(row) * r;
#pragma unroll
    for (int js = 0; js < NS; ++js) in.bo[js] = as_bf16x8(b_cols8<RAG>(brow, 32 * js + 8 * g, r));
}

template <bool DQ, bool RAG, int NS>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(NF4Dev w, int N, int64_t K,
                                                              const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B, int r, float scale,
                                                              uint16_t* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint16_t* sA = smem;                        // [32 NS][kMergeLdA]: A[j][k0 .. k0+256)
    uint16_t* sO = smem + 32 * NS * kMergeLdA;  // [16][kMergeLdA]: one 16 x 256 result tile
    __shared__ float sT[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, g = lane >> 4;
    // column window; the last one is moved left to end at K (its columns
    // shared with the previous window get the same bytes twice)
    const bool narrow = K < kMergeCols;
    const int64_t k0 = narrow ? 0 : std::min<int64_t>(static_cast<int64_t>(blockIdx.x) * kMergeCols, K - kMergeCols);
    const int nrb = (N + 15) / 16;  // 16-row blocks; this workgroup takes blockIdx.y, + gridDim.y, ...
    const int step = static_cast<int>(gridDim.y);
    if (tid < 16) sT[tid] = kNF4Host[tid];

    // wave w: columns 64 w .. 64 w + 63 of the window (clamped into K for a
    // narrow matrix); lane (li, g): columns 16 g .. 16 g + 15 of those, row
    // li of each 16-row block. Rows past N are computed as row N - 1, so the
    // loop has no branches. The first two blocks' inputs are requested before
    // A is staged, later ones two blocks ahead of the MFMAs.
    const int kw = 64 * wave;
    const int64_t k = std::min<int64_t>(k0 + kw, K - 64) + 16 * g;
    // three input slots in a ring (no register copies between them)
    int rb = blockIdx.y;
    MergeIn<NS> s0, s1, s2;
    merge_load<DQ, RAG>(s0, w, std::min(16 * rb + li, N - 1), K, k, B, r, g);
    merge_load<DQ, RAG>(s1, w, std::min(16 * (rb + step) + li, N - 1), K, k, B, r, g);

    // stage A[j][k0 .. k0+256) for j < 32 NS (zero beyond r and beyond K)
    for (int c = tid; c < 32 * NS * (kMergeCols / 8); c += kMergeThreads) {
        const int j = c / (kMergeCols / 8), col = 8 * (c % (kMergeCols / 8));
        const int64_t kk = k0 + col;
        const uint4 v = (j < r && kk < K) ? *reinterpret_cast<const uint4*>(A + j * K + kk) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(sA + j * kMergeLdA + col) = v;
    }
    __syncthreads();
    const float mu = DQ ? *w.mean : 0.0f;
    // store phase: wave w writes rows 4 w .. 4 w + 3 of the tile, two rows of
    // 512 bytes per instruction
    // (a narrow matrix's stage columns c >= K hold column K - 64 + c % 64)
    const int srow = 4 * wave + (lane >> 5), scol = 8 * (lane & 31);
    const int64_t ocol = (narrow && scol >= K) ? K - 64 + (scol & 63) : k0 + scol;
    const int kws = narrow ? static_cast<int>(std::min<int64_t>(kw, K - 64)) : kw;

    // one 16-row block: request the inputs of the block two ahead into
    // `fill` (loads and stores share one in-order completion counter, so the
    // wait for a block's inputs also waits for every store issued before
    // them; two blocks back, those have drained), then compute from `use`
    auto block = [&](const MergeIn<NS>& use, MergeIn<NS>& fill, int rbi) {
        merge_load<DQ, RAG>(fill, w, std::min(16 * (rbi + 2 * step) + li, N - 1), K, k, B, r, g);

        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int js = 0; js < NS; ++js)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8_t ao = lds_rows8(sA, 32 * js + 8 * g, kws + 16 * (li & 3) + 4 * t, li);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, use.bo[js], acc[t], 0, 0, 0);
            }
        // acc[t][q] = D[n][k + 4 t + q]; element 2j of a code word is the
        // high nibble of its byte j, element 2j + 1 the low nibble
        const float a = DQ ? e4m3_value(use.c8) * use.s + mu : use.s;
        uint32_t o[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t cw = h == 0 ? use.codes.x : use.codes.y;
            uint32_t ev = (cw >> 2) & 0x3C3C3C3Cu;  // 4 x code of the even elements, one a byte
            uint32_t od = (cw << 2) & 0x3C3C3C3Cu;  // 4 x code of the odd elements
            // keep the byte-wise form: one extraction per element below
            asm("" : "+v"(ev), "+v"(od));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float* te = reinterpret_cast<const float*>(reinterpret_cast<const char*>(sT) + code_byte(ev, j));
                const float* to = reinterpret_cast<const float*>(reinterpret_cast<const char*>(sT) + code_byte(od, j));
                const int t = 2 * h + (j >> 1), q = 2 * (j & 1);
                o[4 * h + j] = pack_bf16x2(__builtin_fmaf(scale, acc[t][q], *te * a),
                                           __builtin_fmaf(scale, acc[t][q + 1], *to * a));
            }
        }
        uint4* so = reinterpret_cast<uint4*>(sO + li * kMergeLdA + kw + 16 * g);
        so[0] = make_uint4(o[0], o[1], o[2], o[3]);
        so[1] = make_uint4(o[4], o[5], o[6], o[7]);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = srow + 2 * i;
            const uint4 v = *reinterpret_cast<const uint4*>(sO + row * kMergeLdA + scol);
            const int n = std::min(16 * rbi + row, N - 1);
            // streaming store: the merged weight is written once, not read here
            __builtin_nontemporal_store(u32x4m{v.x, v.y, v.z, v.w},
                                        reinterpret_cast<u32x4m*>(out + static_cast<int64_t>(n) * K + ocol));
        }
        __syncthreads();
    };
    for (; rb < nrb; rb += 3 * step) {
        block(s0, s2, rb);
        if (rb + step >= nrb) break;
        block(s1, s0, rb + step);
        if (rb + 2 * step >= nrb) break;
        block(s2, s1, rb + 2 * step);
    }
}

}  // namespace

size_t merge_lds_bytes(int r) {
    const int rp32 = (r + 31) / 32 * 32;
    return static_cast<size_t>(rp32 + 16) * kMergeLdA * sizeof(uint16_t);
}

namespace {

// Workgroups of one merge_kernel instance that fit on the device at once
// (queried once per device and instance).
template <bool DQ, bool RAG, int NS>
int merge_slots(size_t lds) {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&merge_kernel<DQ, RAG, NS>),
                                                     kMergeThreads, lds) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    v = cus * per_cu;
    cached[dev].store(v, std::memory_order_relaxed);
    return v;
}

template <bool DQ, bool RAG, int NS>
int launch_merge_ns(const NF4Dev& w, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int r, float scale,
                    uint16_t* out, hipStream_t stream) {
    const size_t lds = merge_lds_bytes(32 * NS);
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&merge_kernel<DQ, RAG, NS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)) != hipSuccess)
        return set_error(QL_ERR_HIP, "adapter merge: LDS size %zu not accepted", lds);
    // one resident round: every workgroup strides over the 16-row blocks of
    // its column window
    const int64_t windows = ceil_div(K, kMergeCols), nrb = ceil_div(N, 16);
    const int64_t per_window = std::max<int64_t>(1, merge_slots<DQ, RAG, NS>(lds) / windows);
    const dim3 grid(static_cast<uint32_t>(windows), static_cast<uint32_t>(std::min(nrb, per_window)));
    timer_begin(QL_KERNEL_MERGE, stream);
    hipLaunchKernelGGL((merge_kernel<DQ, RAG, NS>), grid, dim3(kMergeThreads), lds, stream, w, static_cast<int>(N), K, A,
                       B, r, scale, out);
    timer_end(QL_KERNEL_MERGE, stream);
    return check_launch("adapter merge");
}

template <bool DQ, bool RAG>
int launch_merge_dq(const NF4Dev& w, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int r, float scale,
                    uint16_t* out, hipStream_t stream) {
    switch ((r + 31) / 32) {
        case 1: return launch_merge_ns<DQ, RAG, 1>(w, N, K, A, B, r, scale, out, stream);
        case 2: return launch_merge_ns<DQ, RAG, 2>(w, N, K, A, B, r, scale, out, stream);
        case 3: return launch_merge_ns<DQ, RAG, 3>(w, N, K, A, B, r, scale, out, stream);
        case 4: return launch_merge_ns<DQ, RAG, 4>(w, N, K, A, B, r, scale, out, stream);
        default: return set_error(QL_ERR_SHAPE, "adapter merge: rank %d", r);
    }
}

}  // namespace

int launch_merge(const NF4Dev& w, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int r, float scale,
                 uint16_t* out, hipStream_t stream) {
    if (N >= (int64_t(1) << 31)) return set_error(QL_ERR_SHAPE, "adapter merge: %lld rows", (long long)N);
    const bool rag = r % 8 != 0;
    if (w.dq)
        return rag ? launch_merge_dq<true, true>(w, N, K, A, B, r, scale, out, stream)
                   : launch_merge_dq<true, false>(w, N, K, A, B, r, scale, out, stream);
    return rag ? launch_merge_dq<false, true>(w, N, K, A, B, r, scale, out, stream)
               : launch_merge_dq<false, false>(w, N, K, A, B, r, scale, out, stream);
}

}  // namespace qlnf4
