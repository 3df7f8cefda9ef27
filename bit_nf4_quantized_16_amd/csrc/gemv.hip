// Dequant-GEMV of the frozen-base LoRA linear layer for decode-size T
// (gfx950, bf16 MFMA). The NF4 codes are expanded straight into MFMA operand
// registers: w' = bf16(fl32(T[c] * a')), the value nf4_dequantize produces
// (contraction is off in this file so that a' = fl(fl(E(c8) S) + mu) rounds
// identically).
#include <algorithm>
#include <cstdlib>

#include "arrive.h"
#include "common.h"
#include "internal.h"
#include "mm_common.h"

namespace qlnf4 {

// ===========================================================================
// Dequant-GEMV for T <= 16 (decode). apxml.com "量化 LoRA (QLoRA) 与 4 位训练",
// forward pass: y = W' x + s B (A x).
//
// A workgroup of eight waves owns 16 output rows n0..n0+15. The reduction is
// cut into 256-wide steps (four 64-blocks of each row); wave w takes steps
// w, w+8, w+16, ... In a step, lane (i = l%16, g = l/16):
//  - loads bytes 16g.. and 64+16g.. of row n0+i's 128 code bytes, so every
//    load instruction reads 64 contiguous bytes of each of the 16 rows; one
//    v_permlane16_swap per word then hands each lane one whole block
//    (lane group g gets block 2, 0, 3, 1 of the step);
//  - expands its block with one lookup table into eight MFMA 16x16x32 A
//    operands. The k order inside an MFMA is free as long as both operands
//    share it: slot g of every MFMA belongs to the lane's block, and the A
//    operand keeps the lookup's own element order (no final interleave);
//  - x of the step (T tokens x 256 values) arrives with the codes in
//    coalesced 16-byte loads (512 bytes a token, two tokens an instruction),
//    is put in that element order and written to the wave's own LDS slot,
//    from which each MFMA reads its B operand (token i, the lane's block).
// A wave issues the loads of all its steps before the first multiply (or,
// when it has many, keeps a ring of them in flight), so no wave waits for
// another before the epilogue.
//
// The eight waves' 16x16 partial tiles are added in a fixed order in LDS and
// the adapter term s U B^T is added before rounding to bf16. U = x A^T (fp32,
// [T, r]) is computed once per call inside the same launch: the first
// workgroups of the grid each multiply one 16-row tile of A by one slice of
// kGemvUSteps steps of x (the same wave-per-step layout, A in registers) and
// store each element of their partial as one 64-bit word: the fp32 value and
// a tag of the launch (device-scope stores). A row workgroup, once its own
// rows are done, loads the words (device-scope loads) and adds the partials
// in slice order; if any tag is not this launch's yet, it sleeps a little
// and loads them again (bounded). Workgroups are dispatched in index order,
// so the U workgroups never wait on anything; should the retries still run
// out, the workgroup computes U itself from the same partial products in the
// same order (bit-identical). A launch being captured into a graph (its
// replays reuse the tag) mixes into its tag an epoch word that a kernel
// recorded before it advances at every replay (launch_tag), so a replay
// never takes the previous one's words for its own.
//
// One launch can serve up to kGemvGroup layers that read the same x (q/k/v,
// gate/up): the argument holds a descriptor per layer (weight, adapters,
// outputs, its own workspace slice of tagged words and its epoch word), the grid puts all
// layers' U workgroups first and then all their row workgroups, and each
// workgroup finds its layer from its index. Per layer the arithmetic and its
// order are those of a launch for that layer alone.
//
// Lanes of tokens >= T read token T-1 and their outputs are dropped; rows
// past N read row N-1 and are dropped.
// ===========================================================================
__global__ void advance_epoch_kernel(uint64_t* epoch) {
    if (threadIdx.x == 0) __hip_atomic_fetch_add(epoch, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

void launch_advance_epoch(uint64_t* epoch, hipStream_t stream) {
    hipLaunchKernelGGL(advance_epoch_kernel, dim3(1), dim3(64), 0, stream, epoch);
}

constexpr int kGemvRows = 16;
constexpr int kGemvWaves = 8;
constexpr int kGemvUSteps = 4;  // steps of x in one U workgroup's slice (waves 0..3)

// One weight of a launch: a launch serves up to kGemvGroup weights that share
// x (the same K, T, rank and scale), each with its own U workgroups, row
// workgroups, outputs and workspace.
constexpr int kGemvGroup = kGemvMaxGroup;

struct GemvWeight {
    NF4Dev w;
    int64_t N;
    const uint16_t* A;
    const uint16_t* B;
    uint16_t* Y;
    float* U_out;     // [T, r] fp32 = X A^T, or null
    uint64_t* uword;  // [nks][T][r]: slice ks of U, tag << 32 | fp32 bits (r > 0)

    int nu, nrow;     // its U and row workgroups
    int ub, rb;       // the grid index of its first U and first row workgroup
};

struct GemvArgs {
    const uint16_t* X;
    int T;
    int64_t K;
    int r;
    float scale;
    uint64_t token;   // 40 bits
    uint32_t tag;     // nonzero, from the token (a cleared word is 0)
    const uint64_t* epoch;  // captured launch: the epoch word its tag mixes in (launch_tag), else null
    int nks, rt;      // U workgroups of a weight = rt (16-row tiles of A) x nks (slices of kGemvUSteps steps)
    int spin;         // loads of the U words before computing U locally
    int ngroup;       // weights in this launch
    int nu_all;       // U workgroups of all weights (they come first in the grid)
    GemvWeight g[kGemvGroup];
};

// Steps whose loads one wave keeps in flight, by TX = 16-byte x loads per
// lane and step (T <= 2 * TX): fewer when x needs more registers.
template <int TX>
constexpr int gemv_max_steps() {
    return TX == 1 ? 6 : (TX == 2 ? 4 : (TX == 4 ? 3 : 2));
}

// Depth of the ring when a wave has more steps than that.
template <int TX>
constexpr int gemv_ring_depth() {
    return TX == 1 ? 4 : (TX == 2 ? 3 : 2);
}

// Codes, block constant and x of one step for one lane.
template <int TX>
struct GemvStage {
    uint4 c0, c1;  // code bytes 16g.. and 64+16g.. of the row's step (before the swap)
    uint32_t c8;   // E4M3 code of the block constant (double quantization)
    float s;       // its group scale, or the fp32 absmax itself
    uint4 x[TX];   // token 2u + l/32, values 8 (l%32) .. +8 of the step
};

// Block of the step that lane group g holds after the swap.
__device__ __forceinline__ int gemv_block_of(int g) { return (g & 1) ? (g >> 1) : 2 + (g >> 1); }

// Four waves per SIMD (two workgroups per CU) where that costs no spills: the
// ring for the widest x needs more registers, and spilling them measured
// slower than one workgroup per CU.
template <int TX, int NS>
constexpr int gemv_min_waves() {
    return (TX == 8 && NS == 0) ? 1 : 4;
}

// NS > 0: every wave has NS steps, or NS - 1 (all issued up front);
// NS == 0: a ring of gemv_ring_depth<TX>() steps, refilled as they are used.
template <int TX, int NS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(gemv_min_waves<TX, NS>()))) void gemv_kernel(
    GemvArgs p) {
    constexpr int D = NS > 0 ? NS : gemv_ring_depth<TX>();
    // each wave's x slot (2 TX tokens x 32 pieces); after its last step the
    // wave's 16 x 16 fp32 partial tile takes the slot's first KiB
    static_assert(2 * TX * 32 >= kGemvRows * 16 / 4, "partial tile fits the slot");
    __shared__ uint4 xw[kGemvWaves][2 * TX * 32];
    __shared__ float sU[16 * QL_MAX_RANK];
    __shared__ uint16_t sB[kGemvRows * QL_MAX_RANK];
    // this workgroup's weight (the U workgroups of all weights come first)
    const int bid = static_cast<int>(blockIdx.x);
    const bool is_u = bid < p.nu_all;
    int wi = 0;
    while (wi + 1 < p.ngroup && bid >= (is_u ? p.g[wi + 1].ub : p.g[wi + 1].rb)) ++wi;
    const GemvWeight& gw = p.g[wi];
    const NF4Dev& w = gw.w;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar step loop
    const int li = lane & 15, g = lane >> 4;
    const int64_t K = p.K, N = gw.N;
    const int T = p.T, r = p.r;
    const int64_t nblk = K / 64, rowbytes = K / 2;
    const int nbs = static_cast<int>((nblk + 3) / 4);
    const int tok = std::min(li, T - 1);
    const int pb = gemv_block_of(g);
    const uint32_t tag = launch_tag(p.tag, p.epoch);
    uint4* const slot = xw[wave];
    auto red = [&](int ww) { return reinterpret_cast<float*>(xw[ww]); };

    // x of step s (T tokens x 256 values) in coalesced loads: token 2u + l/32,
    // values 8 (l%32) .. +8
    auto load_x = [&](uint4 (&x)[TX], int64_t s) {
        const int64_t kx = std::min<int64_t>(256 * s + 8 * (lane & 31), K - 8);
#pragma unroll
        for (int u = 0; u < TX; ++u) {
            const int j = std::min(2 * u + (lane >> 5), T - 1);
            x[u] = *reinterpret_cast<const uint4*>(p.X + j * K + kx);
        }
    };
    // into the wave's slot in the lookup's element order: piece c of token j
    // at j*32 + (c ^ j), so the 16 lanes reading one piece column of 16 tokens
    // hit distinct banks; xin(m) is then the B operand of MFMA m (token li,
    // the lane's block)
    auto put_x = [&](const uint4 (&x)[TX]) {
#pragma unroll
        for (int u = 0; u < TX; ++u) {
            const int j = 2 * u + (lane >> 5), c = lane & 31;
            slot[j * 32 + (c ^ (j & 15))] = x_slot_order(x[u]);
        }
    };
    auto xin = [&](int m) { return slot[tok * 32 + ((8 * pb + m) ^ (tok & 15))]; };

    // U^T tile jt over the eight steps of slice ks: this wave's step, A rows
    // 16 jt .. +15 as the A operands (put in the same element order as x)
    auto u_unit = [&](int jt, int ks) {
        f32x4 ua = {0.f, 0.f, 0.f, 0.f};
        const int s = ks * kGemvUSteps + wave;
        if (wave < kGemvUSteps && s < nbs) {
            uint4 x[TX], av[8];
            load_x(x, s);
            const int64_t arow = std::min(16 * jt + li, r - 1);
#pragma unroll
            for (int m = 0; m < 8; ++m)
                av[m] = *reinterpret_cast<const uint4*>(gw.A + arow * K +
                                                        std::min<int64_t>(256 * s + 64 * pb + 8 * m, K - 8));
            put_x(x);
            const bool kin = 4 * s + pb < nblk;  // a block past K adds zeros
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint4 a = kin ? x_slot_order(av[m]) : make_uint4(0, 0, 0, 0);
                ua = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(xin(m)), ua, 0, 0, 0);
            }
        }
        return ua;
    };
    // D[4 g + rr][li] of each wave into its slot; thread e < 256 then adds
    // element e = 16 row + token over the waves in a fixed order
    auto put_tile = [&](const f32x4& a) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) red(wave)[(4 * g + rr) * 16 + li] = a[rr];
    };
    auto sum_tile = [&](int e) {
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kGemvWaves; ++ww) v += red(ww)[e];
        return v;
    };

    if (is_u) {
        // a U workgroup: its slice of one 16-row tile of U^T, published
        const int local = bid - gw.ub;
        const int jt = local % p.rt, ks = local / p.rt;
        put_tile(u_unit(jt, ks));
        __syncthreads();
        if (tid < 256) {
            const int j = 16 * jt + (tid >> 4), t = tid & 15;
            const float v = sum_tile(tid);
            if (t < T && j < r)  // device scope: read on other XCDs
                __hip_atomic_store(gw.uword + (static_cast<int64_t>(ks) * T + t) * r + j,
                                   (uint64_t{tag} << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }

    const int64_t n0 = static_cast<int64_t>(bid - gw.rb) * kGemvRows;
    const int64_t row = std::min<int64_t>(n0 + li, N - 1);
    const int nsw = wave < nbs ? (nbs - 1 - wave) / kGemvWaves + 1 : 0;  // steps of this wave
    const uint8_t* const rowcodes = w.packed + row * rowbytes;
    const int64_t rowblk = row * nblk;
    // block constants without a branch on the format: with double quantization
    // the E4M3 code and its group scale, else the absmax (and a dummy byte)
    const bool dq = w.dq != 0;
    const uint8_t* const c8p = dq ? w.c8 : reinterpret_cast<const uint8_t*>(w.absmax);
    const float* const sp = dq ? w.scale : w.absmax;
    static_assert(QL_DQ_BLOCKSIZE == 256, "group shift");
    const int sshift = dq ? 8 : 0;  // log2 of the group size
    const float mu = dq ? *w.mean : 0.0f;

    // rows n0.. of B for the epilogue, loaded first (one value a register:
    // packing two would wait for both loads)
    constexpr int kBQ = kGemvRows * QL_MAX_RANK / 512;
    uint32_t bpre[kBQ];
    const int nb = kGemvRows * r;
    if (r > 0) {
        const int64_t last = N * r - 1;
#pragma unroll
        for (int q = 0; q < kBQ; ++q) bpre[q] = gw.B[std::min<int64_t>(n0 * r + std::min(tid + 512 * q, nb - 1), last)];
    }

    auto issue = [&](GemvStage<TX>& st, int k) {
        const int64_t s = std::min(wave + kGemvWaves * k, nbs - 1);  // clamped: ring loads past the end
        const int64_t o0 = std::min<int64_t>(128 * s + 16 * g, rowbytes - 16);
        const int64_t o1 = std::min<int64_t>(128 * s + 64 + 16 * g, rowbytes - 16);
        st.c0 = *reinterpret_cast<const uint4*>(rowcodes + o0);
        st.c1 = *reinterpret_cast<const uint4*>(rowcodes + o1);
        const int64_t blk = rowblk + std::min<int64_t>(4 * s + pb, nblk - 1);
        st.c8 = c8p[blk];
        st.s = sp[blk >> sshift];
        load_x(st.x, s);
    };

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto consume = [&](const GemvStage<TX>& st, int k) {
        const int64_t s = wave + kGemvWaves * k;
        put_x(st.x);
        // the lane's whole block: low 16 bytes from the swapped second load,
        // high 16 bytes from the swapped first one
        uint32_t lo[4], hi[4];
        const uint32_t c0w[4] = {st.c0.x, st.c0.y, st.c0.z, st.c0.w};
        const uint32_t c1w[4] = {st.c1.x, st.c1.y, st.c1.z, st.c1.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const auto sw = __builtin_amdgcn_permlane16_swap(c1w[d], c0w[d], false, false);
            lo[d] = sw[0];
            hi[d] = sw[1];
        }
        const int64_t blr = 4 * s + pb;
        const float a = dq ? e4m3_value(st.c8) * st.s + mu : st.s;
        const Lut16 L = make_lut(blr < nblk ? a : 0.0f);  // a block past K adds zeros
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t cw = m < 4 ? lo[m] : hi[m - 4];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dequant8_lut_slots(cw, L)), as_bf16x8(xin(m)),
                                                          acc, 0, 0, 0);
        }
    };

    if constexpr (NS > 0) {
        // every wave has NS or NS - 1 steps: all issued now, the last one only
        // when the wave has it
        GemvStage<TX> st[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k)
            if (k + 1 < NS || k < nsw) issue(st[k], k);
#pragma unroll
        for (int k = 0; k < NS; ++k)
            if (k + 1 < NS || k < nsw) consume(st[k], k);
    } else {
        GemvStage<TX> ring[D];
#pragma unroll
        for (int q = 0; q < D; ++q) issue(ring[q], q);
        for (int k0 = 0; k0 < nsw; k0 += D) {
#pragma unroll
            for (int q = 0; q < D; ++q) {
                if (k0 + q < nsw) consume(ring[q], k0 + q);
                issue(ring[q], k0 + q + D);
            }
        }
    }

    // First try at the U words (one element a thread, all its slices at once),
    // issued before the reduction so that their latency overlaps it
    constexpr int kEarlyKs = TX <= 2 ? 16 : 8;  // fewer registers where x takes more
    const int nur = T * r;
    const bool early = r > 0 && nur <= 512 && p.nks <= kEarlyKs;
    uint64_t raw[kEarlyKs];
    if (early && tid < nur) {
#pragma unroll
        for (int ks = 0; ks < kEarlyKs; ++ks)
            raw[ks] = ks < p.nks ? __hip_atomic_load(gw.uword + static_cast<int64_t>(ks) * nur + tid, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                 : 0;
    }

    // D[4 g + rr][li]: rows n0 + 4 g + rr, token li
    put_tile(acc);
    if (r > 0) {
#pragma unroll
        for (int q = 0; q < kBQ; ++q)
            if (tid + 512 * q < nb) sB[tid + 512 * q] = static_cast<uint16_t>(bpre[q]);
    }
    __syncthreads();
    const float base = tid < 256 ? sum_tile(tid) : 0.0f;
    if (r > 0) {
        constexpr int kUE = 16 * QL_MAX_RANK / 512;  // U elements a thread adds
        float uv[kUE];
        int ok = 0;
        if (early && p.spin > 0) {
            bool bad = false;
            float v = 0.0f;
            if (tid < nur) {
#pragma unroll
                for (int ks = 0; ks < kEarlyKs; ++ks)
                    if (ks < p.nks) {
                        bad = bad || static_cast<uint32_t>(raw[ks] >> 32) != tag;
                        v += __uint_as_float(static_cast<uint32_t>(raw[ks]));
                    }
            }
            uv[0] = v;
#pragma unroll
            for (int q = 1; q < kUE; ++q) uv[q] = 0.0f;
            ok = !__syncthreads_or(bad);  // also: every wave's partial tile has been read
        }
        for (int it = 0; !ok && it < p.spin; ++it) {
            bool bad = false;
#pragma unroll
            for (int q = 0; q < kUE; ++q) {
                const int e = tid + 512 * q;
                float v = 0.0f;
                if (e < nur)
                    for (int ks = 0; ks < p.nks; ++ks) {
                        const uint64_t wd = __hip_atomic_load(gw.uword + static_cast<int64_t>(ks) * nur + e,
                                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        bad = bad || static_cast<uint32_t>(wd >> 32) != tag;
                        v += __uint_as_float(static_cast<uint32_t>(wd));
                    }
                uv[q] = v;
            }
            if (!__syncthreads_or(bad)) {  // also: every wave's partial tile has been read
                ok = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(8);
        }
        if (ok) {
#pragma unroll
            for (int q = 0; q < kUE; ++q)
                if (tid + 512 * q < nur) sU[tid + 512 * q] = uv[q];
        } else {
            // U here, from the same partial products added in the same order
            __syncthreads();  // every wave's partial tile has been read
            for (int e = tid; e < nur; e += 512) sU[e] = 0.0f;
            for (int jt = 0; jt < p.rt; ++jt)
                for (int ks = 0; ks < p.nks; ++ks) {
                    __syncthreads();  // every slot is free: the previous tile is read
                    put_tile(u_unit(jt, ks));
                    __syncthreads();
                    if (tid < 256) {
                        const int j = 16 * jt + (tid >> 4), t = tid & 15;
                        const float v = sum_tile(tid);
                        if (t < T && j < r) sU[t * r + j] += v;
                    }
                }
        }
        __syncthreads();  // sU is complete
        if (gw.U_out != nullptr && n0 == 0)
            for (int e = tid; e < nur; e += 512) gw.U_out[e] = sU[e];
    }
    if (tid < 256) {
        const int ol = tid >> 4, ot = tid & 15;  // output (row n0 + ol, token ot)
        const int64_t n = n0 + ol;
        if (n < N && ot < T) {
            float sum = base;
            if (r > 0) {
                float lora = 0.0f;
                for (int j = 0; j < r; ++j) lora = __builtin_fmaf(sU[ot * r + j], bf16_to_f32(sB[ol * r + j]), lora);
                sum += p.scale * lora;
            }
            gw.Y[ot * N + n] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(sum));
        }
    }
}

namespace {

// U partials: 16-row tiles of A and slices of eight 256-wide steps
struct GemvUPlan {
    int rt, nks;
    size_t part_bytes;
};

GemvUPlan gemv_u_plan(int64_t T, int64_t K, int r) {
    GemvUPlan u;
    u.rt = (r + 15) / 16;
    u.nks = static_cast<int>(ceil_div(ceil_div(K / 64, 4), kGemvUSteps));
    u.part_bytes = (static_cast<size_t>(u.nks) * T * r * sizeof(uint64_t) + 255) / 256 * 256;
    return u;
}

}  // namespace

size_t gemv_ws_bytes(int64_t T, int64_t K, int r) {
    if (r <= 0) return 0;
    const GemvUPlan u = gemv_u_plan(T, K, r);
    return (u.part_bytes + sizeof(uint64_t) + 255) / 256 * 256;  // the words, then the epoch word
}

namespace {

template <int TX>
void launch_gemv_tx(int ns, dim3 grid, const GemvArgs& g, hipStream_t stream) {
    const dim3 block(64 * kGemvWaves);
    constexpr int M = gemv_max_steps<TX>();
    switch (ns > M ? 0 : ns) {
        case 1: hipLaunchKernelGGL((gemv_kernel<TX, 1>), grid, block, 0, stream, g); break;
        case 2: hipLaunchKernelGGL((gemv_kernel<TX, 2>), grid, block, 0, stream, g); break;
        case 3:
            if constexpr (M >= 3) hipLaunchKernelGGL((gemv_kernel<TX, 3>), grid, block, 0, stream, g);
            break;
        case 4:
            if constexpr (M >= 4) hipLaunchKernelGGL((gemv_kernel<TX, 4>), grid, block, 0, stream, g);
            break;
        case 5:
            if constexpr (M >= 5) hipLaunchKernelGGL((gemv_kernel<TX, 5>), grid, block, 0, stream, g);
            break;
        case 6:
            if constexpr (M >= 6) hipLaunchKernelGGL((gemv_kernel<TX, 6>), grid, block, 0, stream, g);
            break;
        default: hipLaunchKernelGGL((gemv_kernel<TX, 0>), grid, block, 0, stream, g); break;
    }
}

}  // namespace

int launch_gemv_group(const GemvCall* calls, int nw, const uint16_t* X, int64_t T, int64_t K, int r, float scale,
                      void* ws, hipStream_t stream) {
    if (nw < 1 || nw > kGemvGroup) return set_error(QL_ERR_SHAPE, "dequant GEMV: %d weights in one launch", nw);
    GemvArgs g{};
    g.X = X;
    g.T = static_cast<int>(T);
    g.K = K;
    g.r = r;
    g.scale = scale;
    g.ngroup = nw;
    int nu = 0;
    if (r > 0) {
        const GemvUPlan u = gemv_u_plan(T, K, r);
        g.token = next_token() & ((uint64_t{1} << 40) - 1);
        g.tag = static_cast<uint32_t>(g.token % 0xFFFFFFFFull) + 1u;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return set_error(QL_ERR_HIP, "dequant GEMV: capture query");
        // a captured launch: the epoch word of weight 0's workspace slice
        g.epoch = cs != hipStreamCaptureStatusNone
                      ? reinterpret_cast<const uint64_t*>(static_cast<char*>(ws) + gemv_u_plan(T, K, r).part_bytes)
                      : nullptr;
        g.rt = u.rt;
        g.nks = u.nks;
        nu = u.rt * u.nks;
        // QLORA_NF4_GEMV_SPIN=n: loads of the U words before computing U locally
        // (0: every workgroup computes U itself)
        const char* e = std::getenv("QLORA_NF4_GEMV_SPIN");
        g.spin = e ? std::max(0, std::atoi(e)) : (1 << 14);
    }
    // grid: the U workgroups of every weight, then the row workgroups of every weight
    const size_t wsb = gemv_ws_bytes(T, K, r);
    int64_t total = static_cast<int64_t>(nu) * nw;
    g.nu_all = static_cast<int>(total);
    for (int i = 0; i < nw; ++i) {
        GemvWeight& gw = g.g[i];
        gw.w = calls[i].w;
        gw.N = calls[i].N;
        gw.A = calls[i].A;
        gw.B = calls[i].B;
        gw.Y = calls[i].Y;
        gw.U_out = calls[i].U_out;
        if (r > 0) {
            char* wbase = static_cast<char*>(ws) + wsb * i;
            gw.uword = reinterpret_cast<uint64_t*>(wbase);
        }
        gw.nu = nu;
        gw.ub = nu * i;
        gw.nrow = static_cast<int>(ceil_div(calls[i].N, kGemvRows));
        gw.rb = static_cast<int>(total);
        total += gw.nrow;
    }
    if (total >= (int64_t{1} << 31)) return set_error(QL_ERR_SHAPE, "dequant GEMV: grid too large");
    timer_begin(QL_KERNEL_GEMV, stream);
    if (g.epoch != nullptr)  // every replay advances the epoch before the launch reads it
        launch_advance_epoch(const_cast<uint64_t*>(g.epoch), stream);
    const dim3 grid(static_cast<uint32_t>(total));
    const int64_t nbs = ceil_div(K / 64, 4);
    const int ns = static_cast<int>(std::min<int64_t>(ceil_div(nbs, kGemvWaves), 1 << 20));
    const int tx = T <= 2 ? 1 : (T <= 4 ? 2 : (T <= 8 ? 4 : 8));
    switch (tx) {
        case 1: launch_gemv_tx<1>(ns, grid, g, stream); break;
        case 2: launch_gemv_tx<2>(ns, grid, g, stream); break;
        case 4: launch_gemv_tx<4>(ns, grid, g, stream); break;
        default: launch_gemv_tx<8>(ns, grid, g, stream); break;
    }
    timer_end(QL_KERNEL_GEMV, stream);
    return check_launch("dequant GEMV");
}

int launch_gemv(const NF4Dev& w, const uint16_t* X, int64_t T, int64_t N, int64_t K, const uint16_t* A,
                const uint16_t* B, int r, float scale, uint16_t* Y, float* U_out, void* ws, hipStream_t stream) {
    const GemvCall c{w, N, A, B, Y, U_out};
    return launch_gemv_group(&c, 1, X, T, K, r, scale, ws, stream);
}

}  // namespace qlnf4
