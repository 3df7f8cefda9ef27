// Dequant-in-LDS GEMMs of the frozen-base LoRA layer (gfx950, bf16 MFMA
// 32x32x16, fp32 accumulation).
//
//   forward  Y[t][n]  = sum_k X[t][k] W'[n][k]  + sum_j sU[t][j] B[n][j]
//   dX       dX[t][k] = sum_n dY[t][n] W'[n][k] + sum_j G[t][j] A[j][k]
//
// apxml.com "量化 LoRA (QLoRA) 与 4 位训练": the 4-bit weight is dequantized to
// bf16 for the matmul and the adapter output is added; aivaro.ru "Как работает
// QLoRA", §7: the backward dequantizes the 4-bit weight on the fly as well.
//
// One kernel template serves both. The MFMA "A side" is the output feature
// dimension (n for the forward, k for dX); the "B side" is the tokens. A
// workgroup owns a TA x TT output tile: eight waves (4 along A x 2 along the
// tokens) for the 256 x 256 tile, four (2 x 2) for the 128 x 128 one. Each
// reduction step of 64 reads a token tile and an expanded bf16 weight tile
// from LDS; both are double buffered. The token tile arrives by direct
// global-to-LDS loads (no registers; 128-byte rows with an XOR swizzle of the
// 16-byte chunks instead of padding, so the operand reads hit distinct
// banks). The weight codes are loaded into registers two steps ahead, and
// step s+1's codes are expanded to bf16 and stored inside step s's MFMA
// stream, so dequantization overlaps the matrix cores. Load addresses are
// clamped into the matrix, so the step body has no branches; rows past the
// edge feed only outputs that are not stored, except past-the-end reduction
// rows of dX, whose weight rows are expanded with a zero absmax.
// The weight tile is row-major in both directions (a thread expands one
// block, or half of one, with a single absmax); dX reads its A operand
// through ds_read_b64_tr_b16, which hands each lane a column segment. The
// LoRA term follows as rp/64 extra reduction steps over the rank. The
// launch can also compute that term's token operand itself (U = X A^T for the
// forward, G = s dY B for dX): its first workgroups then run the rank-r
// projection (proj_dma.h) and hand it to the tiles in tagged words
// (arrive.h), on CUs the tiles leave free.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "arrive.h"
#include "mm_common.h"
#include "proj_dma.h"

namespace qlnf4 {

constexpr int kStep = 64;

struct TileArgs {
    NF4Dev w;
    const uint16_t* act;  // forward: X [T, K]; dX: dY [T, N]
    int64_t ld_act;
    const uint16_t* lt;  // token-side LoRA operand [T, rp]: forward bf16(s U), dX bf16(G)
    const uint16_t* la;  // A-side LoRA operand: forward B [N, r_la] (row stride ld_la); dX A [r_la, K]
    int64_t ld_la;
    int r_la;
    int rp;
    uint16_t* out;  // forward: Y [T, N]; dX: dX [T, K]
    int64_t T, N, K;
    int tiles_a, tiles_t;
    int splits;   // > 1: the reduction is split over gridDim.y workgroups
    float* part;  // split partial tiles, fp32 [splits, T, MA]
    // The token-side rank operand computed inside the launch (nu > 0; one
    // reduction split, rank r_u 8 or 16): workgroups [0, nu) run the
    // projection of one 16-token block each (proj, unsplit; U = X A^T for
    // the forward, G = s dY B for dX) and store its raw sums as tagged words
    // uword[t][j]; a tile reads its tokens' words before the rank step, in
    // place of lt, as bf16(s_u v).
    int nu;
    ProjArgs proj;
    int r_u;
    float s_u;
    int spin;  // word loads before the tile forms its tokens' U itself
    const uint64_t* epoch;  // captured launch: the epoch word its tag mixes in (launch_tag), else null
    // Grouped dX (the GRP kernels): dX = sum over ng layers that read the same
    // X of dY_L W_L' + G_L A_L. The layers' rows form one reduction of
    // gstep[ng] steps, layer L owning steps [gstep[L], gstep[L + 1]); the
    // split plan cuts that reduction as it cuts one layer's (a workgroup's
    // steps may span layers), and the rank step of layer L runs on split
    // L % splits.
    int ng;
    int gstep[kGemmMaxGroup + 1];
    GemmLayer gl[kGemmMaxGroup];
    // Grouped forward (the GRP kernels with DX false): Y_L = X W_L'^T +
    // Us_L B_L^T for ng layers that read the same X. Layer L owns row tiles
    // [gtile[L], gtile[L + 1]) of the tiles_a; its split partials sit at
    // columns gcol[L] .. of a [splits, T, gcol[ng]] buffer.
    int gtile[kGemmMaxGroup + 1];
    int64_t gcol[kGemmMaxGroup + 1];
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
#define QL_LDS __attribute__((address_space(3)))

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Transposing LDS read: within each 16-lane group, lane i receives element
// i%4 of the 4-element rows addressed by lanes 4e + i/4 (e = 0..3).
__device__ __forceinline__ v4i16 ld_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((QL_LDS v4i16*)(reinterpret_cast<uintptr_t>(p)));
}

// 16-byte chunk c of token-tile row r is stored at chunk c ^ swz(r): rows r
// and r+8 (same banks in a 32-bank LDS) and rows r and r+2 (same banks in a
// 64-bank LDS) get different chunk positions.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Padding (bf16 elements) of the dX weight-tile rows, which are read
// column-wise with transposing LDS loads: with 32, the four rows a 16-lane
// group reads fall in different banks of the 64-bank LDS.
#ifndef QL_GEMM_DX_PAD
#define QL_GEMM_DX_PAD 32
#endif

// dX weight tile: the 16-byte chunk c of row r is stored at chunk c ^ (r & 3).
// The expansion writes eight 64-byte row pieces per 16 lanes, which without
// it fall on four bank groups (4-way conflicts); with it two-way, while the
// transposing reads (whose rows r and r + 4 share the swizzle) stay
// conflict-free. (Measured time-neutral: the conflicts were not what bounds
// the dX kernel.)
__device__ __forceinline__ int dx_col(int r, int c) { return (((c >> 3) ^ (r & 3)) << 3) | (c & 7); }

// End of a pipeline stage: this wave's LDS writes are complete and its
// direct-to-LDS token loads have landed, then the workgroup barrier. The
// token loads of the stage were issued before at least N other vector loads
// (the codes prefetched for a later stage), which stay in flight: vmcnt(N)
// with lgkmcnt(0). A __syncthreads (or any LDS fence, which cannot tell the
// direct-to-LDS loads from the code loads) would drain them all. The memory
// clobber keeps the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
    asm volatile("s_barrier" ::: "memory");
}

template <int TA, int TT, int WA, int WT, bool DX>
struct TileShape {
    static constexpr int NW = WA * WT, NTHR = 64 * NW;      // waves, threads
    static constexpr int MW = TA / WA, TW = TT / WT;         // wave tile
    static constexpr int SA = MW / 32, ST = TW / 32;         // 32x32 MFMA sub-tiles per wave
    static constexpr int DMA = TT / 8 / NW;                  // 1 KiB token loads per wave per step
    static constexpr int CPT = TA * kStep / NTHR;            // codes per thread per step
    static constexpr int CC = CPT / 32;                      // 16-B code chunks per thread
    static constexpr int ROWS_A = DX ? kStep : TA;           // weight-tile rows (reduction rows for dX)
    static constexpr int LDA = DX ? TA + QL_GEMM_DX_PAD : kStep + 8;  // weight-tile LDS row (bf16, padded)
    static constexpr int TPR = DX ? TA / CPT : kStep / CPT;  // threads per weight-tile row
    static_assert(CPT == 32 || CPT == 64, "a thread expands one block or half of one");
    static_assert(DMA >= 1 && TT % (8 * NW) == 0, "token tile split");
};

template <int CC>
struct Codes {
    uint4 c[CC];
    BlockConst bc;
};

template <int TA, int TT, int WA, int WT, bool DX, bool DQ, bool GRP>
__global__ __launch_bounds__(64 * WA * WT, 512 / (64 * WA * WT)) void tile_gemm_kernel(TileArgs p) {
    using S = TileShape<TA, TT, WA, WT, DX>;
    constexpr int SA = S::SA, ST = S::ST, CPT = S::CPT, CC = S::CC, LDA = S::LDA, TPR = S::TPR;
    constexpr int MW = S::MW, TW = S::TW, NW = S::NW, NTHR = S::NTHR;

    // two stages of each tile, as separate arrays so that the compiler can tell
    // the stage being loaded from the stage being read
    __shared__ __attribute__((aligned(16))) uint16_t sA0[S::ROWS_A * LDA];
    __shared__ __attribute__((aligned(16))) uint16_t sA1[S::ROWS_A * LDA];
    __shared__ __attribute__((aligned(16))) uint16_t sX0[TT * kStep];
    __shared__ __attribute__((aligned(16))) uint16_t sX1[TT * kStep];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wa = wave / WT, wt = wave % WT;
    __shared__ int s_flag;

    // ---- U (forward) or G (dX) inside the launch, 256 x 256 tile: projection
    // workgroups. The projection's ring slots and partial sums live in the
    // tile's stages; for dX the projection reads B's rows column-wise.
    constexpr bool kUin = TA == 256 && TT == 256 && NW == 8;
    auto proj_lds = [&]() {
        using D = ProjDma<1>;
        return ProjLds<1>{{reinterpret_cast<uint16_t(*)[D::PS]>(sX0), reinterpret_cast<uint16_t(*)[D::PS]>(sX0 + D::PS * D::NW),
                           reinterpret_cast<uint16_t(*)[D::PS]>(sX1)},
                          {reinterpret_cast<uint16_t(*)[D::QS]>(sX1 + D::PS * D::NW), reinterpret_cast<uint16_t(*)[D::QS]>(sA0),
                           reinterpret_cast<uint16_t(*)[D::QS]>(sA0 + D::QS * D::NW)},
                          reinterpret_cast<float(*)[16][16]>(sA1), &s_flag};
    };
    const int ntiles = p.tiles_a * p.tiles_t;
    if constexpr (kUin) {
        static_assert(ProjDma<1>::NW == NW, "projection workgroups have the tile's eight waves");
        static_assert(2 * ProjDma<1>::PS * NW <= TT * kStep && 2 * ProjDma<1>::QS * NW <= S::ROWS_A * LDA &&
                          NW * 256 * 4 <= S::ROWS_A * LDA * 2,
                      "the projection's LDS fits in the stages");
        if (static_cast<int>(blockIdx.x) < p.nu) {
            ProjArgs pj = p.proj;
            pj.tag = launch_tag(p.proj.tag, p.epoch);
            proj_dma_block<1, DX>(pj, static_cast<int>(blockIdx.x), 0, 1, proj_lds());
            return;
        }
    }
    // dX: with eight waves, the two waves that share a SIMD (w and w+4) run
    // the two halves of a step in opposite order, so one expands codes (VALU)
    // while the other feeds the matrix core. The forward instead interleaves
    // each wave's own work (compute_expand below).
    const bool expand_first = DX && (NW == 8) && ((wave >> 2) & 1);

    // Workgroups are handed to the eight XCDs round robin; give each XCD a
    // contiguous range of tiles, token-major, so one XCD's L2 serves the same
    // activation rows to all its workgroups.
    const int g = static_cast<int>(blockIdx.x) - p.nu, qx = ntiles / 8, rem = ntiles % 8, x = g % 8;
    const int logical = x * qx + (x < rem ? x : rem) + g / 8;
    // a grouped forward: the layer owning this row tile, and the tile's
    // rows within it
    int fl = 0;
    if constexpr (GRP && !DX) {
#pragma unroll
        for (int i = 1; i < kGemmMaxGroup; ++i) fl += (i < p.ng && logical % p.tiles_a >= p.gtile[i]) ? 1 : 0;
    }
    const int64_t m0 = static_cast<int64_t>(logical % p.tiles_a - ((GRP && !DX) ? p.gtile[fl] : 0)) * TA;
    const int64_t t0 = static_cast<int64_t>(logical / p.tiles_a) * TT;
    const int64_t MA = DX ? p.K : ((GRP && !DX) ? p.gl[fl].N : p.N);
    const int64_t RED = DX ? p.N : p.K;
    const int nsteps_all = (GRP && DX) ? p.gstep[p.ng] : static_cast<int>(ceil_div(RED, kStep));
    // split-K: this workgroup covers reduction steps [sb, se)
    const int split = blockIdx.y;
    const int spp = (nsteps_all + p.splits - 1) / p.splits;
    const int sb = split * spp;
    const int se = min(nsteps_all, sb + spp);
    const int msteps = se;
    const float mu = (DQ && !GRP) ? *p.w.mean : 0.0f;
    // The operands of reduction step `step`: the arguments' own, or in a
    // grouped dX those of the layer bound below for the part of [sb, se) that
    // layer owns (its weight, dY with row stride N, N, double-quantization
    // mean, first step).
    NF4Dev gw{};
    const uint16_t* gact = nullptr;
    int64_t gN = 0;
    float gmu = 0.0f;
    int gbase = 0;
    auto lstep = [&](int step) -> int {
        if constexpr (GRP) return step - gbase;
        else return step;
    };
    auto lw = [&](int) -> const NF4Dev& {
        if constexpr (GRP) return gw;
        else return p.w;
    };
    auto lact = [&](int) {
        if constexpr (GRP) return gact;
        else return p.act;
    };
    auto lred = [&](int) -> int64_t {
        if constexpr (GRP) return gN;
        else return RED;
    };
    auto lld = [&](int) -> int64_t {
        if constexpr (GRP) return gN;
        else return p.ld_act;
    };
    auto lmu = [&](int) -> float {
        if constexpr (GRP) return gmu;
        else return mu;
    };
    if constexpr (GRP && !DX) {  // a grouped forward binds its tile's layer once (X, K are shared)
        gw = p.gl[fl].w;
        gact = p.act;
        gN = p.K;
        gmu = DQ ? *p.gl[fl].w.mean : 0.0f;
    }

    // ---- token tile: direct loads into LDS --------------------------------
    // Wave w issues loads q = NW i + w (i < DMA); load q fills rows 8q..8q+7.
    auto dma = [&](int step, uint16_t* sX) {
        const int64_t r0 = static_cast<int64_t>(lstep(step)) * kStep;
#pragma unroll
        for (int i = 0; i < S::DMA; ++i) {
            const int q = NW * i + wave;
            const int row = 8 * q + (lane >> 3);
            const int lc = (lane & 7) ^ swz(row);
            const int64_t t = min(t0 + row, p.T - 1);
            const int64_t col = min(r0 + 8 * lc, lred(step) - 8);
            // the address is formed before the builtin's argument list: with
            // the accessor calls inside it, the host pass of hipcc emitted no
            // launch stubs for this kernel template
            const uint16_t* const src = lact(step) + t * lld(step) + col;
            __builtin_amdgcn_global_load_lds(src, (QL_LDS void*)(sX + q * 512), 16, 0, 0);
        }
    };

    // ---- weight codes: registers, two steps ahead ----------------------------
    // dX with 8 threads per weight-tile row: the rows are 576 B apart (16
    // banks mod 64) and a row's threads 64 B apart, so with the plain order
    // (8 lanes to a row) the threads of a row four apart write the same banks
    // on every 16-byte store. Lanes 0-15 of a wave take 4 rows x threads 0-3
    // instead (lanes 16-31 the same rows, threads 4-7): with the column
    // swizzle of the layout their 16 stores fall in 16 different 4-bank
    // groups. The wave still loads the same 8 code rows, only in another
    // lane order.
    const int wrow = (DX && TPR == 8) ? (tid >> 6) * 8 + (((tid >> 5) & 1) << 2) + ((tid >> 2) & 3) : tid / TPR;
    const int wcol = ((DX && TPR == 8) ? (((tid >> 4) & 1) << 2) + (tid & 3) : tid % TPR) * CPT;
    auto gcodes = [&](int step, Codes<CC>& cs) {
        const int64_t r0 = static_cast<int64_t>(lstep(step)) * kStep;
        int64_t e;
        if constexpr (DX) {
            const int64_t n = min(r0 + wrow, lred(step) - 1);
            e = n * p.K + min(m0 + wcol, p.K - CPT);
        } else {
            const int64_t n = min(m0 + wrow, MA - 1);
            e = n * p.K + r0 + wcol;
        }
        // block constant first, the CC code chunks last (the stage barrier
        // lets the last CC loads of a stage stay in flight)
        const int64_t b = e / 64;
        const NF4Dev& w = lw(step);
        if constexpr (DQ) {
            cs.bc.c8 = w.c8[b];
            cs.bc.s = w.scale[b / QL_DQ_BLOCKSIZE];
        } else {
            cs.bc.c8 = 0;
            cs.bc.s = w.absmax[b];
        }
#pragma unroll
        for (int cc = 0; cc < CC; ++cc) cs.c[cc] = ld16(w.packed + e / 2 + 16 * cc);
    };

    // ---- expand one step's codes into a weight stage -----------------------
    auto expand = [&](int step, const Codes<CC>& cs, uint16_t* sA) {
        float a = block_value(cs.bc, DQ ? 1 : 0, lmu(step));
        if constexpr (DX) a = (static_cast<int64_t>(lstep(step)) * kStep + wrow < lred(step)) ? a : 0.0f;
        const Lut16 L = make_lut(a);
        uint16_t* dst = sA + wrow * LDA;
#pragma unroll
        for (int cc = 0; cc < CC; ++cc) {
            const uint32_t words[4] = {cs.c[cc].x, cs.c[cc].y, cs.c[cc].z, cs.c[cc].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = wcol + 32 * cc + 8 * q;
                st16(dst + (DX ? dx_col(wrow, c) : c), dequant8_lut(words[q], L));
            }
        }
    };

    f32x16 acc[SA][ST];
#pragma unroll
    for (int a = 0; a < SA; ++a)
#pragma unroll
        for (int b = 0; b < ST; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    auto load_a = [&](const uint16_t* sA, int a, int ks) -> bf16x8_t {
        if constexpr (!DX) {
            return as_bf16x8(ld16(sA + (wa * MW + a * 32 + (lane & 31)) * LDA + ks * 16 + 8 * (lane >> 5)));
        } else {
            // rows (reduction) 16 ks + 8 (lane/32) + 0..7 of column (k out) lane%32
            const int grp = lane >> 4, j = lane & 15;
            const int r = ks * 16 + 8 * (grp >> 1) + (j >> 2);  // and r + 4, same swizzle
            const uint16_t* base = sA + r * LDA + dx_col(r, wa * MW + a * 32 + 16 * (grp & 1) + 4 * (j & 3));
            const v4i16 lo = ld_tr16(base);
            const v4i16 hi = ld_tr16(base + 4 * LDA);
            const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8_t, v);
        }
    };
    auto load_b = [&](const uint16_t* sX, int b, int ks) -> bf16x8_t {
        const int row = wt * TW + b * 32 + (lane & 31);
        const int chunk = (2 * ks + (lane >> 5)) ^ swz(row);
        return as_bf16x8(ld16(sX + row * kStep + 8 * chunk));
    };
    auto compute = [&](const uint16_t* sA, const uint16_t* sX) {
#pragma unroll
        for (int ks = 0; ks < kStep / 16; ++ks) {
            bf16x8_t av[SA], bv[ST];
#pragma unroll
            for (int a = 0; a < SA; ++a) av[a] = load_a(sA, a, ks);
#pragma unroll
            for (int b = 0; b < ST; ++b) bv[b] = load_b(sX, b, ks);
#pragma unroll
            for (int a = 0; a < SA; ++a)
#pragma unroll
                for (int b = 0; b < ST; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
    };

    // Forward step: the MFMAs on one stage fused with the expansion of the
    // next step's codes into the other, a quarter of the expansion after each
    // 16-wide slice of the reduction, and scheduling groups that issue the
    // next slice's operand reads between this slice's MFMAs (six reads ahead)
    // with five VALU instructions after each MFMA. The three pipes then
    // overlap within every wave; measured 8-10 % faster than the two-wave
    // ping-pong of separate compute and expand phases, which the dX kernel
    // keeps (its A operands take two transposing reads each, and the fused
    // form measured slower there).
    auto compute_expand = [&](const uint16_t* sA, const uint16_t* sX, const Codes<CC>& cs, uint16_t* sAo) {
        const Lut16 L = make_lut(block_value(cs.bc, DQ ? 1 : 0, lmu(0)));
        uint16_t* dst = sAo + wrow * LDA + wcol;
        constexpr int NQ = CC * 4, PER = NQ / (kStep / 16);  // 8-code words per slice
        static_assert(NQ % (kStep / 16) == 0, "expansion split over the slices");
#pragma unroll
        for (int ks = 0; ks < kStep / 16; ++ks) {
            bf16x8_t av[SA], bv[ST];
#pragma unroll
            for (int a = 0; a < SA; ++a) av[a] = load_a(sA, a, ks);
#pragma unroll
            for (int b = 0; b < ST; ++b) bv[b] = load_b(sX, b, ks);
#pragma unroll
            for (int a = 0; a < SA; ++a)
#pragma unroll
                for (int b = 0; b < ST; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
#pragma unroll
            for (int j = ks * PER; j < (ks + 1) * PER; ++j) {
                const int cc = j / 4, q = j % 4;
                const uint32_t w = q == 0 ? cs.c[cc].x : q == 1 ? cs.c[cc].y : q == 2 ? cs.c[cc].z : cs.c[cc].w;
                st16(dst + 32 * cc + 8 * q, dequant8_lut(w, L));
            }
        }
    };
    auto interleave_step = [&]() {
        if constexpr (!DX) {
            __builtin_amdgcn_sched_group_barrier(0x100, SA + ST, 0);  // LDS reads: operands of slice 0
#pragma unroll
            for (int ks = 0; ks < kStep / 16; ++ks)
#pragma unroll
                for (int i = 0; i < SA * ST; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    if (ks + 1 < kStep / 16 && i < SA + ST)
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // an operand of slice ks + 1
                    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);      // VALU
                }
        }
    };

    // Pipeline (two steps per iteration, stages named statically):
    //   step s:   token loads for s+1 -> the other stage; codes for s+2 -> the
    //             free register set; MFMAs on stage s; expand step s+1.
    Codes<CC> cs0, cs1;
    if constexpr (GRP && DX) {
        // A grouped dX: the same pipeline (dX form) over the part of [sb, se)
        // each layer owns, layer by layer into the same accumulators; each
        // part ends with every wave past a barrier after its last MFMA, so
        // the stages are free for the next. (Kept apart from the one-layer
        // text below, whose code it would otherwise change.)
        for (int L = 0; L < p.ng; ++L) {
            const int b = max(sb, p.gstep[L]), e = min(se, p.gstep[L + 1]);
            if (b >= e) continue;
            gw = p.gl[L].w;
            gact = p.gl[L].act;
            gN = p.gl[L].N;
            gmu = DQ ? *p.gl[L].w.mean : 0.0f;
            gbase = p.gstep[L];
            dma(b, sX0);
            gcodes(b, cs0);
            gcodes(min(b + 1, e - 1), cs1);
            expand(b, cs0, sA0);
            __syncthreads();
            for (int s = b; s < e; s += 2) {
                dma(min(s + 1, e - 1), sX1);
                __builtin_amdgcn_sched_barrier(0);
                gcodes(min(s + 2, e - 1), cs0);
                if (expand_first) {
                    expand(s + 1, cs1, sA1);
                    compute(sA0, sX0);
                } else {
                    compute(sA0, sX0);
                    expand(s + 1, cs1, sA1);
                }
                stage_barrier<CC>();
                if (s + 1 >= e) break;
                dma(min(s + 2, e - 1), sX0);
                __builtin_amdgcn_sched_barrier(0);
                gcodes(min(s + 3, e - 1), cs1);
                if (expand_first) {
                    expand(s + 2, cs0, sA0);
                    compute(sA1, sX1);
                } else {
                    compute(sA1, sX1);
                    expand(s + 2, cs0, sA0);
                }
                stage_barrier<CC>();
            }
        }
    } else if (sb < se) {
    dma(sb, sX0);
    gcodes(sb, cs0);
    gcodes(min(sb + 1, msteps - 1), cs1);
    expand(sb, cs0, sA0);
    __syncthreads();
    for (int s = sb; s < msteps; s += 2) {
        dma(min(s + 1, msteps - 1), sX1);
        __builtin_amdgcn_sched_barrier(0);  // the token loads stay ahead of the code loads
        gcodes(min(s + 2, msteps - 1), cs0);
        interleave_step();
        if constexpr (!DX) {
            compute_expand(sA0, sX0, cs1, sA1);
        } else if (expand_first) {
            expand(s + 1, cs1, sA1);
            compute(sA0, sX0);
        } else {
            compute(sA0, sX0);
            expand(s + 1, cs1, sA1);
        }
        stage_barrier<CC>();
        if (s + 1 >= msteps) break;
        dma(min(s + 2, msteps - 1), sX0);
        __builtin_amdgcn_sched_barrier(0);
        gcodes(min(s + 3, msteps - 1), cs1);
        interleave_step();
        if constexpr (!DX) {
            compute_expand(sA1, sX1, cs0, sA0);
        } else if (expand_first) {
            expand(s + 2, cs0, sA0);
            compute(sA1, sX1);
        } else {
            compute(sA1, sX1);
            expand(s + 2, cs0, sA0);
        }
        stage_barrier<CC>();
    }
    }  // sb < se

    // U (forward) or G (dX) inside the launch: the token operand of the rank
    // step from the words of this tile's tokens (TT x r_u, at most 8 a
    // thread), each converted as the separate projection converts it, bf16(s_u v), and
    // stored straight into the stage (a retry overwrites it). While any tag
    // is not this launch's, the workgroup sleeps and loads again, at most
    // spin times. The projection workgroups come first in the grid and wait
    // on nothing, so that bound is a safety net only: should it run out, the
    // tile forms its values itself, each an fp32 sum of the products in k
    // order (plain fused multiply-adds, a few registers; the same values up
    // to rounding, not bit for bit). Ranks r_u .. 63 are zero.
    auto stage_u_words = [&]() {
        if constexpr (kUin) {
        constexpr int WPT = TT * 16 / NTHR;  // words a thread, at most
        const int lg = p.r_u == 16 ? 4 : 3;  // r_u is 8 or 16
        const uint32_t tag = launch_tag(p.proj.tag, p.epoch);
        const int nw = TT << lg;
        auto stage_words = [&]() -> bool {
            bool ok = true;
#pragma unroll
            for (int i = 0; i < WPT; ++i) {
                const int e = tid + NTHR * i;
                if (e < nw) {
                    const int row = e >> lg, j = e & (p.r_u - 1);
                    const int64_t t = t0 + row;
                    uint64_t wd = 0;
                    if (t < p.T) {
                        wd = __hip_atomic_load(p.proj.uword + (t << lg) + j, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        ok = ok && static_cast<uint32_t>(wd >> 32) == tag;
                    }
                    sX0[row * kStep + 8 * ((j >> 3) ^ swz(row)) + (j & 7)] =
                        to_bf16_bits(p.s_u * __uint_as_float(static_cast<uint32_t>(wd)));
                }
            }
            return ok;
        };
        auto all_ok = [&](bool ok) -> bool {
            __syncthreads();
            if (tid == 0) s_flag = 1;
            __syncthreads();
            if (!ok) s_flag = 0;
            __syncthreads();
            return s_flag != 0;
        };
        bool ok = p.spin >= 0 && all_ok(stage_words());  // spin < 0: always form U locally (tests)
        for (int it = 0; !ok && it < p.spin; ++it) {
            __builtin_amdgcn_s_sleep(8);
            ok = all_ok(stage_words());
        }
        if (!ok) {
#pragma unroll 1
            for (int i = 0; i < WPT; ++i) {
                const int e = tid + NTHR * i;
                if (e >= nw) continue;
                const int row = e >> lg, j = e & (p.r_u - 1);
                const int64_t t = t0 + row;
                float u = 0.0f;
                if (t < p.T) {
                    const uint16_t* xr = p.proj.P + t * p.proj.ldp;
                    if constexpr (DX) {
                        // G: column j of B [kred, ldq], one element a step
                        const uint16_t* bc = p.proj.Q + j;
#pragma unroll 1
                        for (int64_t k = 0; k < p.proj.kred; k += 8) {
                            const uint4 xv = ld16(xr + k);
                            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                u = fmaf(bf16_to_f32(xw[q] & 0xFFFFu), bf16_to_f32(bc[(k + 2 * q) * p.proj.ldq]), u);
                                u = fmaf(bf16_to_f32(xw[q] >> 16), bf16_to_f32(bc[(k + 2 * q + 1) * p.proj.ldq]), u);
                            }
                        }
                    } else {
                        const uint16_t* ar = p.proj.Q + j * p.proj.ldq;
#pragma unroll 1
                        for (int64_t k = 0; k < p.proj.kred; k += 8) {
                            const uint4 xv = ld16(xr + k), av = ld16(ar + k);
                            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                u = fmaf(bf16_to_f32(xw[q] & 0xFFFFu), bf16_to_f32(aw[q] & 0xFFFFu), u);
                                u = fmaf(bf16_to_f32(xw[q] >> 16), bf16_to_f32(aw[q] >> 16), u);
                            }
                        }
                    }
                }
                sX0[row * kStep + 8 * ((j >> 3) ^ swz(row)) + (j & 7)] = to_bf16_bits(p.s_u * u);
            }
        }
        // ranks r_u .. 63 are zero
#pragma unroll
        for (int i = 0; i < TT * 8 / NTHR; ++i) {
            const int c = tid + NTHR * i;
            const int row = c >> 3, lc = c & 7;
            if (8 * lc >= p.r_u) st16(sX0 + row * kStep + 8 * (lc ^ swz(row)), make_uint4(0, 0, 0, 0));
        }
        }
    };

    // LoRA term: rp/64 more reduction steps over the rank, staged directly
    // (by the first split only; in a grouped dX, each layer's by split
    // L % splits: rank step ls of this split is step ls % nr of layer
    // split + (ls / nr) splits).
    const int nr = p.rp / kStep;
    constexpr bool kGdx = GRP && DX, kGfwd = GRP && !DX;
    const int nls = kGdx ? (split < p.ng ? nr * ((p.ng - 1 - split) / p.splits + 1) : 0) : (split == 0 ? nr : 0);
    for (int ls = 0; ls < nls; ++ls) {
        const int rl = kGdx ? split + (ls / nr) * p.splits : fl;  // the rank step's layer
        const uint16_t* const lt = GRP ? p.gl[rl].lt : p.lt;
        const uint16_t* const la = GRP ? p.gl[rl].la : p.la;
        const int64_t j0 = static_cast<int64_t>(kGdx ? ls % nr : ls) * kStep;
        if (kUin && p.nu > 0) {
            stage_u_words();  // rp == 64: the one rank step
        } else {
#pragma unroll
            for (int i = 0; i < TT * 8 / NTHR; ++i) {
                const int c = tid + NTHR * i;
                const int row = c >> 3, lc = c & 7;
                const int64_t t = t0 + row;
                const uint4 v = (t < p.T) ? ld16(lt + t * p.rp + j0 + 8 * lc) : make_uint4(0, 0, 0, 0);
                st16(sX0 + row * kStep + 8 * (lc ^ swz(row)), v);
            }
        }
        if constexpr (!DX) {
            // B rows n, 64 rank columns
#pragma unroll
            for (int i = 0; i < TA * 8 / NTHR; ++i) {
                const int c = tid + NTHR * i;
                const int64_t n = m0 + (c >> 3);
                const int64_t j = j0 + 8 * (c & 7);
                const uint4 v = (n < MA && j < p.r_la) ? ld16(la + n * p.ld_la + j) : make_uint4(0, 0, 0, 0);
                st16(sA0 + (c >> 3) * LDA + 8 * (c & 7), v);
            }
        } else {
            // A rows j (reduction), TA columns k: the same row-major layout as W'
#pragma unroll
            for (int i = 0; i < TA * 8 / NTHR; ++i) {
                const int c = tid + NTHR * i;
                const int row = c / (TA / 8), col = 8 * (c % (TA / 8));
                const int64_t j = j0 + row;
                const int64_t k = m0 + col;
                const uint4 v = (j < p.r_la && k < p.K) ? ld16(la + j * p.ld_la + k) : make_uint4(0, 0, 0, 0);
                st16(sA0 + row * LDA + dx_col(row, col), v);
            }
        }
        __syncthreads();
        compute(sA0, sX0);
        __syncthreads();
    }

    // Epilogue: D[m][t] -> out[t][m]; acc element r of sub-tile (a, b) sits at
    // m = 32a + 8(r/4) + 4(lane/32) + r%4, t = 32b + lane%32 of the wave tile.
    if (p.splits > 1) {
        // fp32 partial tile of this split (staging these through LDS like the
        // bf16 tile below measured no faster); a grouped forward's layer
        // writes its columns of the shared partial rows
        const int64_t pld = kGfwd ? p.gcol[p.ng] : MA;
        const int64_t pcol = kGfwd ? p.gcol[fl] : 0;
#pragma unroll
        for (int a = 0; a < SA; ++a)
#pragma unroll
            for (int b = 0; b < ST; ++b)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int64_t m = m0 + wa * MW + a * 32 + 8 * qq + 4 * (lane >> 5);
                    const int64_t t = t0 + wt * TW + b * 32 + (lane & 31);
                    if (t < p.T && m < MA) {
                        const float4 v = make_float4(acc[a][b][4 * qq], acc[a][b][4 * qq + 1], acc[a][b][4 * qq + 2],
                                                     acc[a][b][4 * qq + 3]);
                        *reinterpret_cast<float4*>(p.part + (static_cast<int64_t>(split) * p.T + t) * pld + pcol + m) = v;
                    }
                }
        return;
    }
    // bf16 tile through the (now idle) LDS stages, transposed to [t][m], so
    // that every global store writes whole 16-byte chunks of output rows
    // (lanes 8 bytes each in 32 different rows would scatter the writes).
    // Rows of TA bf16, a quarter of the TT rows per stage array, the 16-byte
    // chunk c of row r stored at c ^ (r % CPR).
    constexpr int RPA = TT / 4, CPR = TA / 8;
    static_assert(RPA * TA * 2 <= TT * kStep * 2 && RPA * TA * 2 <= S::ROWS_A * LDA * 2, "output staging fits");
    auto out_row = [&](int t) -> char* {
        const int g = t / RPA;
        uint16_t* const base = g == 0 ? sA0 : g == 1 ? sA1 : g == 2 ? sX0 : sX1;
        return reinterpret_cast<char*>(base) + (t % RPA) * (TA * 2);
    };
    __syncthreads();  // every wave is done reading the stages
#pragma unroll
    for (int a = 0; a < SA; ++a)
#pragma unroll
        for (int b = 0; b < ST; ++b)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int m = wa * MW + a * 32 + 8 * qq + 4 * (lane >> 5);
                const int t = wt * TW + b * 32 + (lane & 31);
                uint2 v;
                v.x = pack_bf16x2(acc[a][b][4 * qq], acc[a][b][4 * qq + 1]);
                v.y = pack_bf16x2(acc[a][b][4 * qq + 2], acc[a][b][4 * qq + 3]);
                const int c = (m / 8) ^ (t % RPA % CPR);
                *reinterpret_cast<uint2*>(out_row(t) + c * 16 + (m % 8) * 2) = v;
            }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TT * CPR / NTHR; ++i) {
        const int q = i * NTHR + tid;
        const int t = q / CPR, c = q % CPR;
        const int64_t gt = t0 + t, gm = m0 + 8 * c;
        if (gt >= p.T || gm >= MA) continue;  // MA is a multiple of 8: a chunk is whole or outside
        const uint4 v = *reinterpret_cast<const uint4*>(out_row(t) + (c ^ (t % RPA % CPR)) * 16);
        *reinterpret_cast<uint4*>((kGfwd ? p.gl[fl].out : p.out) + gt * MA + gm) = v;
    }
}

namespace {

int cu_count() {
    static int cached = 0;
    if (cached == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cached = n;
        else
            cached = 256;
    }
    return cached;
}

__global__ void split_reduce_kernel(const float* __restrict__ part, int splits, int64_t n4, uint16_t* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n4) return;
    float4 s = reinterpret_cast<const float4*>(part)[i];
    for (int k = 1; k < splits; ++k) {
        const float4 v = reinterpret_cast<const float4*>(part)[k * n4 + i];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    uint2 o;
    o.x = pack_bf16x2(s.x, s.y);
    o.y = pack_bf16x2(s.z, s.w);
    reinterpret_cast<uint2*>(out)[i] = o;
}

// A grouped forward's reduce pass: the summed partials of column chunk m of
// the layers' concatenated columns go to the layer owning m (every layer's
// column count is a multiple of 8, so a 4-column chunk has one owner).
struct GroupOut {
    uint16_t* out[kGemmMaxGroup];
    int64_t col[kGemmMaxGroup + 1];
    int ng;
};

__global__ void split_reduce_group_kernel(const float* __restrict__ part, int splits, int64_t T, GroupOut g) {
    const int64_t ncat = g.col[g.ng], n4 = T * ncat / 4;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n4) return;
    float4 s = reinterpret_cast<const float4*>(part)[i];
    for (int k = 1; k < splits; ++k) {
        const float4 v = reinterpret_cast<const float4*>(part)[k * n4 + i];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    const int64_t t = 4 * i / ncat, m = 4 * i - t * ncat;
    int L = 0;
    for (int j = 1; j < g.ng; ++j) L += m >= g.col[j] ? 1 : 0;
    const int64_t n = g.col[L + 1] - g.col[L];
    uint2 o;
    o.x = pack_bf16x2(s.x, s.y);
    o.y = pack_bf16x2(s.z, s.w);
    *reinterpret_cast<uint2*>(g.out[L] + t * n + (m - g.col[L])) = o;
}

// GRP: a grouped dX (a.ng layers, a.gstep set) or forward (a.gtile, a.gcol
// set, a.N the row tiles' total rows, the 256 tile only); a.w only gives
// the format.
template <bool DX, bool GRP = false>
int launch_tiles(TileArgs& a, float* split_ws, int kid, const char* what, hipStream_t stream, int nu = 0) {
    const int64_t MA = DX ? a.K : a.N;
    const GemmPlan pl = plan_gemm(MA, a.T, (GRP && DX) ? int64_t{kStep} * a.gstep[a.ng] : (DX ? a.N : a.K));
    const int tile = pl.tile;
    if (GRP && !DX && tile != 256) return set_error(QL_ERR_UNSUPPORTED, "%s: needs the 256 tile", what);
    a.tiles_a = static_cast<int>(ceil_div(MA, tile));
    a.tiles_t = static_cast<int>(ceil_div(a.T, tile));
    a.splits = pl.splits;
    a.part = split_ws;
    if (a.splits > 1 && split_ws == nullptr) return set_error(QL_ERR_WORKSPACE, "%s: split workspace missing", what);
    a.nu = nu;
    if (nu > 0 && (tile != 256 || a.splits != 1))
        return set_error(QL_ERR_UNSUPPORTED, "%s: the projection inside the launch needs the unsplit 256 tile", what);
    const dim3 grid(static_cast<uint32_t>(nu + static_cast<int64_t>(a.tiles_a) * a.tiles_t),
                    static_cast<uint32_t>(a.splits));
    timer_begin(kid, stream);
    if (tile == 256) {
        if (a.w.dq)
            hipLaunchKernelGGL((tile_gemm_kernel<256, 256, 4, 2, DX, true, GRP>), grid, dim3(512), 0, stream, a);
        else
            hipLaunchKernelGGL((tile_gemm_kernel<256, 256, 4, 2, DX, false, GRP>), grid, dim3(512), 0, stream, a);
    } else {
        if (a.w.dq)
            hipLaunchKernelGGL((tile_gemm_kernel<128, 128, 2, 2, DX, true, GRP>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((tile_gemm_kernel<128, 128, 2, 2, DX, false, GRP>), grid, dim3(256), 0, stream, a);
    }
    if (a.splits > 1 && GRP && !DX) {
        GroupOut g{};
        g.ng = a.ng;
        for (int i = 0; i < a.ng; ++i) g.out[i] = a.gl[i].out;
        for (int i = 0; i <= a.ng; ++i) g.col[i] = a.gcol[i];
        const int64_t n4 = a.T * a.gcol[a.ng] / 4;
        hipLaunchKernelGGL(split_reduce_group_kernel, dim3(static_cast<uint32_t>(ceil_div(n4, 256))), dim3(256), 0,
                           stream, split_ws, a.splits, a.T, g);
    } else if (a.splits > 1) {
        const int64_t n4 = a.T * MA / 4;
        hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<uint32_t>(ceil_div(n4, 256))), dim3(256), 0, stream,
                           split_ws, a.splits, n4, a.out);
    }
    timer_end(kid, stream);
    return check_launch(what);
}

}  // namespace

// Tile and split plan for an MA x T output with a reduction of RED. The
// 256x256 tile (eight waves) moves the least LDS traffic per flop; when its
// grid cannot fill the chip the reduction is split (partial fp32 tiles added
// in a fixed order afterwards) or, for short reductions, the 128x128 tile is
// used. QLORA_NF4_GEMM_TILE=128 or 256 forces the tile (tests run both),
// QLORA_NF4_GEMM_SPLITS=n forces the split count of the 256 tile.
GemmPlan plan_gemm(int64_t MA, int64_t T, int64_t RED) {
    GemmPlan pl;
    const char* e = std::getenv("QLORA_NF4_GEMM_TILE");
    const char* es = std::getenv("QLORA_NF4_GEMM_SPLITS");
    const int64_t cus = cu_count();
    const int64_t steps = ceil_div(RED, 64);
    const int64_t n256 = ceil_div(MA, 256) * ceil_div(T, 256);
    const int64_t n128 = ceil_div(MA, 128) * ceil_div(T, 128);
    int64_t splits = 1;
    if (n256 < cus) splits = std::min<int64_t>(cus / n256, steps / 16);
    if (splits < 1) splits = 1;
    if (es) splits = std::max<int64_t>(1, std::min<int64_t>(std::atoi(es), steps));
    splits = ceil_div(steps, ceil_div(steps, splits));  // no empty split
    // relative cost in 256-tile step units: rounds x steps per round
    const double c256 = static_cast<double>(ceil_div(n256 * splits, cus)) * ceil_div(steps, splits) +
                        (splits > 1 ? 0.15 * steps : 0.0);
    const double c128 = static_cast<double>(ceil_div(n128, 2 * cus)) * steps * 0.5 / 0.7;
    pl.tile = (c128 < c256) ? 128 : 256;
    if (e && std::strcmp(e, "128") == 0) pl.tile = 128;
    if (e && std::strcmp(e, "256") == 0) pl.tile = 256;
    pl.splits = (pl.tile == 256) ? static_cast<int>(splits) : 1;
    pl.cost = pl.tile == 256 ? c256 : c128;
    return pl;
}

size_t gemm_split_bytes(int64_t MA, int64_t T, int64_t RED) {
    const GemmPlan pl = plan_gemm(MA, T, RED);
    return pl.splits > 1 ? static_cast<size_t>(pl.splits) * T * MA * sizeof(float) : 0;
}

int launch_gemm_fwd(const NF4Dev& w, const uint16_t* X, const uint16_t* Us, const uint16_t* Bsrc, int64_t ld_b,
                    int r_b, int rp, uint16_t* Y, int64_t T, int64_t N, int64_t K, float* split_ws, hipStream_t stream) {
    TileArgs a{};
    a.w = w;
    a.act = X;
    a.ld_act = K;
    a.lt = Us;
    a.la = Bsrc;
    a.ld_la = ld_b;
    a.r_la = r_b;
    a.rp = rp;
    a.out = Y;
    a.T = T;
    a.N = N;
    a.K = K;
    return launch_tiles<false>(a, split_ws, QL_KERNEL_GEMM_FWD, "dequant GEMM forward", stream);
}

bool gemm_fwd_u_in_launch(int64_t N, int64_t K, int64_t T, int r) {
    if (r != 8 && r != 16) return false;
    if (const char* e = std::getenv("QLORA_NF4_FWD_U"))
        if (std::strcmp(e, "prepass") == 0) return false;
    const GemmPlan pl = plan_gemm(N, T, K);
    return pl.tile == 256 && pl.splits == 1 && lora_proj_splits(T, r, K, false) == 1;
}

bool gemm_dx_g_in_launch(int64_t N, int64_t K, int64_t T, int r) {
    if (r != 8 && r != 16) return false;
    if (const char* e = std::getenv("QLORA_NF4_FWD_U"))
        if (std::strcmp(e, "prepass") == 0) return false;
    const GemmPlan pl = plan_gemm(K, T, N);
    return pl.tile == 256 && pl.splits == 1 && lora_proj_splits(T, r, N, true) == 1;
}

int launch_gemm_dx_g(const NF4Dev& w, const uint16_t* dY, const uint16_t* A, int r, uint16_t* dX, int64_t T,
                     int64_t N, int64_t K, const ProjArgs& g, uint64_t* words, hipStream_t stream) {
    TileArgs a{};
    a.w = w;
    a.act = dY;
    a.ld_act = N;
    a.lt = nullptr;
    a.la = A;
    a.ld_la = K;
    a.r_la = r;
    a.rp = 64;
    a.out = dX;
    a.T = T;
    a.N = N;
    a.K = K;
    // the projection workgroups: G = s dY B of one 16-token block each, the
    // caller's layouts of it (G^T, U^T) and the raw sums as tagged words
    a.proj = g;
    a.proj.out_b = nullptr;
    a.proj.uword = words;
    a.proj.token = next_token();
    a.proj.tag = static_cast<uint32_t>(a.proj.token % 0xFFFFFFFFull) + 1u;
    a.r_u = r;
    a.s_u = g.alpha_b;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return set_error(QL_ERR_HIP, "dequant GEMM: capture query");
    if (cs != hipStreamCaptureStatusNone) {
        a.epoch = words + static_cast<size_t>(T) * r;
        launch_advance_epoch(words + static_cast<size_t>(T) * r, stream);
    }
    const char* e = std::getenv("QLORA_NF4_GEMM_SPIN");
    a.spin = e ? std::atoi(e) : (1 << 14);
    return launch_tiles<true>(a, nullptr, QL_KERNEL_GEMM_DX, "dequant GEMM dX", stream, static_cast<int>(ceil_div(T, 16)));
}

size_t gemm_fwd_u_words(int64_t T, int r) { return static_cast<size_t>(T) * r + 1; }  // + the epoch word

int launch_gemm_fwd_u(const NF4Dev& w, const uint16_t* X, const uint16_t* A, const uint16_t* B, int r, float scale,
                      uint16_t* Y, float* U_out, int64_t T, int64_t N, int64_t K, uint64_t* words, hipStream_t stream) {
    TileArgs a{};
    a.w = w;
    a.act = X;
    a.ld_act = K;
    a.lt = nullptr;
    a.la = B;
    a.ld_la = r;
    a.r_la = r;
    a.rp = 64;
    a.out = Y;
    a.T = T;
    a.N = N;
    a.K = K;
    // the projection workgroups: U = X A^T of one 16-token block each,
    // fp32 U for the caller and the raw sums as words tagged for this launch
    ProjArgs& pj = a.proj;
    pj.proj = 1;
    pj.P = X;
    pj.ldp = K;
    pj.Q = A;
    pj.ldq = K;
    pj.rq = r;
    pj.T = T;
    pj.kred = K;
    pj.alpha_f = 1.0f;
    pj.out_f = U_out;
    pj.ld_f = r;
    pj.alpha_b = scale;
    pj.uword = words;
    pj.token = next_token();
    // a fresh tag per launch, so words left in the workspace by earlier
    // launches never pass for this one's; a captured launch (replayed with
    // this tag) also mixes in the epoch word after the words, which a kernel
    // recorded before it advances at every replay
    pj.tag = static_cast<uint32_t>(pj.token % 0xFFFFFFFFull) + 1u;
    a.r_u = r;
    a.s_u = scale;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return set_error(QL_ERR_HIP, "dequant GEMM: capture query");
    if (cs != hipStreamCaptureStatusNone) {
        a.epoch = words + static_cast<size_t>(T) * r;
        launch_advance_epoch(words + static_cast<size_t>(T) * r, stream);
    }
    // QLORA_NF4_GEMM_SPIN=n: loads of the words before a tile forms U
    // itself (a negative n: at once, without reading the words)
    const char* e = std::getenv("QLORA_NF4_GEMM_SPIN");
    a.spin = e ? std::atoi(e) : (1 << 14);
    return launch_tiles<false>(a, nullptr, QL_KERNEL_GEMM_FWD, "dequant GEMM forward", stream,
                               static_cast<int>(ceil_div(T, 16)));
}

int launch_gemm_dx(const NF4Dev& w, const uint16_t* dY, const uint16_t* Gp, const uint16_t* A, int r, int rp,
                   uint16_t* dX, int64_t T, int64_t N, int64_t K, float* split_ws, hipStream_t stream) {
    TileArgs a{};
    a.w = w;
    a.act = dY;
    a.ld_act = N;
    a.lt = Gp;
    a.la = A;
    a.ld_la = K;
    a.r_la = r;
    a.rp = rp;
    a.out = dX;
    a.T = T;
    a.N = N;
    a.K = K;
    return launch_tiles<true>(a, split_ws, QL_KERNEL_GEMM_DX, "dequant GEMM dX", stream);
}

namespace {

// Rows of a grouped forward's row tiles (256 rows a tile, per layer).
int64_t fwd_group_rows(const int64_t* N, int ng) {
    int64_t rows = 0;
    for (int i = 0; i < ng; ++i) rows += ceil_div(N[i], 256) * 256;
    return rows;
}

}  // namespace

// One launch when its plan costs less than the layers' own, or up to 5 %
// more when it needs no reduction split and some layer's own plan does:
// the partials' round trip weighs more than the plan's split penalty says
// (q/k/v at T = 2048: 128 against 125 units, measured 17 % faster).
bool gemm_fwd_group_pays(const int64_t* N, int ng, int64_t T, int64_t K) {
    if (ng < 2 || ng > kGemmMaxGroup) return false;
    const GemmPlan g = plan_gemm(fwd_group_rows(N, ng), T, K);
    if (g.tile != 256) return false;
    double sep = 0.0;
    bool split = false;
    for (int i = 0; i < ng; ++i) {
        const GemmPlan pl = plan_gemm(N[i], T, K);
        sep += pl.cost;
        split = split || pl.splits > 1;
    }
    return g.cost < sep || (g.splits == 1 && split && g.cost <= 1.05 * sep);
}

size_t gemm_fwd_group_split_bytes(const int64_t* N, int ng, int64_t T, int64_t K) {
    const GemmPlan g = plan_gemm(fwd_group_rows(N, ng), T, K);
    int64_t ncat = 0;
    for (int i = 0; i < ng; ++i) ncat += N[i];
    return g.splits > 1 ? static_cast<size_t>(g.splits) * T * ncat * sizeof(float) : 0;
}

int launch_gemm_fwd_group(const GemmLayer* layers, int ng, const uint16_t* X, int r, int rp, int64_t T, int64_t K,
                          float* split_ws, hipStream_t stream) {
    if (ng < 1 || ng > kGemmMaxGroup) return set_error(QL_ERR_SHAPE, "grouped forward: %d layers", ng);
    TileArgs a{};
    a.w = layers[0].w;  // the format; every layer has the same
    a.act = X;
    a.ld_act = K;
    a.ng = ng;
    a.gtile[0] = 0;
    a.gcol[0] = 0;
    int64_t N[kGemmMaxGroup];
    for (int i = 0; i < ng; ++i) {
        a.gl[i] = layers[i];
        N[i] = layers[i].N;
        a.gtile[i + 1] = a.gtile[i] + static_cast<int>(ceil_div(layers[i].N, 256));
        a.gcol[i + 1] = a.gcol[i] + layers[i].N;
    }
    a.ld_la = r;
    a.r_la = r;
    a.rp = rp;
    a.T = T;
    a.N = fwd_group_rows(N, ng);
    a.K = K;
    return launch_tiles<false, true>(a, split_ws, QL_KERNEL_GEMM_FWD, "grouped dequant GEMM forward", stream);
}

int64_t gemm_group_steps(const int64_t* N, int ng) {
    int64_t st = 0;
    for (int i = 0; i < ng; ++i) st += ceil_div(N[i], kStep);
    return st;
}

int launch_gemm_dx_group(const GemmLayer* layers, int ng, int r, int rp, uint16_t* dX, int64_t T, int64_t K,
                         float* split_ws, hipStream_t stream) {
    if (ng < 1 || ng > kGemmMaxGroup) return set_error(QL_ERR_SHAPE, "grouped dX: %d layers", ng);
    TileArgs a{};
    a.w = layers[0].w;  // the format; every layer has the same
    a.ng = ng;
    a.gstep[0] = 0;
    for (int i = 0; i < ng; ++i) {
        a.gl[i] = layers[i];
        a.gstep[i + 1] = a.gstep[i] + static_cast<int>(ceil_div(layers[i].N, kStep));
    }
    a.ld_la = K;
    a.r_la = r;
    a.rp = rp;
    a.out = dX;
    a.T = T;
    a.K = K;
    return launch_tiles<true, true>(a, split_ws, QL_KERNEL_GEMM_DX, "grouped dequant GEMM dX", stream);
}

}  // namespace qlnf4
