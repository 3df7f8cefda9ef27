// The rank-r projection V[t][j] = sum_k P[t][k] Q[j][k] of one 16-token block
// with its operands staged in LDS by direct-to-LDS loads (gfx950, bf16 MFMA
// 16x16x32): shared by the projection kernel and by the dequant GEMM
// forward, whose first workgroups can compute U for the GEMM's tiles.
#pragma once

#include <algorithm>

#include "common.h"
#include "internal.h"
#include "mm_common.h"

namespace qlnf4 {

// ---------------------------------------------------------------------------
// The same projection with the operands staged in LDS by direct-to-LDS loads
// (global_load_lds_dwordx4): every load instruction then covers whole
// 128-byte lines (8 rows x 128 bytes of P or of A, or 1 KiB of consecutive
// rows of B), where register loads in MFMA operand order touch 32 half lines
// each. A wave runs its 64-wide reduction steps w, w + NW, ... through a ring
// of three LDS slots: while it multiplies one step, the next two are in
// flight. P and A tiles keep 16-byte chunk c of row r at c ^ swz(r), so the
// 16 lanes reading one chunk column hit every bank twice at most; B tiles are
// read column-wise with transposing LDS loads.
// Used for every A-like Q, and for B-like Q when rq % 4 == 0.
// ---------------------------------------------------------------------------
#define QL_LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ int swz8(int r) { return (r ^ (r >> 3)) & 7; }

// s_waitcnt vmcnt(N), leaving the LDS and export counters alone. LDS writes
// of direct-to-LDS loads are complete once the issuing wave's vmcnt has
// dropped past them; the compiler does not insert this wait by itself.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int RT>
struct ProjDma {
    static constexpr int NW = RT <= 2 ? 8 : (RT == 4 ? 4 : 2);  // waves: three slots per wave fit in LDS
    static constexpr int PS = 16 * 64;                           // P slot: 16 tokens x 64 k
    static constexpr int QS = 16 * RT * 64;                      // Q slot: 16 RT rows x 64 k, or 64 rows of B
};

// LDS of one projection workgroup: three ring slots of P and of Q per wave,
// the waves' partial sums, and the last-split flag. The projection kernel
// declares its own arrays; a kernel that runs projection workgroups inside a
// larger launch points these into its own LDS.
template <int RT>
struct ProjLds {
    uint16_t (*P[3])[ProjDma<RT>::PS];  // [NW][PS] each
    uint16_t (*Q[3])[ProjDma<RT>::QS];  // [NW][QS] each
    float (*red)[16][16];               // [NW][16][16]
    int* last;
};

template <int RT, bool QCOLS>
__device__ __forceinline__ void proj_dma_block(const ProjArgs& p, int bx, int split, int nsplit, const ProjLds<RT>& L) {
    using D = ProjDma<RT>;
    constexpr int NW = D::NW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, g = lane >> 4;
    const int64_t t0 = static_cast<int64_t>(bx) * 16;

    if (p.proj) {
        // this split's 64-wide steps [sbeg, send); wave w takes sbeg + w, sbeg + w + NW, ...
        const int64_t nst = ceil_div(p.kred, 64);
        const int64_t sbeg = nst * split / nsplit, send = nst * (split + 1) / nsplit;
        const int64_t my = send - sbeg > wave ? ceil_div(send - sbeg - wave, NW) : 0;  // this wave's steps
        const int64_t qlast = p.kred * p.rq - 8;

        auto issue = [&](int64_t s, uint16_t* sp, uint16_t* sq) {
            const int64_t k0 = (sbeg + wave + NW * s) * 64;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = 8 * i + (lane >> 3);
                const int c = (lane & 7) ^ swz8(row);
                const int64_t t = std::min<int64_t>(t0 + row, p.T - 1);
                const int64_t col = std::min<int64_t>(k0 + 8 * c, p.kred - 8);
                __builtin_amdgcn_global_load_lds(p.P + t * p.ldp + col, (QL_LDS_AS void*)(sp + 512 * i), 16, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 2 * RT; ++i) {
                if constexpr (!QCOLS) {
                    const int row = 8 * i + (lane >> 3);
                    const int c = (lane & 7) ^ swz8(row);
                    const int64_t j = std::min(row, p.rq - 1);
                    const int64_t col = std::min<int64_t>(k0 + 8 * c, p.kred - 8);
                    __builtin_amdgcn_global_load_lds(p.Q + j * p.ldq + col, (QL_LDS_AS void*)(sq + 512 * i), 16, 0,
                                                     0);
                } else {  // rows k0 .. k0+63 of B are one run of 64 rq values
                    const int64_t e = std::min<int64_t>(k0 * p.rq + 512 * i + 8 * lane, qlast);
                    __builtin_amdgcn_global_load_lds(p.Q + e, (QL_LDS_AS void*)(sq + 512 * i), 16, 0, 0);
                }
            }
        };

        f32x4 acc[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto compute = [&](int64_t s, const uint16_t* sp, const uint16_t* sq) {
            const int64_t k0 = (sbeg + wave + NW * s) * 64;
            const bool partial = k0 + 64 > p.kred;  // wave-uniform
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 4 * h + g;
                uint4 pv = *reinterpret_cast<const uint4*>(sp + li * 64 + 8 * (c ^ swz8(li)));
                if (partial && k0 + 8 * c >= p.kred) pv = make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    bf16x8_t qo;
                    if constexpr (!QCOLS) {
                        const int row = 16 * t + li;
                        qo = as_bf16x8(*reinterpret_cast<const uint4*>(sq + row * 64 + 8 * (c ^ swz8(row))));
                    } else {
                        qo = lds_col8(sq, p.rq, 32 * h + 8 * g, 16 * t, li);
                    }
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qo, as_bf16x8(pv), acc[t], 0, 0, 0);
                }
            }
        };

        // wait for the loads of step s; those of the (at most two) later steps
        // already issued may stay in flight
        constexpr int DPS = 2 + 2 * RT;  // load instructions per step
        auto wait_step = [&](int64_t s) {
            if (s + 2 < my)
                wait_vmcnt<2 * DPS>();
            else if (s + 1 < my)
                wait_vmcnt<DPS>();
            else
                wait_vmcnt<0>();
        };
        if (0 < my) issue(0, L.P[0][wave], L.Q[0][wave]);
        if (1 < my) issue(1, L.P[1][wave], L.Q[1][wave]);
        if (2 < my) issue(2, L.P[2][wave], L.Q[2][wave]);
        for (int64_t s = 0; s < my; s += 3) {
            wait_step(s);
            compute(s, L.P[0][wave], L.Q[0][wave]);
            if (s + 3 < my) {
                wave_lds_sync();  // slot 0 has been read
                issue(s + 3, L.P[0][wave], L.Q[0][wave]);
            }
            if (s + 1 < my) {
                wait_step(s + 1);
                compute(s + 1, L.P[1][wave], L.Q[1][wave]);
                if (s + 4 < my) {
                    wave_lds_sync();
                    issue(s + 4, L.P[1][wave], L.Q[1][wave]);
                }
            }
            if (s + 2 < my) {
                wait_step(s + 2);
                compute(s + 2, L.P[2][wave], L.Q[2][wave]);
                if (s + 5 < my) {
                    wave_lds_sync();
                    issue(s + 5, L.P[2][wave], L.Q[2][wave]);
                }
            }
        }

        // every layout the consumers read, from the final value v of
        // (rank j, token t)
        auto emit = [&](int j, int64_t t, float v) {
            if (p.out_f != nullptr && j < p.rq) p.out_f[t * p.ld_f + j] = p.alpha_f * v;
            if (p.uword != nullptr && j < p.rq)  // device scope: read by other workgroups of the launch
                __hip_atomic_store(p.uword + t * p.rq + j, (uint64_t{p.tag} << 32) | __float_as_uint(v),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint16_t hb = to_bf16_bits(j < p.rq ? p.alpha_b * v : 0.0f);
            if (p.out_b != nullptr && j < p.ld_b) p.out_b[t * p.ld_b + j] = hb;
            if (p.out_bt != nullptr && j < p.rows_bt) p.out_bt[j * p.ld_bt + t] = hb;
        };
        // with splits, this split's partial of rank tile rt, element
        // e = 16 jl + tl, goes to part[((bx nsplit + split) RT + rt) 256 + e]
        float* const mypart = p.part + ((static_cast<int64_t>(bx) * nsplit + split) * RT) * 256;

        // D[j = 4 g + rr][token li] of each rank tile; fixed-order sum of the waves
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (rt > 0) __syncthreads();
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) L.red[wave][4 * g + rr][li] = acc[rt][rr];
            __syncthreads();
            for (int e = tid; e < 256; e += 64 * NW) {
                const int jl = e >> 4, tl = e & 15;
                float v = 0.0f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) v += L.red[ww][jl][tl];
                if (nsplit > 1) {
                    // device-scope store: read back by another workgroup,
                    // possibly on another XCD
                    __hip_atomic_store(mypart + rt * 256 + e, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    continue;
                }
                const int64_t t = t0 + tl;
                if (t < p.T) emit(16 * rt + jl, t, v);
            }
        }
        if (nsplit > 1) {
            // The last split of this token block to arrive (a per-block
            // counter tagged with the launch token; a counter carrying another
            // token counts as zero) adds the partials in split order, so the
            // result does not depend on the arrival order. The last arrival
            // leaves the count at zero, so a launch replayed with the same
            // token (a captured graph) starts from zero as well.
            // Ordering: the partials are written and read only by agent-scope
            // atomic stores and loads, which are performed at the device's
            // coherence point, not in an XCD's own cache. Every thread waits for
            // its stores to complete (vmcnt counts per wave) before the barrier
            // and thread 0's count; the last split's loads are issued only after
            // the count has returned (barrier, branch on the last flag). So no cache
            // write-back or invalidation is needed, which is all an
            // acquire-release exchange would add here: one L2 write-back per
            // workgroup, measured at 45 us per benchmark step.
            __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
            __syncthreads();
            if (tid == 0) {
                uint64_t* c = p.cnt + bx;
                uint64_t old = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                uint64_t nv;
                int arrived;
                do {
                    arrived = static_cast<int>(((old >> 8) == p.token) ? (old & 0xFFu) : 0u) + 1;
                    nv = (p.token << 8) | static_cast<uint64_t>(arrived == nsplit ? 0 : arrived);
                } while (!__hip_atomic_compare_exchange_strong(c, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT));
                *L.last = arrived == nsplit;
            }
            __syncthreads();
            if (*L.last) {
                const float* const blockpart = p.part + static_cast<int64_t>(bx) * nsplit * RT * 256;
                for (int e = tid; e < RT * 256; e += 64 * NW) {
                    float v = 0.0f;
                    for (int sp = 0; sp < nsplit; ++sp)
                        v += __hip_atomic_load(blockpart + sp * RT * 256 + e, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    const int rt = e >> 8, jl = (e >> 4) & 15, tl = e & 15;
                    const int64_t t = t0 + tl;
                    if (t < p.T) emit(16 * rt + jl, t, v);
                }
            }
        }
        if (p.out_b != nullptr && split == 0) {  // zero columns past the rank tiles
            for (int e = tid; e < 16 * (p.ld_b - 16 * RT); e += 64 * NW) {
                const int64_t tt = t0 + (e & 15);
                if (tt < p.T) p.out_b[tt * p.ld_b + 16 * RT + (e >> 4)] = 0;
            }
        }
    }
    if (p.Ut != nullptr && split == 0) {
        for (int e = tid; e < 16 * p.rows_ut; e += 64 * NW) {
            const int j = e >> 4;
            const int64_t tt = t0 + (e & 15);
            if (tt < p.T) p.Ut[j * p.ld_ut + tt] = to_bf16_bits(j < p.ru ? p.Usrc[tt * p.ru + j] : 0.0f);
        }
    }
}


}  // namespace qlnf4
