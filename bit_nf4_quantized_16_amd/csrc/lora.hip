// LoRA-side kernels of the frozen-base linear layer (gfx950, bf16 MFMA): the
// rank-r projections and the adapter gradients.
//
//   U = X A^T              forward (apxml.com "量化 LoRA (QLoRA) 与 4 位训练":
//                          h = dequant(W_NF4) x + B A x)
//   G = s dY B             backward, the rank-r half of dX = dY W' + G A
//   dA = G^T X, dB = s dY^T U
//                          aivaro.ru "Как работает QLoRA", §2: B in R^{d x r},
//                          A in R^{r x k}; the frozen 4-bit base gets no
//                          gradient, only the adapters do
//
// Each product is one launch: the projection kernel writes every layout its
// consumers read (fp32 U for the caller, bf16 s U / G padded for the GEMM
// epilogues, bf16 G^T and U^T for the gradient kernel), and the gradient
// kernel computes dA and dB in one grid.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <chrono>

#include "common.h"
#include "internal.h"
#include "mm_common.h"
#include "proj_dma.h"

namespace qlnf4 {

// ===========================================================================
// Projection: V[t][j] = sum_k P[t][k] Q[j][k], j < rq <= 128.
// Q is either rows of the reduction (A [r, K]: Q[j][k] = A[j][k]) or its
// transpose in memory (B [N, r]: Q[j][n] = B[n][j]).
// A workgroup owns 16 tokens; its eight waves take the 128-wide reduction
// steps w, w+8, ... In a step, lane (i = l%16, g = l/16) reads 32 values of
// P row t0+i (k = 128 st + 32 g ...) as four MFMA B operands, and for every
// 16-row tile of the rank the matching A operands: straight from A's rows,
// or, for B, through a wave-private LDS tile of the step's 128 rows of B read
// back with transposing LDS loads. All loads of a pass are issued before any
// arithmetic; the eight waves' sums are added in a fixed order.
// ===========================================================================
constexpr int kProjWaves = 8;

template <int RT>
constexpr int proj_steps() {
    return RT <= 1 ? 4 : (RT == 2 ? 2 : 1);
}

template <int RT, bool QCOLS>
__global__ __launch_bounds__(512) void lora_proj_kernel(ProjArgs p) {
    constexpr int S = proj_steps<RT>();
    __shared__ float red[kProjWaves][16][16];
    __shared__ __attribute__((aligned(16))) uint16_t qtile[QCOLS ? kProjWaves : 1][QCOLS ? 128 * 16 : 8];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, g = lane >> 4;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;

    if (p.proj) {
        const int64_t ksteps = ceil_div(p.kred, 128);
        const uint16_t* prow = p.P + std::min<int64_t>(t0 + li, p.T - 1) * p.ldp;
        f32x4 acc[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int64_t base = 0; base < ksteps; base += kProjWaves * S) {
            uint4 pv[S][4];
            uint4 qv[S][RT][4];
#pragma unroll
            for (int i = 0; i < S; ++i) {
                const int64_t st = std::min<int64_t>(base + wave + kProjWaves * i, ksteps - 1);
                const int64_t k = st * 128 + 32 * g;
#pragma unroll
                for (int m = 0; m < 4; ++m)  // the reduction length is a multiple of 8
                    pv[i][m] = *reinterpret_cast<const uint4*>(prow + std::min<int64_t>(k + 8 * m, p.kred - 8));
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    if constexpr (!QCOLS) {
                        const uint16_t* qrow = p.Q + std::min(16 * t + li, p.rq - 1) * p.ldq;
#pragma unroll
                        for (int m = 0; m < 4; ++m)
                            qv[i][t][m] =
                                *reinterpret_cast<const uint4*>(qrow + std::min<int64_t>(k + 8 * m, p.kred - 8));
                    } else {
                        // 128 rows x 16 columns of B: 256 pieces of 8, four per lane
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int q = lane + 64 * u;
                            const int64_t n = std::min<int64_t>(st * 128 + (q >> 1), p.kred - 1);
                            qv[i][t][u] = load_cols8(p.Q + n * p.rq, 16 * t + 8 * (q & 1), p.rq);
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < S; ++i) {
                const int64_t st = base + wave + kProjWaves * i;
                if (st >= ksteps) break;
                if (st * 128 + 128 > p.kred) {  // last, partial step (wave-uniform): zero P past the end
                    const int64_t k = st * 128 + 32 * g;
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        if (k + 8 * m >= p.kred) pv[i][m] = make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    bf16x8_t qo[4];
                    if constexpr (!QCOLS) {
#pragma unroll
                        for (int m = 0; m < 4; ++m) qo[m] = as_bf16x8(qv[i][t][m]);
                    } else {
                        uint16_t* tile = qtile[wave];
                        wave_lds_sync();  // the previous tile's reads are done
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int q = lane + 64 * u;
                            *reinterpret_cast<uint4*>(tile + (q >> 1) * 16 + 8 * (q & 1)) = qv[i][t][u];
                        }
                        wave_lds_sync();
#pragma unroll
                        for (int m = 0; m < 4; ++m) qo[m] = lds_col8(tile, 16, 32 * g + 8 * m, 0, li);
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qo[m], as_bf16x8(pv[i][m]), acc[t], 0, 0, 0);
                }
            }
        }
        // D[j = 4 g + rr][token li] of each rank tile; fixed-order sum of the waves
        const int jl = tid >> 4, tl = tid & 15;
        const int64_t t = t0 + tl;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (rt > 0) __syncthreads();
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) red[wave][4 * g + rr][li] = acc[rt][rr];
            __syncthreads();
            if (tid < 256 && t < p.T) {
                float v = 0.0f;
#pragma unroll
                for (int ww = 0; ww < kProjWaves; ++ww) v += red[ww][jl][tl];
                const int j = 16 * rt + jl;
                if (p.out_f != nullptr && j < p.rq) p.out_f[t * p.ld_f + j] = p.alpha_f * v;
                const uint16_t hb = to_bf16_bits(j < p.rq ? p.alpha_b * v : 0.0f);
                if (p.out_b != nullptr && j < p.ld_b) p.out_b[t * p.ld_b + j] = hb;
                if (p.out_bt != nullptr && j < p.rows_bt) p.out_bt[j * p.ld_bt + t] = hb;
            }
        }
        if (p.out_b != nullptr) {  // zero columns past the rank tiles
            for (int e = tid; e < 16 * (p.ld_b - 16 * RT); e += 512) {
                const int64_t tt = t0 + (e & 15);
                if (tt < p.T) p.out_b[tt * p.ld_b + 16 * RT + (e >> 4)] = 0;
            }
        }
    }
    // side job: Ut[j][t] = bf16(U[t][j]) for the tokens of this workgroup
    if (p.Ut != nullptr) {
        for (int e = tid; e < 16 * p.rows_ut; e += 512) {
            const int j = e >> 4;
            const int64_t tt = t0 + (e & 15);
            if (tt < p.T) p.Ut[j * p.ld_ut + tt] = to_bf16_bits(j < p.ru ? p.Usrc[tt * p.ru + j] : 0.0f);
        }
    }
}

// The projection with the operands staged in LDS by direct-to-LDS loads
// (proj_dma.h): one workgroup per 16-token block and split.
template <int RT, bool QCOLS>
__global__ __launch_bounds__(64 * ProjDma<RT>::NW) void lora_proj_dma_kernel(ProjArgs p) {
    using D = ProjDma<RT>;
    constexpr int NW = D::NW;
    __shared__ __attribute__((aligned(16))) uint16_t sP0[NW][D::PS];
    __shared__ __attribute__((aligned(16))) uint16_t sP1[NW][D::PS];
    __shared__ __attribute__((aligned(16))) uint16_t sP2[NW][D::PS];
    __shared__ __attribute__((aligned(16))) uint16_t sQ0[NW][D::QS];
    __shared__ __attribute__((aligned(16))) uint16_t sQ1[NW][D::QS];
    __shared__ __attribute__((aligned(16))) uint16_t sQ2[NW][D::QS];
    __shared__ float red[NW][16][16];
    __shared__ int s_last;
    const ProjLds<RT> L{{sP0, sP1, sP2}, {sQ0, sQ1, sQ2}, red, &s_last};
    proj_dma_block<RT, QCOLS>(p, static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y),
                              static_cast<int>(gridDim.y), L);
}

// A fresh 56-bit token per launch, so that split counters left in a reused
// workspace by earlier launches count as zero (a launch that ends normally
// leaves its counters at zero anyway; the token covers a workspace that held
// anything else before).
uint64_t next_token() {
    static std::atomic<uint64_t> ctr{
        (static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count()) * 0x9E3779B97F4A7C15ull) >>
        8};
    return ctr.fetch_add(1) & ((1ull << 56) - 1);
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

int proj_rt(int rq) {
    const int tiles = (rq + 15) / 16;
    return tiles <= 2 ? tiles : (tiles <= 4 ? 4 : 8);
}

int proj_waves(int rt) { return rt == 1 ? ProjDma<1>::NW : rt == 2 ? ProjDma<2>::NW : rt == 4 ? ProjDma<4>::NW : ProjDma<8>::NW; }

// Workgroups per 16-token block: enough blocks to cover the CUs, each
// split keeping at least five steps per wave (with fewer, splitting
// measured slower than not: the partial-sum hand-off costs a few memory
// round trips); at most 8, and 1 for the register-path kernel.
// QLORA_NF4_PROJ_SPLITS=n forces n (at most 32, at least one step per wave).
int proj_splits(int64_t T, int rq, int64_t kred, bool q_cols) {
    if (q_cols && rq % 4 != 0) return 1;
    const int64_t nblk = ceil_div(T, 16);
    const int64_t nst = ceil_div(kred, 64);
    const int nw = proj_waves(proj_rt(rq));
    int64_t s = cu_count() / nblk;
    s = std::min<int64_t>(s, nst / (5 * nw));
    s = std::max<int64_t>(1, std::min<int64_t>(s, 8));
    if (const char* e = std::getenv("QLORA_NF4_PROJ_SPLITS"))
        s = std::max<int64_t>(1, std::min<int64_t>({static_cast<int64_t>(std::atoi(e)), 32, nst / nw}));
    return static_cast<int>(s);
}

}  // namespace

int lora_proj_splits(int64_t T, int rq, int64_t kred, bool q_cols) { return proj_splits(T, rq, kred, q_cols); }

size_t lora_proj_ws_bytes(int64_t T, int rq, int64_t kred, bool q_cols) {
    if (T <= 0 || rq < 1) return 0;
    const int s = proj_splits(T, rq, kred, q_cols);
    if (s == 1) return 0;
    const int64_t nblk = ceil_div(T, 16);
    const size_t part = static_cast<size_t>(nblk) * s * proj_rt(rq) * 256 * sizeof(float);
    return (part + 255) / 256 * 256 + static_cast<size_t>(nblk) * sizeof(uint64_t);
}

template <bool QCOLS>
static void launch_proj_dma_rt(int rt, const ProjArgs& a, int splits, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(ceil_div(a.T, 16)), static_cast<uint32_t>(splits));
    switch (rt) {
        case 1:
            hipLaunchKernelGGL((lora_proj_dma_kernel<1, QCOLS>), grid, dim3(64 * ProjDma<1>::NW), 0, stream, a);
            break;
        case 2:
            hipLaunchKernelGGL((lora_proj_dma_kernel<2, QCOLS>), grid, dim3(64 * ProjDma<2>::NW), 0, stream, a);
            break;
        case 4:
            hipLaunchKernelGGL((lora_proj_dma_kernel<4, QCOLS>), grid, dim3(64 * ProjDma<4>::NW), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL((lora_proj_dma_kernel<8, QCOLS>), grid, dim3(64 * ProjDma<8>::NW), 0, stream, a);
            break;
    }
}

template <bool QCOLS>
static void launch_proj_rt(int rt, const ProjArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(ceil_div(a.T, 16))), block(64 * kProjWaves);
    switch (rt) {
        case 1: hipLaunchKernelGGL((lora_proj_kernel<1, QCOLS>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((lora_proj_kernel<2, QCOLS>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((lora_proj_kernel<4, QCOLS>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((lora_proj_kernel<8, QCOLS>), grid, block, 0, stream, a); break;
    }
}

int launch_lora_proj(const ProjArgs& args, bool q_cols, void* ws, hipStream_t stream) {
    ProjArgs a = args;
    if (a.rq < 1 || a.rq > QL_MAX_RANK) return set_error(QL_ERR_SHAPE, "LoRA projection: rank %d out of range", a.rq);
    if (a.T <= 0) return QL_OK;
    const int rt = proj_rt(a.rq);
    if (a.out_b != nullptr && a.ld_b < a.rq)
        return set_error(QL_ERR_SHAPE, "LoRA projection: bf16 output narrower than the rank");
    const int splits = a.proj ? proj_splits(a.T, a.rq, a.kred, q_cols) : 1;
    a.part = nullptr;
    a.cnt = nullptr;
    a.token = next_token();
    if (splits > 1) {
        if (ws == nullptr) return set_error(QL_ERR_WORKSPACE, "LoRA projection: split workspace missing");
        const int64_t nblk = ceil_div(a.T, 16);
        const size_t part = static_cast<size_t>(nblk) * splits * rt * 256 * sizeof(float);
        a.part = static_cast<float*>(ws);
        a.cnt = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + (part + 255) / 256 * 256);
    }
    if (!q_cols)
        launch_proj_dma_rt<false>(rt, a, splits, stream);
    else if (a.rq % 4 == 0)
        launch_proj_dma_rt<true>(rt, a, splits, stream);
    else
        launch_proj_rt<true>(rt, a, stream);
    return check_launch("LoRA projection");
}

// ===========================================================================
// Adapter gradients, reductions over tokens:
//   out[j][c] (dA) or out[c][j] (dB) = scale * sum_t Vt[j][t] M[t][c]
// with M = X, Vt = G^T for dA and M = dY, Vt = U^T, scale = s for dB. One
// grid holds both problems: workgroups [0, nblk0) take 64-column blocks of
// the first, the rest those of the second. A workgroup's eight waves take
// 32-token chunks in turn; each wave stages its chunk of M in a private LDS
// tile and reads it back column-wise with transposing LDS loads (8
// consecutive tokens of one column per lane, the MFMA B operand); the A
// operand is a 16-byte load from Vt. With one token split the workgroup
// writes the gradient itself (fixed-order sum of the waves); with several,
// fp32 partials go to the workspace and a second kernel adds them in order.
// ===========================================================================
int lora_grad_rp(int r) { return (r + 15) / 16 * 16; }
int64_t lora_vt_ld(int64_t T) { return ceil_div(T, 8) * 8; }

constexpr int kGradCols = 64;  // columns of M per workgroup
constexpr int kGradRows = 32;  // token rows per MFMA step
constexpr int kGradWaves = 8;  // waves per workgroup, taking chunks in turn
constexpr int kGradLd = kGradCols + 8;

int lora_grad_splits(int64_t T, int64_t cols_total) {
    // one split (no second kernel) while a workgroup's token loop stays short,
    // and when neither gradient is asked for (no columns)
    if (T <= 2048 || cols_total <= 0) return 1;
    const int64_t col_blocks = ceil_div(cols_total, kGradCols);
    int64_t s = ceil_div(512, col_blocks);
    const int64_t max_s = ceil_div(T, kGradWaves * kGradRows);
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    return static_cast<int>(s);
}

template <int RT>
__global__ __launch_bounds__(64 * kGradWaves) void lora_grads_kernel(GradArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sm[kGradWaves][kGradRows * kGradLd];
    __shared__ float red[kGradWaves][16][kGradCols];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, g = lane >> 4;
    const bool second = static_cast<int>(blockIdx.x) >= a.nblk0;
    const GradProblem& pb = second ? a.pb[1] : a.pb[0];
    const uint16_t* __restrict__ M = pb.M;
    const uint16_t* __restrict__ Vt = pb.Vt;
    const int64_t C = pb.C, ldm = pb.ldm, ldv = pb.ldv;
    const int64_t c0 = static_cast<int64_t>(second ? blockIdx.x - a.nblk0 : blockIdx.x) * kGradCols;
    const int ts = blockIdx.y;
    const int64_t tb = ts * a.t_per;
    const int64_t te = std::min<int64_t>(tb + a.t_per, a.T);
    f32x4 acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rt][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint16_t* tile = sm[wave];
    auto load_chunk = [&](int64_t t, uint4 (&v)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (lane >> 3) + 8 * i;
            const int64_t c = c0 + 8 * (lane & 7);
            v[i] = (t + row < te && c < C) ? *reinterpret_cast<const uint4*>(M + (t + row) * ldm + c)
                                           : make_uint4(0, 0, 0, 0);
        }
    };
    uint4 cur[4];
    int64_t t = tb + kGradRows * wave;
    if (t < te) load_chunk(t, cur);
    for (; t < te; t += kGradWaves * kGradRows) {
        uint4 nxt[4];
        const int64_t tn = t + kGradWaves * kGradRows;
        if (tn < te) load_chunk(tn, nxt);
        wave_lds_sync();  // the previous chunk's reads are done
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(tile + ((lane >> 3) + 8 * i) * kGradLd + 8 * (lane & 7)) = cur[i];
        wave_lds_sync();
        bf16x8_t bv[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) bv[cb] = lds_col8(tile, kGradLd, 8 * g, 16 * cb, li);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int64_t tt = t + 8 * g;
            const uint16_t* vrow = Vt + (16 * rt + li) * ldv;
            uint4 av;
            if (tt + 8 <= te) {
                av = *reinterpret_cast<const uint4*>(vrow + tt);
            } else {  // last partial chunk of the split: element by element
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = (tt + e < te) ? vrow[tt + e] : 0u;
                av = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
            }
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                acc[rt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), bv[cb], acc[rt][cb], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
    }
    const bool direct = gridDim.y == 1;
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][4 * g + r][16 * cb + li] = acc[rt][cb][r];
        __syncthreads();
        for (int e = tid; e < 16 * kGradCols; e += 64 * kGradWaves) {
            const int jl = e / kGradCols, cl = e % kGradCols;
            const int j = 16 * rt + jl;
            const int64_t c = c0 + cl;
            if (c >= C) continue;
            float v = red[0][jl][cl];
#pragma unroll
            for (int ww = 1; ww < kGradWaves; ++ww) v += red[ww][jl][cl];
            if (direct) {
                if (j < a.r) {
                    const int64_t idx = pb.layout_jc ? j * C + c : c * a.r + j;
                    const float o = pb.scale * v;
                    pb.out[idx] = a.accumulate ? pb.out[idx] + o : o;
                }
            } else {
                pb.part[(static_cast<int64_t>(ts) * RT * 16 + j) * C + c] = v;
            }
        }
        __syncthreads();
    }
}

// sum of the token splits of both problems, in split order
__global__ void lora_grads_final_kernel(GradArgs a, int splits, int rpad) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t n0 = static_cast<int64_t>(a.r) * a.pb[0].C;
    const int64_t n1 = static_cast<int64_t>(a.r) * a.pb[1].C;
    if (idx >= n0 + n1) return;
    const bool second = idx >= n0;
    const GradProblem& pb = second ? a.pb[1] : a.pb[0];
    const int64_t e = second ? idx - n0 : idx;
    const int64_t C = pb.C;
    int64_t j, c;
    if (pb.layout_jc) {
        j = e / C;
        c = e % C;
    } else {
        c = e / a.r;
        j = e % a.r;
    }
    float s = 0.0f;
    for (int ts = 0; ts < splits; ++ts) s += pb.part[(static_cast<int64_t>(ts) * rpad + j) * C + c];
    const float v = pb.scale * s;
    pb.out[e] = a.accumulate ? pb.out[e] + v : v;
}

size_t lora_grads_part_bytes(int64_t T, int64_t C0, int64_t C1, int r) {
    const int sp = lora_grad_splits(T, C0 + C1);
    if (sp == 1) return 0;
    return static_cast<size_t>(sp) * lora_grad_rp(r) * (C0 + C1) * sizeof(float);
}

int launch_lora_grads(GradArgs a, float* part, hipStream_t stream) {
    const int rp16 = lora_grad_rp(a.r);
    const int64_t C0 = a.pb[0].out ? a.pb[0].C : 0, C1 = a.pb[1].out ? a.pb[1].C : 0;
    if (C0 == 0 && C1 == 0) return QL_OK;
    if (C0 == 0) {  // only the second problem: move it first
        a.pb[0] = a.pb[1];
        a.pb[1] = GradProblem{};
    }
    const int64_t c0 = a.pb[0].out ? a.pb[0].C : 0, c1 = a.pb[1].out ? a.pb[1].C : 0;
    if (c1 == 0) a.pb[1].C = 0;
    const int splits = lora_grad_splits(a.T, c0 + c1);
    a.t_per = ceil_div(ceil_div(a.T, splits), kGradWaves * kGradRows) * kGradWaves * kGradRows;
    a.nblk0 = static_cast<int>(ceil_div(c0, kGradCols));
    if (splits > 1) {
        if (part == nullptr) return set_error(QL_ERR_WORKSPACE, "LoRA gradient: workspace missing");
        a.pb[0].part = part;
        a.pb[1].part = part + static_cast<size_t>(splits) * rp16 * c0;
    }
    const dim3 grid(static_cast<uint32_t>(a.nblk0 + ceil_div(c1, kGradCols)), static_cast<uint32_t>(splits));
    timer_begin(QL_KERNEL_LORA_GRAD, stream);
    switch (rp16 / 16) {
#define QL_GRAD_CASE(R_)                                                                   \
    case R_:                                                                               \
        hipLaunchKernelGGL(lora_grads_kernel<R_>, grid, dim3(64 * kGradWaves), 0, stream, a); \
        break;
        QL_GRAD_CASE(1)
        QL_GRAD_CASE(2)
        QL_GRAD_CASE(3)
        QL_GRAD_CASE(4)
        QL_GRAD_CASE(5)
        QL_GRAD_CASE(6)
        QL_GRAD_CASE(7)
        QL_GRAD_CASE(8)
#undef QL_GRAD_CASE
        default:
            return set_error(QL_ERR_SHAPE, "LoRA gradient: rank %d out of range", a.r);
    }
    if (splits > 1) {
        const int64_t total = static_cast<int64_t>(a.r) * (c0 + c1);
        hipLaunchKernelGGL(lora_grads_final_kernel, dim3(static_cast<uint32_t>(ceil_div(total, 256))), dim3(256), 0,
                           stream, a, splits, rp16);
    }
    timer_end(QL_KERNEL_LORA_GRAD, stream);
    return check_launch("LoRA gradients");
}

// dst[i][j] = src[i][j] for j < cols, 0 for cols <= j < ldd.
__global__ void pad_copy_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
                                uint16_t* __restrict__ dst, int64_t ldd) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= rows * ldd) return;
    const int64_t i = idx / ldd, j = idx % ldd;
    dst[idx] = (j < cols) ? src[i * cols + j] : static_cast<uint16_t>(0);
}

int launch_pad_copy(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst, int64_t ldd, hipStream_t stream) {
    hipLaunchKernelGGL(pad_copy_kernel, dim3(static_cast<uint32_t>(ceil_div(rows * ldd, 256))), dim3(256), 0, stream,
                       src, rows, cols, dst, ldd);
    return check_launch("pad copy");
}

}  // namespace qlnf4
