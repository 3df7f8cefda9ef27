// C ABI of the QLoRA NF4 library: argument validation (before any launch),
// workspace carving, dispatch to the gfx950 kernels, error text and kernel
// timers. No C++ exception crosses this file's extern "C" functions.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <vector>

#include "common.h"
#include "internal.h"
#include "qlora_nf4.h"

namespace qlnf4 {

namespace {
thread_local char g_last_error[512] = "";

struct TimerState {
    bool armed = false;
    std::vector<hipEvent_t> starts, stops;
    size_t used = 0;
    bool open = false;
};
TimerState g_timers[QL_KERNEL_COUNT];
std::mutex g_timer_mu;
}  // namespace

int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(QL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return QL_OK;
}

void timer_begin(int kid, hipStream_t stream) {
    TimerState& t = g_timers[kid];
    if (!t.armed) return;
    std::lock_guard<std::mutex> lk(g_timer_mu);
    if (t.used == t.starts.size()) {
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) return;
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            return;
        }
        t.starts.push_back(a);
        t.stops.push_back(b);
    }
    (void)hipEventRecord(t.starts[t.used], stream);
    t.open = true;
}

void timer_end(int kid, hipStream_t stream) {
    TimerState& t = g_timers[kid];
    if (!t.armed || !t.open) return;
    std::lock_guard<std::mutex> lk(g_timer_mu);
    (void)hipEventRecord(t.stops[t.used], stream);
    ++t.used;
    t.open = false;
}

namespace {

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Sequential carving of one workspace buffer into 256-byte aligned parts.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(size_t count) {
        off = align_up(off, 256);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

int rank_pad64(int r) { return r <= 0 ? 0 : (r + 63) / 64 * 64; }

int check_ptr(const void* p, const char* name) {
    if (p == nullptr) return set_error(QL_ERR_NULL, "%s is NULL", name);
    if (!aligned16(p)) return set_error(QL_ERR_ALIGN, "%s is not 16-byte aligned", name);
    return QL_OK;
}

int check_weight(const ql_nf4_weight* w) {
    if (w == nullptr) return set_error(QL_ERR_NULL, "weight descriptor is NULL");
    if (w->rows <= 0 || w->cols <= 0)
        return set_error(QL_ERR_SHAPE, "weight shape %lld x %lld", (long long)w->rows, (long long)w->cols);
    if (w->blocksize != QL_NF4_BLOCKSIZE)
        return set_error(QL_ERR_UNSUPPORTED, "blocksize %d (only 64 is offered)", w->blocksize);
    if (w->dq_blocksize != 0 && w->dq_blocksize != QL_DQ_BLOCKSIZE)
        return set_error(QL_ERR_UNSUPPORTED, "dq_blocksize %d (0 or 256)", w->dq_blocksize);
    int s;
    if ((s = check_ptr(w->packed, "packed")) != QL_OK) return s;
    if (w->dq_blocksize) {
        if ((s = check_ptr(w->c8, "c8")) != QL_OK) return s;
        if ((s = check_ptr(w->dq_scale, "dq_scale")) != QL_OK) return s;
        if ((s = check_ptr(w->dq_mean, "dq_mean")) != QL_OK) return s;
    } else {
        if ((s = check_ptr(w->absmax, "absmax")) != QL_OK) return s;
    }
    return QL_OK;
}

NF4Dev to_dev(const ql_nf4_weight* w) {
    NF4Dev d;
    d.packed = w->packed;
    d.absmax = w->absmax;
    d.c8 = w->c8;
    d.scale = w->dq_scale;
    d.mean = w->dq_mean;
    d.dq = w->dq_blocksize != 0 ? 1 : 0;
    return d;
}

int check_linear_shape(const ql_nf4_weight* w, int64_t T, int32_t r) {
    if (T < 0) return set_error(QL_ERR_SHAPE, "T = %lld", (long long)T);
    if (w->cols % 64 != 0) return set_error(QL_ERR_SHAPE, "K = %lld is not a multiple of 64", (long long)w->cols);
    if (w->rows % 8 != 0) return set_error(QL_ERR_SHAPE, "N = %lld is not a multiple of 8", (long long)w->rows);
    if (r < 0 || r > QL_MAX_RANK) return set_error(QL_ERR_SHAPE, "rank %d outside [0, %d]", r, QL_MAX_RANK);
    if (T > (int64_t(1) << 31) / 1) return set_error(QL_ERR_SHAPE, "T = %lld too large", (long long)T);
    return QL_OK;
}

// ---- forward workspace -------------------------------------------------
struct FwdWs {
    uint16_t* Xd = nullptr;  // bf16 [T, K] = X * keep (dropout only)
    uint16_t* Us = nullptr;  // bf16 [T, rp64] = bf16(s U), GEMM path
    uint16_t* Bp = nullptr;  // bf16 [N, rp64], GEMM path when r % 8 != 0
    void* proj = nullptr;    // split partials of the U projection
    float* split = nullptr;  // fp32 split-K partials of the GEMM path
    void* gemv = nullptr;    // GEMV path: fp32 U and its projection's partials
    uint64_t* uword = nullptr;  // GEMM path with U inside the launch: U words and counters
    size_t bytes = 0;
};

constexpr int64_t kGemvMaxT = 16;

// Dropout (a keep mask) always takes the GEMM path: the GEMV feeds the base
// and the adapter the same x operands.
FwdWs carve_fwd(void* ws, int64_t N, int64_t K, int64_t T, int32_t r, bool drop = false) {
    Carver c(ws);
    FwdWs f;
    const int rp = rank_pad64(r);
    if (T <= kGemvMaxT && !drop) {
        const size_t gb = gemv_ws_bytes(T, K, r);
        if (gb) f.gemv = c.take<char>(gb);
    } else {
        if (r > 0 && !drop && gemm_fwd_u_in_launch(N, K, T, r)) {
            f.uword = c.take<uint64_t>(gemm_fwd_u_words(T, r));  // U inside the GEMM launch
        } else if (r > 0) {
            if (drop) f.Xd = c.take<uint16_t>(static_cast<size_t>(T) * K);
            f.Us = c.take<uint16_t>(static_cast<size_t>(T) * rp);
            if (r % 8 != 0) f.Bp = c.take<uint16_t>(static_cast<size_t>(N) * rp);
            const size_t pb = lora_proj_ws_bytes(T, r, K, false);
            if (pb) f.proj = c.take<char>(pb);
        }
        const size_t sb = gemm_split_bytes(N, T, K);
        if (sb) f.split = c.take<float>(sb / sizeof(float));
    }
    f.bytes = align_up(c.off, 256);
    return f;
}

// ---- backward workspace ------------------------------------------------
struct BwdWs {
    uint16_t* Xd = nullptr;  // bf16 [T, K] = X * keep (dropout, for dA or a recomputed U)
    uint16_t* Gp = nullptr;  // bf16 [T, rp64] = G = s dY B, dX's LoRA operand
    uint16_t* Gt = nullptr;  // bf16 [rp16, T] = G^T, dA's MFMA operand
    uint16_t* Ut = nullptr;  // bf16 [rp16, T] = U^T, dB's MFMA operand
    float* gpart = nullptr;  // fp32 token-split partials of dA and dB
    void* proj = nullptr;    // split partials of the G (and U) projections, used in turn
    float* split = nullptr;  // fp32 split-K partials of the dX GEMM
    uint64_t* gword = nullptr;  // dX GEMM with G inside its launch: G words and the epoch word
    size_t bytes = 0;
};

BwdWs carve_bwd(void* ws, int64_t N, int64_t K, int64_t T, int32_t r, bool want_dx, bool want_da, bool want_db,
                bool drop = false) {
    Carver c(ws);
    BwdWs b;
    if (r > 0) {
        if (drop && (want_da || want_db)) b.Xd = c.take<uint16_t>(static_cast<size_t>(T) * K);
        const int rp = rank_pad64(r);
        const int rp16 = lora_grad_rp(r);
        if (want_dx && !drop && gemm_dx_g_in_launch(N, K, T, r))
            b.gword = c.take<uint64_t>(gemm_fwd_u_words(T, r));  // G inside the dX GEMM launch
        else if (want_dx)
            b.Gp = c.take<uint16_t>(static_cast<size_t>(T) * rp);
        if (want_da) b.Gt = c.take<uint16_t>(static_cast<size_t>(rp16) * lora_vt_ld(T));
        if (want_db) b.Ut = c.take<uint16_t>(static_cast<size_t>(rp16) * lora_vt_ld(T));
        const size_t gb = lora_grads_part_bytes(T, want_da ? K : 0, want_db ? N : 0, r);
        if (gb) b.gpart = c.take<float>(gb / sizeof(float));
        const size_t pb = std::max(lora_proj_ws_bytes(T, r, N, true), lora_proj_ws_bytes(T, r, K, false));
        if (pb) b.proj = c.take<char>(pb);
    }
    if (want_dx) {
        const size_t sb = gemm_split_bytes(K, T, N);
        if (sb) b.split = c.take<float>(sb / sizeof(float));
    }
    b.bytes = align_up(c.off, 256);
    return b;
}

// ---- grouped backward workspace -----------------------------------------
// Layers that read the same X: G of every layer (the grouped dX GEMM reads
// them all), one set of gradient operands and partials reused layer by layer
// (stream order), and the dX GEMM's split partials.
struct GroupBwdWs {
    uint16_t* Gp[kGemmMaxGroup] = {};  // bf16 [T, rp64] per layer
    uint16_t* Gt = nullptr;            // bf16 [rp16, T], the layer being processed
    uint16_t* Ut = nullptr;
    float* gpart = nullptr;
    void* proj = nullptr;
    float* split = nullptr;
    size_t bytes = 0;
};

GroupBwdWs carve_bwd_group(void* ws, const int64_t* N, int nw, int64_t K, int64_t T, int32_t r, bool want_dx,
                           bool want_da, bool want_db) {
    Carver c(ws);
    GroupBwdWs b;
    if (r > 0) {
        const int rp = rank_pad64(r);
        const int rp16 = lora_grad_rp(r);
        if (want_dx)
            for (int i = 0; i < nw; ++i) b.Gp[i] = c.take<uint16_t>(static_cast<size_t>(T) * rp);
        if (want_da) b.Gt = c.take<uint16_t>(static_cast<size_t>(rp16) * lora_vt_ld(T));
        if (want_db) b.Ut = c.take<uint16_t>(static_cast<size_t>(rp16) * lora_vt_ld(T));
        size_t gb = 0, pb = lora_proj_ws_bytes(T, r, K, false);
        for (int i = 0; i < nw; ++i) {
            gb = std::max(gb, lora_grads_part_bytes(T, want_da ? K : 0, want_db ? N[i] : 0, r));
            pb = std::max(pb, lora_proj_ws_bytes(T, r, N[i], true));
        }
        if (gb && (want_da || want_db)) b.gpart = c.take<float>(gb / sizeof(float));
        if (pb) b.proj = c.take<char>(pb);
    }
    if (want_dx) {
        const size_t sb = gemm_split_bytes(K, T, int64_t{64} * gemm_group_steps(N, nw));
        if (sb) b.split = c.take<float>(sb / sizeof(float));
    }
    b.bytes = align_up(c.off, 256);
    return b;
}

}  // namespace
}  // namespace qlnf4

using namespace qlnf4;

extern "C" {

size_t nf4_packed_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return static_cast<size_t>((rows * cols + 1) / 2);
}

int64_t nf4_num_blocks(int64_t rows, int64_t cols, int32_t blocksize) {
    if (rows <= 0 || cols <= 0 || blocksize <= 0) return 0;
    return ceil_div(rows * cols, blocksize);
}

int64_t nf4_dq_num_groups(int64_t n1, int32_t dq_blocksize) {
    if (n1 <= 0 || dq_blocksize <= 0) return 0;
    return ceil_div(n1, dq_blocksize);
}

int nf4_quantize(const void* W, int w_dtype, int64_t rows, int64_t cols, int32_t blocksize, uint8_t* packed,
                 float* absmax, void* stream) {
    g_last_error[0] = '\0';
    if (rows <= 0 || cols <= 0)
        return set_error(QL_ERR_SHAPE, "shape %lld x %lld", (long long)rows, (long long)cols);
    if (blocksize != QL_NF4_BLOCKSIZE)
        return set_error(QL_ERR_UNSUPPORTED, "blocksize %d (only 64 is offered)", blocksize);
    if (w_dtype != QL_F32 && w_dtype != QL_BF16) return set_error(QL_ERR_UNSUPPORTED, "input dtype %d", w_dtype);
    int s;
    if ((s = check_ptr(W, "W")) != QL_OK) return s;
    if ((s = check_ptr(packed, "packed")) != QL_OK) return s;
    if ((s = check_ptr(absmax, "absmax")) != QL_OK) return s;
    return launch_quantize(W, w_dtype == QL_BF16, rows * cols, packed, absmax, static_cast<hipStream_t>(stream));
}

size_t nf4_double_quant_workspace(int64_t n1) {
    if (n1 <= 0) return 0;
    return dq_workspace_bytes(n1);
}

int nf4_double_quant(const float* absmax, int64_t n1, int32_t dq_blocksize, uint8_t* c8, float* scale, float* mean,
                     void* ws, size_t ws_bytes, void* stream) {
    g_last_error[0] = '\0';
    if (n1 <= 0) return set_error(QL_ERR_SHAPE, "n1 = %lld", (long long)n1);
    if (dq_blocksize != QL_DQ_BLOCKSIZE)
        return set_error(QL_ERR_UNSUPPORTED, "dq_blocksize %d (only 256 is offered)", dq_blocksize);
    int s;
    if ((s = check_ptr(absmax, "absmax")) != QL_OK) return s;
    if ((s = check_ptr(c8, "c8")) != QL_OK) return s;
    if ((s = check_ptr(scale, "scale")) != QL_OK) return s;
    if ((s = check_ptr(mean, "mean")) != QL_OK) return s;
    const size_t need = dq_workspace_bytes(n1);
    if (ws == nullptr || ws_bytes < need)
        return set_error(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws == nullptr ? 0 : ws_bytes, need);
    if (!aligned16(ws)) return set_error(QL_ERR_ALIGN, "workspace is not 16-byte aligned");
    return launch_double_quant(absmax, n1, c8, scale, mean, static_cast<double*>(ws), static_cast<hipStream_t>(stream));
}

size_t nf4_quantize_dq_workspace(int64_t rows, int64_t cols, int w_dtype) {
    if (rows <= 0 || cols <= 0 || (w_dtype != QL_F32 && w_dtype != QL_BF16)) return 0;
    return quantize_dq_workspace_bytes(w_dtype == QL_BF16, rows * cols);
}

int nf4_quantize_dq(const void* W, int w_dtype, int64_t rows, int64_t cols, int32_t blocksize, uint8_t* packed,
                    float* absmax, int32_t dq_blocksize, uint8_t* c8, float* scale, float* mean, void* ws,
                    size_t ws_bytes, void* stream) {
    g_last_error[0] = '\0';
    if (rows <= 0 || cols <= 0)
        return set_error(QL_ERR_SHAPE, "shape %lld x %lld", (long long)rows, (long long)cols);
    if (blocksize != QL_NF4_BLOCKSIZE)
        return set_error(QL_ERR_UNSUPPORTED, "blocksize %d (only 64 is offered)", blocksize);
    if (dq_blocksize != QL_DQ_BLOCKSIZE)
        return set_error(QL_ERR_UNSUPPORTED, "dq_blocksize %d (only 256 is offered)", dq_blocksize);
    if (w_dtype != QL_F32 && w_dtype != QL_BF16) return set_error(QL_ERR_UNSUPPORTED, "input dtype %d", w_dtype);
    int s;
    if ((s = check_ptr(W, "W")) != QL_OK) return s;
    if ((s = check_ptr(packed, "packed")) != QL_OK) return s;
    if ((s = check_ptr(absmax, "absmax")) != QL_OK) return s;
    if ((s = check_ptr(c8, "c8")) != QL_OK) return s;
    if ((s = check_ptr(scale, "scale")) != QL_OK) return s;
    if ((s = check_ptr(mean, "mean")) != QL_OK) return s;
    const size_t need = quantize_dq_workspace_bytes(w_dtype == QL_BF16, rows * cols);
    if (ws == nullptr || ws_bytes < need)
        return set_error(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws == nullptr ? 0 : ws_bytes, need);
    if (!aligned16(ws)) return set_error(QL_ERR_ALIGN, "workspace is not 16-byte aligned");
    return launch_quantize_dq(W, w_dtype == QL_BF16, rows * cols, packed, absmax, c8, scale, mean, ws,
                              static_cast<hipStream_t>(stream));
}

int nf4_dequantize(const ql_nf4_weight* w, void* out, int out_dtype, void* stream) {
    g_last_error[0] = '\0';
    int s;
    if ((s = check_weight(w)) != QL_OK) return s;
    if (out_dtype != QL_F32 && out_dtype != QL_BF16) return set_error(QL_ERR_UNSUPPORTED, "output dtype %d", out_dtype);
    if ((s = check_ptr(out, "out")) != QL_OK) return s;
    return launch_dequantize(*w, out, out_dtype == QL_BF16, static_cast<hipStream_t>(stream));
}

size_t q4_quant_error_workspace(int64_t rows, int64_t cols, int w_dtype) {
    if (rows <= 0 || cols <= 0 || (w_dtype != QL_F32 && w_dtype != QL_BF16)) return 0;
    return q4_error_ws_bytes(w_dtype == QL_BF16, rows * cols);
}

int q4_quant_error(const void* W, int w_dtype, int64_t rows, int64_t cols, int32_t blocksize, int32_t grid,
                   double* stats, void* ws, size_t ws_bytes, void* stream) {
    g_last_error[0] = '\0';
    if (rows <= 0 || cols <= 0)
        return set_error(QL_ERR_SHAPE, "shape %lld x %lld", (long long)rows, (long long)cols);
    if (blocksize != QL_NF4_BLOCKSIZE)
        return set_error(QL_ERR_UNSUPPORTED, "blocksize %d (only 64 is offered)", blocksize);
    if (w_dtype != QL_F32 && w_dtype != QL_BF16) return set_error(QL_ERR_UNSUPPORTED, "input dtype %d", w_dtype);
    if (grid != QL_GRID_NF4 && grid != QL_GRID_UNIFORM) return set_error(QL_ERR_UNSUPPORTED, "grid %d", grid);
    int s;
    if ((s = check_ptr(W, "W")) != QL_OK) return s;
    if ((s = check_ptr(stats, "stats")) != QL_OK) return s;
    const size_t need = q4_error_ws_bytes(w_dtype == QL_BF16, rows * cols);
    if (need > 0) {
        if (ws == nullptr || ws_bytes < need)
            return set_error(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws == nullptr ? 0 : ws_bytes, need);
        if (!aligned16(ws)) return set_error(QL_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    return launch_q4_error(W, w_dtype == QL_BF16, rows * cols, grid, stats, ws, static_cast<hipStream_t>(stream));
}

int qlora_merge(const ql_nf4_weight* w, const uint16_t* A, const uint16_t* B, int32_t r, float scale, uint16_t* out,
                void* stream) {
    g_last_error[0] = '\0';
    int s;
    if ((s = check_weight(w)) != QL_OK) return s;
    if ((s = check_linear_shape(w, 0, r)) != QL_OK) return s;
    if ((s = check_ptr(out, "out")) != QL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (r == 0) return launch_dequantize(*w, out, true, st);
    if ((s = check_ptr(A, "A")) != QL_OK) return s;
    if ((s = check_ptr(B, "B")) != QL_OK) return s;
    return launch_merge(to_dev(w), w->rows, w->cols, A, B, r, scale, out, st);
}

size_t qlora_linear_fwd_workspace(int64_t rows, int64_t cols, int64_t T, int32_t r) {
    if (rows <= 0 || cols <= 0 || T <= 0 || r < 0 || r > QL_MAX_RANK) return 0;
    return carve_fwd(nullptr, rows, cols, T, r).bytes;
}

int qlora_linear_fwd_u_in_launch(int64_t rows, int64_t cols, int64_t T, int32_t r) {
    if (rows <= 0 || cols <= 0 || T <= kGemvMaxT || r < 0 || r > QL_MAX_RANK) return 0;
    return gemm_fwd_u_in_launch(rows, cols, T, r) ? 1 : 0;
}

int qlora_linear_bwd_g_in_launch(int64_t rows, int64_t cols, int64_t T, int32_t r) {
    if (rows <= 0 || cols <= 0 || T <= 0 || r < 0 || r > QL_MAX_RANK) return 0;
    return gemm_dx_g_in_launch(rows, cols, T, r) ? 1 : 0;
}

size_t qlora_linear_fwd_dropout_workspace(int64_t rows, int64_t cols, int64_t T, int32_t r) {
    if (rows <= 0 || cols <= 0 || T <= 0 || r < 0 || r > QL_MAX_RANK) return 0;
    return carve_fwd(nullptr, rows, cols, T, r, true).bytes;
}

}  // extern "C"

namespace {

int check_dropout(const uint8_t* keep, float p) {
    int s;
    if ((s = check_ptr(keep, "keep")) != QL_OK) return s;
    if (!(p >= 0.0f && p < 1.0f)) return set_error(QL_ERR_UNSUPPORTED, "dropout p = %g (0 <= p < 1)", (double)p);
    return QL_OK;
}

int linear_fwd(const ql_nf4_weight* w, const uint16_t* X, int64_t T, const uint16_t* A, const uint16_t* B, int32_t r,
               float scale, const uint8_t* keep, float p, uint16_t* Y, float* U_out, void* ws, size_t ws_bytes,
               void* stream) {
    g_last_error[0] = '\0';
    int s;
    if ((s = check_weight(w)) != QL_OK) return s;
    if ((s = check_linear_shape(w, T, r)) != QL_OK) return s;
    const bool drop = keep != nullptr;
    if (drop && (s = check_dropout(keep, p)) != QL_OK) return s;
    if (T == 0) return QL_OK;
    const int64_t N = w->rows, K = w->cols;
    if ((s = check_ptr(X, "X")) != QL_OK) return s;
    if ((s = check_ptr(Y, "Y")) != QL_OK) return s;
    if (r > 0) {
        if ((s = check_ptr(A, "A")) != QL_OK) return s;
        if ((s = check_ptr(B, "B")) != QL_OK) return s;
        if (U_out != nullptr && (s = check_ptr(U_out, "U_out")) != QL_OK) return s;
    }
    const FwdWs need = carve_fwd(nullptr, N, K, T, r, drop);
    if (need.bytes > 0) {
        if (ws == nullptr || ws_bytes < need.bytes)
            return set_error(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws == nullptr ? 0 : ws_bytes,
                             need.bytes);
        if (!aligned16(ws)) return set_error(QL_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const FwdWs f = carve_fwd(ws, N, K, T, r, drop);
    const NF4Dev wd = to_dev(w);
    if (T <= kGemvMaxT && !drop) return launch_gemv(wd, X, T, N, K, A, B, r, scale, Y, U_out, f.gemv, st);
    if (f.uword != nullptr) return launch_gemm_fwd_u(wd, X, A, B, r, scale, Y, U_out, T, N, K, f.uword, st);
    const int rp = rank_pad64(r);
    const uint16_t* Bsrc = B;
    int64_t ld_b = r;
    int r_b = r;
    if (r > 0) {
        // U = X A^T (with dropout: c (X * keep) A^T, c = 1 / (1 - p)): fp32
        // for the caller, bf16(s U) padded to rp for the epilogue
        const float c = drop ? 1.0f / (1.0f - p) : 1.0f;
        if (drop && (s = launch_keep_apply(X, keep, T, K, f.Xd, st)) != QL_OK) return s;
        ProjArgs a{};
        a.proj = 1;
        a.P = drop ? f.Xd : X;
        a.ldp = K;
        a.Q = A;
        a.ldq = K;
        a.rq = r;
        a.T = T;
        a.kred = K;
        a.alpha_f = c;
        a.out_f = U_out;
        a.ld_f = r;
        a.alpha_b = scale * c;
        a.out_b = f.Us;
        a.ld_b = rp;
        if ((s = launch_lora_proj(a, false, f.proj, st)) != QL_OK) return s;
        if (r % 8 != 0) {  // rows of B are not 16-byte aligned: pad them
            if ((s = launch_pad_copy(B, N, r, f.Bp, rp, st)) != QL_OK) return s;
            Bsrc = f.Bp;
            ld_b = rp;
            r_b = rp;
        }
    }
    return launch_gemm_fwd(wd, X, f.Us, Bsrc, ld_b, r_b, rp, Y, T, N, K, f.split, st);
}

// A grouped forward at T > 16 takes one GEMM launch over all layers' row
// tiles when r is a multiple of 8 (B's rows 16-byte aligned) and the plan
// says it beats the layers' own launches; otherwise the layers run one
// after another.
bool fwd_group_one_launch(const int64_t* rows, int32_t nw, int64_t cols, int64_t T, int32_t r) {
    return T > kGemvMaxT && r % 8 == 0 && gemm_fwd_group_pays(rows, nw, T, cols);
}

// Its workspace: bf16(s U_i) per layer, the U projection's partials, the
// GEMM's split partials.
struct FwdGroupWs {
    uint16_t* Us[kGemmMaxGroup] = {};
    void* proj = nullptr;
    float* split = nullptr;
    size_t bytes = 0;
};

FwdGroupWs carve_fwd_group(void* ws, const int64_t* rows, int32_t nw, int64_t K, int64_t T, int32_t r) {
    Carver c(ws);
    FwdGroupWs f;
    if (r > 0) {
        for (int i = 0; i < nw; ++i) f.Us[i] = c.take<uint16_t>(static_cast<size_t>(T) * rank_pad64(r));
        const size_t pb = lora_proj_ws_bytes(T, r, K, false);
        if (pb) f.proj = c.take<char>(pb);
    }
    const size_t sb = gemm_fwd_group_split_bytes(rows, nw, T, K);
    if (sb) f.split = c.take<float>(sb / sizeof(float));
    f.bytes = align_up(c.off, 256);
    return f;
}

size_t group_fwd_ws(const int64_t* rows, int32_t nw, int64_t cols, int64_t T, int32_t r) {
    if (rows == nullptr || nw < 1 || nw > kGemvMaxGroup || cols <= 0 || T <= 0 || r < 0 || r > QL_MAX_RANK) return 0;
    size_t m = 0;
    for (int i = 0; i < nw; ++i) {
        if (rows[i] <= 0) return 0;
        m = std::max(m, carve_fwd(nullptr, rows[i], cols, T, r).bytes);
    }
    // decode: one launch, a workspace slice per weight; larger T: one GEMM
    // launch over all weights, or the weights one after another sharing one
    // workspace
    // (layers of mixed formats take the one-after-another path: enough for both)
    if (T <= kGemvMaxT) return static_cast<size_t>(nw) * gemv_ws_bytes(T, cols, r);
    return fwd_group_one_launch(rows, nw, cols, T, r) ? std::max(m, carve_fwd_group(nullptr, rows, nw, cols, T, r).bytes)
                                                      : m;
}

int linear_fwd_group(const ql_nf4_weight* const* w, int32_t nw, const uint16_t* X, int64_t T,
                     const uint16_t* const* A, const uint16_t* const* B, int32_t r, float scale, uint16_t* const* Y,
                     float* const* U_out, void* ws, size_t ws_bytes, void* stream) {
    g_last_error[0] = '\0';
    int s;
    if (nw < 1 || nw > kGemvMaxGroup) return set_error(QL_ERR_SHAPE, "%d weights in a group (1 to %d)", nw, kGemvMaxGroup);
    // w, A, B, Y and U_out are host arrays of pointers: only NULL is an error
    if (w == nullptr || Y == nullptr) return set_error(QL_ERR_NULL, "%s array is NULL", w == nullptr ? "w" : "Y");
    if (r > 0 && (A == nullptr || B == nullptr))
        return set_error(QL_ERR_NULL, "%s array is NULL", A == nullptr ? "A" : "B");
    int64_t rows[kGemvMaxGroup];
    for (int i = 0; i < nw; ++i) {
        if ((s = check_weight(w[i])) != QL_OK) return s;
        if ((s = check_linear_shape(w[i], T, r)) != QL_OK) return s;
        if (w[i]->cols != w[0]->cols)
            return set_error(QL_ERR_SHAPE, "weight %d has %lld columns, weight 0 %lld", i, (long long)w[i]->cols,
                             (long long)w[0]->cols);
        rows[i] = w[i]->rows;
        if ((s = check_ptr(Y[i], "Y[i]")) != QL_OK) return s;
        if (r > 0) {
            if ((s = check_ptr(A[i], "A[i]")) != QL_OK) return s;
            if ((s = check_ptr(B[i], "B[i]")) != QL_OK) return s;
            if (U_out != nullptr && U_out[i] != nullptr && (s = check_ptr(U_out[i], "U_out[i]")) != QL_OK) return s;
        }
    }
    if (T == 0) return QL_OK;
    if ((s = check_ptr(X, "X")) != QL_OK) return s;
    const int64_t K = w[0]->cols;
    bool same_format = true;
    for (int i = 1; i < nw; ++i) same_format = same_format && (w[i]->dq_blocksize != 0) == (w[0]->dq_blocksize != 0);
    if (T > kGemvMaxT && !(same_format && fwd_group_one_launch(rows, nw, K, T, r))) {
        for (int i = 0; i < nw; ++i)
            if ((s = linear_fwd(w[i], X, T, r > 0 ? A[i] : nullptr, r > 0 ? B[i] : nullptr, r, scale, nullptr, 0.0f,
                                Y[i], (r > 0 && U_out != nullptr) ? U_out[i] : nullptr, ws, ws_bytes, stream)) != QL_OK)
                return s;
        return QL_OK;
    }
    if (T > kGemvMaxT) {
        // one GEMM launch over all layers' row tiles, after each layer's U
        // projection (fp32 U for the caller, bf16(s U) for the rank step)
        const FwdGroupWs f = carve_fwd_group(ws, rows, nw, K, T, r);
        if (f.bytes > 0) {
            if (ws == nullptr || ws_bytes < f.bytes)
                return set_error(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws == nullptr ? 0 : ws_bytes,
                                 f.bytes);
            if (!aligned16(ws)) return set_error(QL_ERR_ALIGN, "workspace is not 16-byte aligned");
        }
        hipStream_t st = static_cast<hipStream_t>(stream);
        const int rp = rank_pad64(r);
        GemmLayer layers[kGemmMaxGroup];
        for (int i = 0; i < nw; ++i) {
            if (r > 0) {
                ProjArgs a{};
                a.proj = 1;
                a.P = X;
                a.ldp = K;
                a.Q = A[i];
                a.ldq = K;
                a.rq = r;
                a.T = T;
                a.kred = K;
                a.alpha_f = 1.0f;
                a.out_f = U_out != nullptr ? U_out[i] : nullptr;
                a.ld_f = r;
                a.alpha_b = scale;
                a.out_b = f.Us[i];
                a.ld_b = rp;
                if ((s = launch_lora_proj(a, false, f.proj, st)) != QL_OK) return s;
            }
            layers[i] = GemmLayer{to_dev(w[i]), nullptr, rows[i], r > 0 ? f.Us[i] : nullptr, r > 0 ? B[i] : nullptr, Y[i]};
        }
        return launch_gemm_fwd_group(layers, nw, X, r, rp, T, K, f.split, st);
    }
    const size_t need = group_fwd_ws(rows, nw, K, T, r);
    if (need > 0) {
        if (ws == nullptr || ws_bytes < need)
            return set_error(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws == nullptr ? 0 : ws_bytes, need);
        if (!aligned16(ws)) return set_error(QL_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    GemvCall calls[kGemvMaxGroup];
    for (int i = 0; i < nw; ++i)
        calls[i] = GemvCall{to_dev(w[i]), rows[i], r > 0 ? A[i] : nullptr, r > 0 ? B[i] : nullptr, Y[i],
                            (r > 0 && U_out != nullptr) ? U_out[i] : nullptr};
    return launch_gemv_group(calls, nw, X, T, K, r, scale, ws, static_cast<hipStream_t>(stream));
}

int linear_bwd(const ql_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t T, const uint16_t* A,
               const uint16_t* B, int32_t r, float scale, const uint8_t* keep, float p, const float* U_saved,
               uint16_t* dX, float* dA, float* dB, int accumulate, void* ws, size_t ws_bytes, void* stream) {
    g_last_error[0] = '\0';
    int s;
    if ((s = check_weight(w)) != QL_OK) return s;
    if ((s = check_linear_shape(w, T, r)) != QL_OK) return s;
    const bool drop = keep != nullptr;
    if (drop && (s = check_dropout(keep, p)) != QL_OK) return s;
    const float c = drop ? 1.0f / (1.0f - p) : 1.0f;
    if (accumulate != 0 && accumulate != 1) return set_error(QL_ERR_UNSUPPORTED, "accumulate = %d", accumulate);
    if (r == 0 && (dA != nullptr || dB != nullptr))
        return set_error(QL_ERR_SHAPE, "dA / dB requested with rank 0");
    if (T == 0) return QL_OK;
    const int64_t N = w->rows, K = w->cols;
    const bool want_dx = dX != nullptr, want_da = dA != nullptr, want_db = dB != nullptr;
    if (!want_dx && !want_da && !want_db) return QL_OK;
    if ((s = check_ptr(dY, "dY")) != QL_OK) return s;
    if (want_dx && (s = check_ptr(dX, "dX")) != QL_OK) return s;
    if (want_da && (s = check_ptr(dA, "dA")) != QL_OK) return s;
    if (want_db && (s = check_ptr(dB, "dB")) != QL_OK) return s;
    if (r > 0) {
        if ((s = check_ptr(A, "A")) != QL_OK) return s;
        if ((s = check_ptr(B, "B")) != QL_OK) return s;
    }
    const bool have_u = U_saved != nullptr;
    if (have_u && (s = check_ptr(U_saved, "U_saved")) != QL_OK) return s;
    if ((want_da || (want_db && !have_u)) && (s = check_ptr(X, "X")) != QL_OK) return s;
    const BwdWs need = carve_bwd(nullptr, N, K, T, r, want_dx, want_da, want_db, drop);
    if (need.bytes > 0) {
        if (ws == nullptr || ws_bytes < need.bytes)
            return set_error(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws == nullptr ? 0 : ws_bytes,
                             need.bytes);
        if (!aligned16(ws)) return set_error(QL_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const BwdWs b = carve_bwd(ws, N, K, T, r, want_dx, want_da, want_db, drop);
    const NF4Dev wd = to_dev(w);
    const int rp = rank_pad64(r);
    const int rp16 = lora_grad_rp(r);
    const int64_t ldv = lora_vt_ld(T);
    ProjArgs gproj{};
    if (r > 0 && (want_dx || want_da || (want_db && have_u))) {
        // G = s dY B (B read in its own layout): bf16 row-major padded to rp
        // for the dX epilogue, bf16 transposed for dA; U^T from U_saved for dB
        ProjArgs a{};
        a.proj = (want_dx || want_da) ? 1 : 0;
        a.P = dY;
        a.ldp = N;
        a.Q = B;
        a.ldq = r;
        a.rq = r;
        a.T = T;
        a.kred = N;
        a.alpha_b = scale;
        a.out_b = want_dx ? b.Gp : nullptr;
        a.ld_b = rp;
        a.out_bt = want_da ? b.Gt : nullptr;
        a.rows_bt = rp16;
        a.ld_bt = ldv;
        if (want_db && have_u) {
            a.Usrc = U_saved;
            a.ru = r;
            a.Ut = b.Ut;
            a.rows_ut = rp16;
            a.ld_ut = ldv;
        }
        if (b.gword != nullptr) {
            gproj = a;  // run by the dX GEMM's first workgroups below
        } else if ((s = launch_lora_proj(a, true, b.proj, st)) != QL_OK) {
            return s;
        }
    }
    // dropout: the adapter input X * keep, for dA and a recomputed U
    const bool need_xd = drop && r > 0 && (want_da || (want_db && !have_u));
    if (need_xd && (s = launch_keep_apply(X, keep, T, K, b.Xd, st)) != QL_OK) return s;
    const uint16_t* Xa = need_xd ? b.Xd : X;
    if (r > 0 && want_db && !have_u) {  // U^T = (X A^T)^T recomputed (c (X * keep) A^T with dropout)
        ProjArgs a{};
        a.proj = 1;
        a.P = Xa;
        a.ldp = K;
        a.Q = A;
        a.ldq = K;
        a.rq = r;
        a.T = T;
        a.kred = K;
        a.alpha_b = c;
        a.out_bt = b.Ut;
        a.rows_bt = rp16;
        a.ld_bt = ldv;
        if ((s = launch_lora_proj(a, false, b.proj, st)) != QL_OK) return s;
    }
    if (want_dx) {
        // with dropout the adapter term is masked per element: the GEMM takes
        // only dY W', a second kernel adds c (G A) * keep
        if (b.gword != nullptr) {
            if ((s = launch_gemm_dx_g(wd, dY, A, r, dX, T, N, K, gproj, b.gword, st)) != QL_OK) return s;
        } else if ((s = launch_gemm_dx(wd, dY, b.Gp, A, r, drop ? 0 : rp, dX, T, N, K, b.split, st)) != QL_OK) {
            return s;
        }
        if (drop && r > 0 && (s = launch_lora_dx_keep(b.Gp, rp, A, r, keep, c, T, K, dX, st)) != QL_OK) return s;
    }
    if (want_da || want_db) {
        GradArgs g{};
        g.r = r;
        g.T = T;
        g.accumulate = accumulate;
        if (want_da) g.pb[0] = GradProblem{Xa, K, K, b.Gt, ldv, dA, 1, c, nullptr};
        if (want_db) g.pb[1] = GradProblem{dY, N, N, b.Ut, ldv, dB, 0, scale, nullptr};
        if ((s = launch_lora_grads(g, b.gpart, st)) != QL_OK) return s;
    }
    return QL_OK;
}

size_t group_bwd_ws(const int64_t* rows, int32_t nw, int64_t cols, int64_t T, int32_t r) {
    if (rows == nullptr || nw < 1 || nw > kGemmMaxGroup || cols <= 0 || T <= 0 || r < 0 || r > QL_MAX_RANK) return 0;
    for (int i = 0; i < nw; ++i)
        if (rows[i] <= 0) return 0;
    return carve_bwd_group(nullptr, rows, nw, cols, T, r, true, true, true).bytes;
}

int linear_bwd_group(const ql_nf4_weight* const* w, int32_t nw, const uint16_t* X, const uint16_t* const* dY,
                     int64_t T, const uint16_t* const* A, const uint16_t* const* B, int32_t r, float scale,
                     const float* const* U_saved, uint16_t* dX, float* const* dA, float* const* dB, int accumulate,
                     void* ws, size_t ws_bytes, void* stream) {
    g_last_error[0] = '\0';
    int s;
    if (nw < 1 || nw > kGemmMaxGroup)
        return set_error(QL_ERR_SHAPE, "%d weights in a group (1 to %d)", nw, kGemmMaxGroup);
    // w, dY, A, B, U_saved, dA and dB are host arrays of pointers
    if (w == nullptr || dY == nullptr) return set_error(QL_ERR_NULL, "%s array is NULL", w == nullptr ? "w" : "dY");
    if (r > 0 && (A == nullptr || B == nullptr))
        return set_error(QL_ERR_NULL, "%s array is NULL", A == nullptr ? "A" : "B");
    if (accumulate != 0 && accumulate != 1) return set_error(QL_ERR_UNSUPPORTED, "accumulate = %d", accumulate);
    int64_t rows[kGemmMaxGroup];
    bool want_da = false, want_db = false, need_x = false;
    for (int i = 0; i < nw; ++i) {
        if ((s = check_weight(w[i])) != QL_OK) return s;
        if ((s = check_linear_shape(w[i], T, r)) != QL_OK) return s;
        if (w[i]->cols != w[0]->cols)
            return set_error(QL_ERR_SHAPE, "weight %d has %lld columns, weight 0 %lld", i, (long long)w[i]->cols,
                             (long long)w[0]->cols);
        if ((w[i]->dq_blocksize != 0) != (w[0]->dq_blocksize != 0))
            return set_error(QL_ERR_UNSUPPORTED, "weight %d and weight 0 differ in double quantization", i);
        rows[i] = w[i]->rows;
        const bool da = dA != nullptr && dA[i] != nullptr, db = dB != nullptr && dB[i] != nullptr;
        const bool hu = U_saved != nullptr && U_saved[i] != nullptr;
        if (r == 0 && (da || db)) return set_error(QL_ERR_SHAPE, "dA / dB requested with rank 0");
        if (da && (s = check_ptr(dA[i], "dA[i]")) != QL_OK) return s;
        if (db && (s = check_ptr(dB[i], "dB[i]")) != QL_OK) return s;
        if (hu && (s = check_ptr(U_saved[i], "U_saved[i]")) != QL_OK) return s;
        if (r > 0) {
            if ((s = check_ptr(A[i], "A[i]")) != QL_OK) return s;
            if ((s = check_ptr(B[i], "B[i]")) != QL_OK) return s;
        }
        want_da = want_da || da;
        want_db = want_db || db;
        need_x = need_x || da || (db && !hu);
    }
    const bool want_dx = dX != nullptr;
    if (T == 0 || (!want_dx && !want_da && !want_db)) return QL_OK;
    for (int i = 0; i < nw; ++i)
        if ((s = check_ptr(dY[i], "dY[i]")) != QL_OK) return s;
    if (want_dx && (s = check_ptr(dX, "dX")) != QL_OK) return s;
    if (need_x && (s = check_ptr(X, "X")) != QL_OK) return s;
    const int64_t K = w[0]->cols;
    const GroupBwdWs need = carve_bwd_group(nullptr, rows, nw, K, T, r, want_dx, want_da, want_db);
    if (need.bytes > 0) {
        if (ws == nullptr || ws_bytes < need.bytes)
            return set_error(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws == nullptr ? 0 : ws_bytes,
                             need.bytes);
        if (!aligned16(ws)) return set_error(QL_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const GroupBwdWs b = carve_bwd_group(ws, rows, nw, K, T, r, want_dx, want_da, want_db);
    const int rp = rank_pad64(r);
    const int rp16 = lora_grad_rp(r);
    const int64_t ldv = lora_vt_ld(T);
    // layer by layer: G (for dX, kept per layer; G^T for dA), U^T for dB, then
    // that layer's dA and dB (the operands are reused by the next layer)
    for (int i = 0; i < nw && r > 0; ++i) {
        const int64_t N = rows[i];
        const bool da = dA != nullptr && dA[i] != nullptr, db = dB != nullptr && dB[i] != nullptr;
        const bool hu = U_saved != nullptr && U_saved[i] != nullptr;
        if (want_dx || da || (db && hu)) {
            ProjArgs a{};
            a.proj = (want_dx || da) ? 1 : 0;
            a.P = dY[i];
            a.ldp = N;
            a.Q = B[i];
            a.ldq = r;
            a.rq = r;
            a.T = T;
            a.kred = N;
            a.alpha_b = scale;
            a.out_b = want_dx ? b.Gp[i] : nullptr;
            a.ld_b = rp;
            a.out_bt = da ? b.Gt : nullptr;
            a.rows_bt = rp16;
            a.ld_bt = ldv;
            if (db && hu) {
                a.Usrc = U_saved[i];
                a.ru = r;
                a.Ut = b.Ut;
                a.rows_ut = rp16;
                a.ld_ut = ldv;
            }
            if ((s = launch_lora_proj(a, true, b.proj, st)) != QL_OK) return s;
        }
        if (db && !hu) {  // U^T = (X A^T)^T recomputed
            ProjArgs a{};
            a.proj = 1;
            a.P = X;
            a.ldp = K;
            a.Q = A[i];
            a.ldq = K;
            a.rq = r;
            a.T = T;
            a.kred = K;
            a.alpha_b = 1.0f;
            a.out_bt = b.Ut;
            a.rows_bt = rp16;
            a.ld_bt = ldv;
            if ((s = launch_lora_proj(a, false, b.proj, st)) != QL_OK) return s;
        }
        if (da || db) {
            GradArgs g{};
            g.r = r;
            g.T = T;
            g.accumulate = accumulate;
            if (da) g.pb[0] = GradProblem{X, K, K, b.Gt, ldv, dA[i], 1, 1.0f, nullptr};
            if (db) g.pb[1] = GradProblem{dY[i], N, N, b.Ut, ldv, dB[i], 0, scale, nullptr};
            if ((s = launch_lora_grads(g, b.gpart, st)) != QL_OK) return s;
        }
    }
    if (want_dx) {
        GemmLayer layers[kGemmMaxGroup];
        for (int i = 0; i < nw; ++i)
            layers[i] = GemmLayer{to_dev(w[i]), dY[i], rows[i], r > 0 ? b.Gp[i] : nullptr, r > 0 ? A[i] : nullptr,
                                  nullptr};
        if ((s = launch_gemm_dx_group(layers, nw, r, rp, dX, T, K, b.split, st)) != QL_OK) return s;
    }
    return QL_OK;
}

}  // namespace

extern "C" {

int qlora_linear_fwd(const ql_nf4_weight* w, const uint16_t* X, int64_t T, const uint16_t* A, const uint16_t* B,
                     int32_t r, float scale, uint16_t* Y, float* U_out, void* ws, size_t ws_bytes, void* stream) {
    return linear_fwd(w, X, T, A, B, r, scale, nullptr, 0.0f, Y, U_out, ws, ws_bytes, stream);
}

size_t qlora_linear_fwd_group_workspace(const int64_t* rows, int32_t nw, int64_t cols, int64_t T, int32_t r) {
    return group_fwd_ws(rows, nw, cols, T, r);
}

int qlora_linear_fwd_group_one_launch(const int64_t* rows, int32_t nw, int64_t cols, int64_t T, int32_t r) {
    if (rows == nullptr || nw < 1 || nw > kGemvMaxGroup || cols <= 0 || T <= 0 || r < 0 || r > QL_MAX_RANK) return 0;
    for (int i = 0; i < nw; ++i)
        if (rows[i] <= 0) return 0;
    return fwd_group_one_launch(rows, nw, cols, T, r) ? 1 : 0;
}

int qlora_linear_fwd_group(const ql_nf4_weight* const* w, int32_t nw, const uint16_t* X, int64_t T,
                           const uint16_t* const* A, const uint16_t* const* B, int32_t r, float scale,
                           uint16_t* const* Y, float* const* U_out, void* ws, size_t ws_bytes, void* stream) {
    return linear_fwd_group(w, nw, X, T, A, B, r, scale, Y, U_out, ws, ws_bytes, stream);
}

int qlora_linear_fwd_dropout(const ql_nf4_weight* w, const uint16_t* X, int64_t T, const uint16_t* A,
                             const uint16_t* B, int32_t r, float scale, const uint8_t* keep, float p, uint16_t* Y,
                             float* U_out, void* ws, size_t ws_bytes, void* stream) {
    if (keep == nullptr) {
        g_last_error[0] = '\0';
        return set_error(QL_ERR_NULL, "keep is NULL");
    }
    return linear_fwd(w, X, T, A, B, r, scale, keep, p, Y, U_out, ws, ws_bytes, stream);
}

size_t qlora_linear_bwd_workspace(int64_t rows, int64_t cols, int64_t T, int32_t r) {
    if (rows <= 0 || cols <= 0 || T <= 0 || r < 0 || r > QL_MAX_RANK) return 0;
    return carve_bwd(nullptr, rows, cols, T, r, true, true, true).bytes;
}

size_t qlora_linear_bwd_dropout_workspace(int64_t rows, int64_t cols, int64_t T, int32_t r) {
    if (rows <= 0 || cols <= 0 || T <= 0 || r < 0 || r > QL_MAX_RANK) return 0;
    return carve_bwd(nullptr, rows, cols, T, r, true, true, true, true).bytes;
}

int qlora_linear_bwd(const ql_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t T, const uint16_t* A,
                     const uint16_t* B, int32_t r, float scale, const float* U_saved, uint16_t* dX, float* dA,
                     float* dB, int accumulate, void* ws, size_t ws_bytes, void* stream) {
    return linear_bwd(w, X, dY, T, A, B, r, scale, nullptr, 0.0f, U_saved, dX, dA, dB, accumulate, ws, ws_bytes,
                      stream);
}

size_t qlora_linear_bwd_group_workspace(const int64_t* rows, int32_t nw, int64_t cols, int64_t T, int32_t r) {
    return group_bwd_ws(rows, nw, cols, T, r);
}

int qlora_linear_bwd_group(const ql_nf4_weight* const* w, int32_t nw, const uint16_t* X, const uint16_t* const* dY,
                           int64_t T, const uint16_t* const* A, const uint16_t* const* B, int32_t r, float scale,
                           const float* const* U_saved, uint16_t* dX, float* const* dA, float* const* dB,
                           int accumulate, void* ws, size_t ws_bytes, void* stream) {
    return linear_bwd_group(w, nw, X, dY, T, A, B, r, scale, U_saved, dX, dA, dB, accumulate, ws, ws_bytes, stream);
}

int qlora_linear_bwd_dropout(const ql_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t T,
                             const uint16_t* A, const uint16_t* B, int32_t r, float scale, const uint8_t* keep,
                             float p, const float* U_saved, uint16_t* dX, float* dA, float* dB, int accumulate,
                             void* ws, size_t ws_bytes, void* stream) {
    if (keep == nullptr) {
        g_last_error[0] = '\0';
        return set_error(QL_ERR_NULL, "keep is NULL");
    }
    return linear_bwd(w, X, dY, T, A, B, r, scale, keep, p, U_saved, dX, dA, dB, accumulate, ws, ws_bytes, stream);
}

}  // extern "C"

// ---- the forward without a workspace -------------------------------------
// Scratch of qlora_linear_fwd_noalloc: device memory of the library itself,
// one copy on every GPU the library runs on, held until the process ends.
// In host code the array's name is a host-side stand-in, not a device
// address; the address of each GPU's copy comes from hipGetSymbolAddress
// (with that GPU current) and only that address is handed to the kernels.
static __device__ __align__(256) unsigned char scratch[QL_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the GPU that `stream` runs on, looked up
// once per device on its first call.
int scratch_address(hipStream_t stream, void** out) {
    int dev = 0;
    const hipError_t eq = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
    if (eq != hipSuccess) return set_error(QL_ERR_HIP, "device of the stream: %s", hipGetErrorString(eq));
    if (dev < 0 || dev >= kMaxDevices) return set_error(QL_ERR_UNSUPPORTED, "device %d (at most %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return set_error(QL_ERR_HIP, "hipGetDevice failed");
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return set_error(QL_ERR_HIP, "hipSetDevice(%d) failed", dev);
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || ptr == nullptr)
            return set_error(QL_ERR_HIP, "address of the scratch array on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return QL_OK;
}
}  // namespace

extern "C" {

int qlora_linear_fwd_noalloc(const ql_nf4_weight* w, const uint16_t* X, int64_t T, const uint16_t* A,
                             const uint16_t* B, int32_t r, float scale, uint16_t* Y, float* U_out, void* stream) {
    g_last_error[0] = '\0';
    int s;
    if ((s = check_weight(w)) != QL_OK) return s;
    if ((s = check_linear_shape(w, T, r)) != QL_OK) return s;
    if (T == 0) return QL_OK;
    const size_t need = carve_fwd(nullptr, w->rows, w->cols, T, r).bytes;
    if (need > QL_NOALLOC_SCRATCH_BYTES)
        return set_error(QL_ERR_WORKSPACE,
                         "qlora_linear_fwd_noalloc: this call needs %zu bytes of scratch, the library holds %zu "
                         "(qlora_linear_fwd takes a workspace of any size)",
                         need, static_cast<size_t>(QL_NOALLOC_SCRATCH_BYTES));
    void* ptr = nullptr;
    if (need > 0 && (s = scratch_address(static_cast<hipStream_t>(stream), &ptr)) != QL_OK) return s;
    return linear_fwd(w, X, T, A, B, r, scale, nullptr, 0.0f, Y, U_out, ptr, need > 0 ? QL_NOALLOC_SCRATCH_BYTES : 0,
                      stream);
}

size_t qlora_paged_adamw_workspace(int64_t n) { return n <= 0 ? 0 : adamw_page_ws_bytes(n); }

int qlora_paged_adamw(float* param, uint16_t* param_bf16, const float* grad, float* exp_avg, float* exp_avg_sq,
                      int64_t n, int64_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                      void* ws, size_t ws_bytes, void* stream, void* copy_stream) {
    g_last_error[0] = '\0';
    if (n <= 0) return set_error(QL_ERR_SHAPE, "n = %lld", (long long)n);
    if (step < 1) return set_error(QL_ERR_SHAPE, "step = %lld (counted from 1)", (long long)step);
    if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
        return set_error(QL_ERR_UNSUPPORTED, "betas (%g, %g) outside [0, 1)", (double)beta1, (double)beta2);
    if (!(eps >= 0.0f) || !(lr >= 0.0f) || !(weight_decay >= 0.0f))
        return set_error(QL_ERR_UNSUPPORTED, "lr %g, eps %g, weight_decay %g (none may be negative)", (double)lr,
                         (double)eps, (double)weight_decay);
    int s;
    if ((s = check_ptr(param, "param")) != QL_OK) return s;
    if ((s = check_ptr(grad, "grad")) != QL_OK) return s;
    if ((s = check_ptr(exp_avg, "exp_avg")) != QL_OK) return s;
    if ((s = check_ptr(exp_avg_sq, "exp_avg_sq")) != QL_OK) return s;
    if (param_bf16 != nullptr && (s = check_ptr(param_bf16, "param_bf16")) != QL_OK) return s;
    // where the state lives: device memory, or pinned host memory (paged out)
    auto where = [](const void* p, hipMemoryType* t) {
        hipPointerAttribute_t at{};
        if (hipPointerGetAttributes(&at, p) != hipSuccess) {
            (void)hipGetLastError();  // unregistered host memory reports an error here
            *t = hipMemoryTypeUnregistered;
        } else {
            *t = at.type;
        }
    };
    hipMemoryType tm, tv;
    where(exp_avg, &tm);
    where(exp_avg_sq, &tv);
    auto usable = [](hipMemoryType t) { return t == hipMemoryTypeDevice || t == hipMemoryTypeHost; };
    if (!usable(tm) || !usable(tv) || tm != tv)
        return set_error(QL_ERR_UNSUPPORTED,
                         "exp_avg and exp_avg_sq must both be device memory or both pinned host memory "
                         "(memory types %d and %d)",
                         (int)tm, (int)tv);
    const bool paged = tm == hipMemoryTypeHost;
    if (paged) {
        const size_t need = adamw_page_ws_bytes(n);
        if (ws == nullptr || ws_bytes < need)
            return set_error(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws == nullptr ? 0 : ws_bytes, need);
        if (!aligned16(ws)) return set_error(QL_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    return launch_adamw(param, param_bf16, grad, exp_avg, exp_avg_sq, n, step, lr, beta1, beta2, eps, weight_decay,
                        paged, static_cast<float*>(ws), static_cast<hipStream_t>(stream),
                        static_cast<hipStream_t>(copy_stream));
}

const char* qlora_status_string(int status) {
    switch (status) {
        case QL_OK: return "ok";
        case QL_ERR_NULL: return "null pointer";
        case QL_ERR_SHAPE: return "bad shape";
        case QL_ERR_UNSUPPORTED: return "unsupported option";
        case QL_ERR_ALIGN: return "misaligned pointer";
        case QL_ERR_WORKSPACE: return "workspace too small";
        case QL_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* qlora_last_error(void) { return g_last_error; }

int qlora_timer_arm(int kernel_id) {
    if (kernel_id <= 0 || kernel_id >= QL_KERNEL_COUNT) return set_error(QL_ERR_UNSUPPORTED, "kernel id %d", kernel_id);
    std::lock_guard<std::mutex> lk(g_timer_mu);
    g_timers[kernel_id].armed = true;
    g_timers[kernel_id].used = 0;
    g_timers[kernel_id].open = false;
    return QL_OK;
}

int qlora_timer_read(int kernel_id, int64_t* launches, double* total_ms) {
    if (kernel_id <= 0 || kernel_id >= QL_KERNEL_COUNT) return set_error(QL_ERR_UNSUPPORTED, "kernel id %d", kernel_id);
    if (launches == nullptr || total_ms == nullptr) return set_error(QL_ERR_NULL, "output pointer is NULL");
    std::lock_guard<std::mutex> lk(g_timer_mu);
    TimerState& t = g_timers[kernel_id];
    double total = 0.0;
    for (size_t i = 0; i < t.used; ++i) {
        if (hipEventSynchronize(t.stops[i]) != hipSuccess) return set_error(QL_ERR_HIP, "event synchronize failed");
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, t.starts[i], t.stops[i]) != hipSuccess)
            return set_error(QL_ERR_HIP, "event elapsed time failed");
        total += ms;
    }
    *launches = static_cast<int64_t>(t.used);
    *total_ms = total;
    return QL_OK;
}

int qlora_timer_disarm(int kernel_id) {
    if (kernel_id <= 0 || kernel_id >= QL_KERNEL_COUNT) return set_error(QL_ERR_UNSUPPORTED, "kernel id %d", kernel_id);
    std::lock_guard<std::mutex> lk(g_timer_mu);
    g_timers[kernel_id].armed = false;
    g_timers[kernel_id].used = 0;
    g_timers[kernel_id].open = false;
    return QL_OK;
}

}  // extern "C"
