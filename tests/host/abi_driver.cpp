// Host-only exercise of the C ABI for the sanitizer build (AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code): every entry point with
// rejected arguments, and calls with valid shapes and fake (aligned, never
// dereferenced on the host) device pointers, which pass validation, run the
// host-side planning and workspace carving, and stop at their first launch
// (no GPU here) with QL_ERR_HIP or QL_ERR_WORKSPACE. Prints "driver ok" and
// exits 0 when every status is one of those expected.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "qlora_nf4.h"

namespace {
int failures = 0;

void expect(bool ok, const char* what, int line) {
    if (!ok) {
        std::fprintf(stderr, "line %d: %s (last error: %s)\n", line, what, qlora_last_error());
        ++failures;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

void* fake(uintptr_t v) { return reinterpret_cast<void*>(v); }

ql_nf4_weight weight(int64_t rows, int64_t cols, int dq) {
    ql_nf4_weight w{};
    w.rows = rows;
    w.cols = cols;
    w.blocksize = 64;
    w.dq_blocksize = dq ? 256 : 0;
    w.packed = static_cast<const uint8_t*>(fake(0x100000));
    w.absmax = static_cast<const float*>(fake(0x200000));
    w.c8 = static_cast<const uint8_t*>(fake(0x300000));
    w.dq_scale = static_cast<const float*>(fake(0x400000));
    w.dq_mean = static_cast<const float*>(fake(0x500000));
    return w;
}

bool launch_stop(int s) { return s == QL_OK || s == QL_ERR_HIP; }
}  // namespace

int main() {
    uint16_t* P = static_cast<uint16_t*>(fake(0x1000000));
    float* F = static_cast<float*>(fake(0x2000000));
    uint8_t* B8 = static_cast<uint8_t*>(fake(0x3000000));
    void* WS = fake(0x4000000);
    void* MIS = fake(0x4000004);

    // sizes, including out-of-range inputs
    EXPECT(nf4_packed_bytes(-1, 5) == 0 && nf4_packed_bytes(3, 5) == 8);
    EXPECT(nf4_num_blocks(0, 64, 64) == 0 && nf4_num_blocks(1, 65, 64) == 2);
    EXPECT(nf4_dq_num_groups(-3, 256) == 0 && nf4_dq_num_groups(257, 256) == 2);
    EXPECT(nf4_double_quant_workspace(0) == 0 && nf4_double_quant_workspace((int64_t)1 << 40) > 0);
    EXPECT(qlora_paged_adamw_workspace(-5) == 0);
    for (int op = 0; op < 3; ++op)
        for (int64_t T : {1, 16, 17, 1024, 4096, 65536})
            for (int r : {0, 1, 16, 64, 128}) {
                (void)qlora_linear_fwd_workspace(11008, 4096, T, r);
                (void)qlora_linear_bwd_workspace(4096, 11008, T, r);
                (void)qlora_linear_fwd_dropout_workspace(264, 1088, T, r);
                (void)qlora_linear_bwd_dropout_workspace(264, 1088, T, r);
            }
    EXPECT(qlora_linear_fwd_workspace(-1, 64, 4, 8) == 0);
    EXPECT(qlora_linear_fwd_workspace(64, 64, 4, 129) == 0);
    const int64_t rows3[3] = {4096, 1024, 1024};
    EXPECT(qlora_linear_fwd_group_workspace(rows3, 3, 4096, 1, 16) > 0);
    EXPECT(qlora_linear_fwd_group_workspace(rows3, 5, 4096, 1, 16) == 0);
    EXPECT(qlora_linear_fwd_group_workspace(nullptr, 3, 4096, 1, 16) == 0);
    // a grouped forward above decode sizes: one GEMM launch where the plan favours it
    const int64_t qkv[3] = {4096, 4096, 4096}, gu[2] = {11008, 11008};
    EXPECT(qlora_linear_fwd_group_one_launch(qkv, 3, 4096, 1024, 16) == 1);
    EXPECT(qlora_linear_fwd_group_one_launch(qkv, 3, 4096, 16, 16) == 0);
    EXPECT(qlora_linear_fwd_group_one_launch(qkv, 3, 4096, 1024, 12) == 0);
    EXPECT(qlora_linear_fwd_group_one_launch(gu, 2, 4096, 1024, 16) == 0);
    EXPECT(qlora_linear_fwd_group_one_launch(nullptr, 3, 4096, 1024, 16) == 0);
    // where the forward's U and the backward's G run inside the GEMM launch
    EXPECT(qlora_linear_fwd_u_in_launch(11008, 4096, 1024, 16) == 1 &&
           qlora_linear_fwd_u_in_launch(-1, 4096, 1024, 16) == 0);
    EXPECT(qlora_linear_bwd_g_in_launch(4096, 11008, 1024, 16) == 1 &&
           qlora_linear_bwd_g_in_launch(4096, 11008, 1024, 200) == 0);

    // quantize / double quant / dequantize
    EXPECT(nf4_quantize(nullptr, QL_F32, 4, 64, 64, B8, F, nullptr) == QL_ERR_NULL);
    EXPECT(nf4_quantize(P, 7, 4, 64, 64, B8, F, nullptr) == QL_ERR_UNSUPPORTED);
    EXPECT(nf4_quantize(P, QL_F32, 4, 64, 32, B8, F, nullptr) == QL_ERR_UNSUPPORTED);
    EXPECT(nf4_quantize(P, QL_F32, 0, 64, 64, B8, F, nullptr) == QL_ERR_SHAPE);
    EXPECT(nf4_quantize(MIS, QL_F32, 4, 64, 64, B8, F, nullptr) == QL_ERR_ALIGN);
    EXPECT(launch_stop(nf4_quantize(P, QL_BF16, 4097, 4099, 64, B8, F, nullptr)));
    EXPECT(nf4_double_quant(F, 1000, 256, B8, F, F, nullptr, 0, nullptr) == QL_ERR_WORKSPACE);
    EXPECT(nf4_double_quant(F, 1000, 128, B8, F, F, WS, 1 << 20, nullptr) == QL_ERR_UNSUPPORTED);
    EXPECT(nf4_double_quant(F, -2, 256, B8, F, F, WS, 1 << 20, nullptr) == QL_ERR_SHAPE);
    EXPECT(launch_stop(nf4_double_quant(F, (int64_t)4096 * 4096 + 4097, 256, B8, F, F, WS,
                                        nf4_double_quant_workspace((int64_t)4096 * 4096 + 4097), nullptr)));
    // quantize + double quant in one call: both launch plans (the folded
    // tree level up to 4096 quantize workgroups, the three launches past it
    // or with a tail), rejected arguments
    const int64_t qshapes[][2] = {{4096, 4096}, {11008, 4096}, {4, 64}, {3, 100}, {16448, 4096}};
    for (int dt : {QL_F32, QL_BF16})
        for (const auto& rc : qshapes) {
            const size_t qw = nf4_quantize_dq_workspace(rc[0], rc[1], dt);
            EXPECT(qw > 0);
            EXPECT(launch_stop(nf4_quantize_dq(P, dt, rc[0], rc[1], 64, B8, F, 256, B8, F, F, WS, qw, nullptr)));
            EXPECT(nf4_quantize_dq(P, dt, rc[0], rc[1], 64, B8, F, 256, B8, F, F, WS, qw - 1, nullptr) ==
                   QL_ERR_WORKSPACE);
        }
    EXPECT(nf4_quantize_dq_workspace(0, 64, QL_F32) == 0 && nf4_quantize_dq_workspace(4, 64, 7) == 0);
    EXPECT(nf4_quantize_dq(P, QL_F32, 4, 64, 64, B8, F, 128, B8, F, F, WS, 1 << 20, nullptr) == QL_ERR_UNSUPPORTED);
    EXPECT(nf4_quantize_dq(P, QL_F32, 4, 64, 64, B8, F, 256, nullptr, F, F, WS, 1 << 20, nullptr) == QL_ERR_NULL);
    EXPECT(nf4_quantize_dq(MIS, QL_F32, 4, 64, 64, B8, F, 256, B8, F, F, WS, 1 << 20, nullptr) == QL_ERR_ALIGN);

    ql_nf4_weight w = weight(4096, 4096, 1);
    EXPECT(launch_stop(nf4_dequantize(&w, P, QL_BF16, nullptr)));
    EXPECT(nf4_dequantize(&w, P, 9, nullptr) == QL_ERR_UNSUPPORTED);
    ql_nf4_weight bad = weight(4096, 4096, 1);
    bad.blocksize = 128;
    EXPECT(nf4_dequantize(&bad, P, QL_BF16, nullptr) == QL_ERR_UNSUPPORTED);
    bad = weight(0, 4096, 1);
    EXPECT(nf4_dequantize(&bad, P, QL_BF16, nullptr) == QL_ERR_SHAPE);
    EXPECT(nf4_dequantize(nullptr, P, QL_BF16, nullptr) == QL_ERR_NULL);

    // the linear layer: rejected arguments, then every T regime with valid shapes
    EXPECT(qlora_linear_fwd(&w, P, 4, P, P, 129, 2.0f, P, F, WS, 1 << 30, nullptr) == QL_ERR_SHAPE);
    bad = weight(4096, 4000, 1);
    EXPECT(qlora_linear_fwd(&bad, P, 4, P, P, 16, 2.0f, P, F, WS, 1 << 30, nullptr) == QL_ERR_SHAPE);
    EXPECT(qlora_linear_fwd(&w, P, 4, nullptr, P, 16, 2.0f, P, F, WS, 1 << 30, nullptr) == QL_ERR_NULL);
    EXPECT(qlora_linear_fwd(&w, P, 1024, P, P, 16, 2.0f, P, F, WS, 16, nullptr) == QL_ERR_WORKSPACE);
    struct Shape {
        int64_t N, K;
    };
    const Shape shapes[] = {{4096, 4096}, {11008, 4096}, {4096, 11008}, {264, 192}, {8, 64}, {22016, 8192}};
    for (const Shape& sh : shapes) {
        ql_nf4_weight ww = weight(sh.N, sh.K, 1);
        for (int64_t T : {1, 3, 16, 17, 300, 1024, 2049, 4096}) {
            for (int r : {0, 5, 16, 64, 128}) {
                const size_t fw = qlora_linear_fwd_workspace(sh.N, sh.K, T, r);
                EXPECT(launch_stop(qlora_linear_fwd(&ww, P, T, r ? P : nullptr, r ? P : nullptr, r, 2.0f, P,
                                                    r ? F : nullptr, WS, fw, nullptr)));
                const size_t bw = qlora_linear_bwd_workspace(sh.N, sh.K, T, r);
                EXPECT(launch_stop(qlora_linear_bwd(&ww, P, P, T, r ? P : nullptr, r ? P : nullptr, r, 2.0f,
                                                    r ? F : nullptr, P, r ? F : nullptr, r ? F : nullptr, 0, WS, bw,
                                                    nullptr)));
                // dX alone, the adapter gradients skipped
                EXPECT(launch_stop(qlora_linear_bwd(&ww, P, P, T, r ? P : nullptr, r ? P : nullptr, r, 2.0f, nullptr,
                                                    P, nullptr, nullptr, 0, WS, bw, nullptr)));
                if (r > 0) {
                    const size_t dw = qlora_linear_fwd_dropout_workspace(sh.N, sh.K, T, r);
                    EXPECT(launch_stop(
                        qlora_linear_fwd_dropout(&ww, P, T, P, P, r, 2.0f, B8, 0.05f, P, F, WS, dw, nullptr)));
                    const size_t dbw = qlora_linear_bwd_dropout_workspace(sh.N, sh.K, T, r);
                    EXPECT(launch_stop(qlora_linear_bwd_dropout(&ww, P, P, T, P, P, r, 2.0f, B8, 0.05f, F, P, F, F,
                                                                1, WS, dbw, nullptr)));
                    const int s = qlora_linear_fwd_noalloc(&ww, P, T, P, P, r, 2.0f, P, F, nullptr);
                    EXPECT(launch_stop(s) || s == QL_ERR_WORKSPACE);
                }
            }
        }
        EXPECT(launch_stop(qlora_merge(&ww, P, P, 16, 2.0f, P, nullptr)));
        EXPECT(launch_stop(q4_quant_error(P, QL_F32, sh.N, sh.K, 64, QL_GRID_UNIFORM, reinterpret_cast<double*>(F),
                                          WS, q4_quant_error_workspace(sh.N, sh.K, QL_F32), nullptr)));
    }
    EXPECT(qlora_linear_fwd_dropout(&w, P, 4, P, P, 16, 2.0f, nullptr, 0.1f, P, F, WS, 1 << 30, nullptr) ==
           QL_ERR_NULL);
    EXPECT(qlora_linear_fwd_dropout(&w, P, 4, P, P, 16, 2.0f, B8, 1.0f, P, F, WS, 1 << 30, nullptr) ==
           QL_ERR_UNSUPPORTED);

    // grouped decode forward
    ql_nf4_weight gw[3] = {weight(4096, 4096, 1), weight(1024, 4096, 1), weight(1024, 4096, 1)};
    const ql_nf4_weight* gwp[3] = {&gw[0], &gw[1], &gw[2]};
    const uint16_t* As[3] = {P, P, P};
    const uint16_t* Bs[3] = {P, P, P};
    uint16_t* Ys[3] = {P, P, P};
    float* Us[3] = {F, nullptr, F};
    for (int64_t T : {1, 16, 40}) {
        const size_t gws = qlora_linear_fwd_group_workspace(rows3, 3, 4096, T, 16);
        EXPECT(launch_stop(qlora_linear_fwd_group(gwp, 3, P, T, As, Bs, 16, 2.0f, Ys, Us, WS, gws, nullptr)));
    }
    EXPECT(qlora_linear_fwd_group(gwp, 0, P, 1, As, Bs, 16, 2.0f, Ys, Us, WS, 1 << 20, nullptr) == QL_ERR_SHAPE);
    EXPECT(qlora_linear_fwd_group(nullptr, 3, P, 1, As, Bs, 16, 2.0f, Ys, Us, WS, 1 << 20, nullptr) == QL_ERR_NULL);

    // grouped backward: the summed dX of layers that share X, dA and dB per layer
    const int64_t rows2[2] = {11008, 11008};
    ql_nf4_weight bw[2] = {weight(11008, 4096, 1), weight(11008, 4096, 1)};
    const ql_nf4_weight* bwp[2] = {&bw[0], &bw[1]};
    const uint16_t* dYs[2] = {P, P};
    const float* Usv[2] = {F, nullptr};
    float* dAs[2] = {F, F};
    float* dBs[2] = {F, nullptr};
    for (int64_t T : {64, 1024, 4096}) {
        const size_t bws = qlora_linear_bwd_group_workspace(rows2, 2, 4096, T, 16);
        EXPECT(bws > 0);
        EXPECT(launch_stop(
            qlora_linear_bwd_group(bwp, 2, P, dYs, T, As, Bs, 16, 2.0f, Usv, P, dAs, dBs, 0, WS, bws, nullptr)));
    }
    EXPECT(qlora_linear_bwd_group_workspace(rows2, 5, 4096, 64, 16) == 0);
    EXPECT(qlora_linear_bwd_group(bwp, 5, P, dYs, 64, As, Bs, 16, 2.0f, Usv, P, dAs, dBs, 0, WS, 1 << 30, nullptr) ==
           QL_ERR_SHAPE);
    EXPECT(qlora_linear_bwd_group(bwp, 2, P, nullptr, 64, As, Bs, 16, 2.0f, Usv, P, dAs, dBs, 0, WS, 1 << 30,
                                  nullptr) == QL_ERR_NULL);

    // optimizer: rejected arguments (the state's memory type is asked of the
    // runtime only after these)
    EXPECT(qlora_paged_adamw(F, nullptr, F, F, F, 0, 1, 2e-4f, 0.9f, 0.999f, 1e-8f, 0.0f, nullptr, 0, nullptr,
                             nullptr) == QL_ERR_SHAPE);
    EXPECT(qlora_paged_adamw(F, nullptr, F, F, F, 100, 0, 2e-4f, 0.9f, 0.999f, 1e-8f, 0.0f, nullptr, 0, nullptr,
                             nullptr) == QL_ERR_SHAPE);
    EXPECT(qlora_paged_adamw(F, nullptr, F, F, F, 100, 1, 2e-4f, 1.0f, 0.999f, 1e-8f, 0.0f, nullptr, 0, nullptr,
                             nullptr) == QL_ERR_UNSUPPORTED);
    EXPECT(qlora_paged_adamw(nullptr, nullptr, F, F, F, 100, 1, 2e-4f, 0.9f, 0.999f, 1e-8f, 0.0f, nullptr, 0,
                             nullptr, nullptr) == QL_ERR_NULL);

    // diagnostics
    for (int s = -8; s <= 1; ++s) EXPECT(qlora_status_string(s) != nullptr);
    int64_t n = -1;
    double ms = -1.0;
    EXPECT(qlora_timer_arm(QL_KERNEL_GEMM_FWD) == QL_OK);
    EXPECT(qlora_timer_read(QL_KERNEL_GEMM_FWD, &n, &ms) == QL_OK);
    EXPECT(qlora_timer_disarm(QL_KERNEL_GEMM_FWD) == QL_OK);
    EXPECT(qlora_timer_arm(QL_KERNEL_COUNT) == QL_ERR_UNSUPPORTED);
    EXPECT(qlora_timer_read(QL_KERNEL_GEMM_FWD, nullptr, &ms) == QL_ERR_NULL);

    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("driver ok\n");
    return 0;
}
