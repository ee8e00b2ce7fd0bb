// Drives the host-side argument checks of every C ABI entry point
// (csrc/tg_api.cpp) with valid and invalid arguments, linked against
// launcher stand-ins (launch_stubs.cpp), for an AddressSanitizer /
// UndefinedBehaviorSanitizer build.  Fake device addresses are never
// dereferenced: a valid call ends in a stand-in, which returns 77.
#include <stdint.h>
#include <stdio.h>

#include "tokengate.h"

static int fails = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        const int got_ = (call);                                                        \
        if (got_ != (want)) {                                                           \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (want)); \
            ++fails;                                                                    \
        }                                                                               \
    } while (0)

int main() {
    constexpr int R = 77;  // reached the launcher
    uint16_t* A = reinterpret_cast<uint16_t*>(uintptr_t(1) << 20);  // 16-byte aligned, never touched
    uint16_t* M = reinterpret_cast<uint16_t*>((uintptr_t(1) << 20) + 2);
    float* F = reinterpret_cast<float*>(A);
    int32_t* I = reinterpret_cast<int32_t*>(A);
    uint8_t* U = reinterpret_cast<uint8_t*>(A);
    void* W = A;
    const size_t ws = tg_workspace_bytes(512);
    EXPECT(tg_abi_version(), 1);
    for (int s = 0; s >= -6; --s)
        if (!tg_status_string(s)) ++fails;
    if (tg_workspace_bytes(-5) != tg_workspace_bytes(0)) ++fails;
    // scorer
    EXPECT(tg_gate_score(A, A, nullptr, A, 0.f, 512, 256, 64, 1e-6f, 1e-6f, F, nullptr, W, ws, nullptr), R);
    EXPECT(tg_gate_score(A, A, nullptr, A, 0.f, 0, 256, 64, 1e-6f, 1e-6f, F, nullptr, W, ws, nullptr), TG_OK);
    EXPECT(tg_gate_score(A, A, nullptr, A, 0.f, -1, 256, 64, 1e-6f, 1e-6f, F, nullptr, W, ws, nullptr), TG_EINVAL);
    EXPECT(tg_gate_score(A, A, nullptr, A, 0.f, 512, 200, 64, 1e-6f, 1e-6f, F, nullptr, W, ws, nullptr), TG_EUNSUPPORTED);
    EXPECT(tg_gate_score(M, A, nullptr, A, 0.f, 512, 256, 64, 1e-6f, 1e-6f, F, nullptr, W, ws, nullptr), TG_EALIGN);
    EXPECT(tg_gate_score(A, A, nullptr, A, 0.f, 512, 256, 64, 1e-6f, 1e-6f, F, nullptr, W, ws - 1, nullptr), TG_EWORKSPACE);
    EXPECT(tg_gate_score_noalloc(A, A, nullptr, A, 0.f, 512, 256, 64, 1e-6f, 1e-6f, F, nullptr, nullptr), R);
    EXPECT(tg_gate_score_noalloc(A, A, nullptr, A, 0.f, (1 << 22) + 1, 256, 64, 1e-6f, 1e-6f, F, nullptr, nullptr),
           TG_EUNSUPPORTED);
    // select
    const size_t wsl = tg_workspace_bytes(200000);
    EXPECT(tg_select_topk(F, U, 200000, 10, 4000, I, nullptr, W, wsl, nullptr), R);
    EXPECT(tg_select_topk(F, U, 200000, 10, 0, I, nullptr, W, wsl, nullptr), TG_EINVAL);
    EXPECT(tg_select_topk(F, U, 200000, 5000, 4000, I, nullptr, W, wsl, nullptr), TG_EINVAL);
    EXPECT(tg_select_topk(F, nullptr, 200000, 10, 4000, I, nullptr, W, wsl, nullptr), TG_EINVAL);
    EXPECT(tg_select_topk(F, U, 200000, 10, 4000, I, nullptr, W, wsl - 1, nullptr), TG_EWORKSPACE);
    // scorer and select in one call
    EXPECT(tg_gate_score_select(A, A, nullptr, A, 0.f, 200000, 256, 64, 1e-6f, 1e-6f, U, 10, 4000, F, nullptr, I,
                                nullptr, W, wsl, nullptr), R);
    EXPECT(tg_gate_score_select(A, A, nullptr, A, 0.f, 200000, 256, 64, 1e-6f, 1e-6f, U, 10, 0, F, nullptr, I,
                                nullptr, W, wsl, nullptr), TG_EINVAL);
    EXPECT(tg_gate_score_select(A, A, nullptr, A, 0.f, 200000, 200, 64, 1e-6f, 1e-6f, U, 10, 4000, F, nullptr, I,
                                nullptr, W, wsl, nullptr), TG_EUNSUPPORTED);
    EXPECT(tg_gate_score_select(A, A, nullptr, A, 0.f, 200000, 256, 64, 1e-6f, 1e-6f, U, 10, 4000, F + 1, nullptr, I,
                                nullptr, W, wsl, nullptr), TG_EALIGN);
    EXPECT(tg_gate_score_select(A, A, nullptr, A, 0.f, 200000, 256, 64, 1e-6f, 1e-6f, U, 10, 4000, F, nullptr, I,
                                nullptr, W, wsl - 1, nullptr), TG_EWORKSPACE);
    // compaction
    tg_gather g{A, A, 64, 64, 64};
    EXPECT(tg_compact(I, 64, 512, A, A, 256, nullptr, I, F, F, &g, 1, nullptr), R);
    EXPECT(tg_compact(I, 0, 512, A, A, 256, nullptr, I, F, F, nullptr, 0, nullptr), TG_OK);
    EXPECT(tg_compact(I, 64, 512, A, A, 256, nullptr, I, F, F, nullptr, 17, nullptr), TG_EINVAL);
    tg_gather bad{A, A, 24, 32, 32};
    EXPECT(tg_compact(I, 64, 512, A, A, 256, nullptr, I, F, F, &bad, 1, nullptr), TG_EALIGN);
    // RoPE
    EXPECT(tg_rope(A, I, 10, 8, 128, 1e6, nullptr), R);
    EXPECT(tg_rope(A, I, 10, 8, 127, 1e6, nullptr), TG_EINVAL);
    EXPECT(tg_rope_qk(A, A, I, 10, 16, 8, 128, 1e6, nullptr), R);
    EXPECT(tg_rope_qk(A, A, I, 10, 16, 8, 128, -1.0, nullptr), TG_EINVAL);
    // attention and its backward
    EXPECT(tg_gated_attention(A, A, A, F, F, 0.1f, I, 128, 4, 2, 64, A, 0, nullptr), R);
    EXPECT(tg_gated_attention(A, A, A, F, F, 0.1f, I, 128, 6, 4, 64, A, 0, nullptr), TG_EINVAL);
    EXPECT(tg_gated_attention(A, A, A, F, F, 0.1f, I, 1 << 20, 16, 8, 128, A, 0, nullptr), TG_EUNSUPPORTED);
    EXPECT(tg_gated_attention_timed(A, A, A, F, F, 0.1f, I, 128, 4, 2, 64, A, 0, nullptr, A, A), R);
    EXPECT(tg_gated_attention_timed(A, A, A, F, F, 0.1f, I, 128, 4, 2, 64, A + 1, 0, nullptr, A, A), TG_EALIGN);
    const size_t wsb = tg_attention_bwd_workspace_bytes(64, 4, 2, 64);
    EXPECT(tg_gated_attention_bwd(A, A, A, F, F, 0.1f, I, 64, 4, 2, 64, A, F, F, F, F, F, F, W, wsb, nullptr), R);
    EXPECT(tg_gated_attention_bwd(A, A, A, F, F, 0.1f, I, 131072, 64, 8, 128, A, F, F, F, F, F, F, W, wsb, nullptr),
           TG_EUNSUPPORTED);
    // scorer backward
    void* blas = nullptr;
    EXPECT(tg_blas_create(&blas), TG_OK);
    const size_t wsg = tg_gate_score_bwd_workspace_bytes(64, 128, 64);
    EXPECT(tg_gate_score_bwd(blas, A, A, nullptr, A, 64, 128, 64, 1e-6f, 1e-6f, F, F, I, 8, F, F, F, F, F, W, wsg,
                             nullptr), R);
    EXPECT(tg_gate_score_bwd(blas, A, A, nullptr, A, 64, 128, 64, 1e-6f, 1e-6f, F, F, I, 65, F, F, F, F, F, W, wsg,
                             nullptr), TG_EINVAL);
    // recurrent mixer
    EXPECT(tg_gated_delta_rule(A, A, A, F, F, nullptr, 16, 2, 4, 64, 64, F, F, nullptr), R);
    EXPECT(tg_gated_delta_rule(A, A, A, F, F, nullptr, 16, 2, 3, 64, 64, F, F, nullptr), TG_EINVAL);
    {
        const size_t gw = tg_gated_delta_rule_workspace_bytes(16, 4);
        EXPECT(tg_gated_delta_rule_chunked(A, A, A, F, F, nullptr, 16, 2, 4, 64, 64, F, F, W, gw, nullptr), R);
        EXPECT(tg_gated_delta_rule_chunked(A, A, A, F, F, nullptr, 16, 2, 4, 64, 64, F, F, W, gw - 1, nullptr),
               TG_EWORKSPACE);
        EXPECT(tg_gated_delta_rule_chunked(A, A, A, F, F, nullptr, 16, 2, 3, 64, 64, F, F, W, gw, nullptr), TG_EINVAL);
    }
    // layer pieces
    EXPECT(tg_rmsnorm(A, A, A, 4, 128, 1e-6f, nullptr), R);
    EXPECT(tg_rmsnorm(A, A, A, 4, 7, 1e-6f, nullptr), TG_EINVAL);
    EXPECT(tg_swiglu(A, A, 4, 128, nullptr), R);
    EXPECT(tg_linear(blas, A, A, nullptr, A, 4, 128, 64, nullptr), R);
    EXPECT(tg_blas_destroy(blas), TG_OK);
    if (fails) return 1;
    puts("abi driver ok");
    return 0;
}
