// Stand-ins for the kernel launchers and the rocBLAS wrappers, so the C ABI's
// host-side checks (csrc/tg_api.cpp) build and run on the CPU under
// AddressSanitizer / UndefinedBehaviorSanitizer.  Each returns kReached: the
// call got past every check.
#include "tg_internal.h"

namespace tgi {
constexpr int kReached = 77;
int launch_gate_score_noalloc(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, float, int64_t, int,
                              int, float, float, float*, float*, void*) { return kReached; }
int launch_gate_score(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, float, int64_t, int, int,
                      float, float, float*, float*, void*, void*) { return kReached; }
int launch_select_topk(const float*, const uint8_t*, int64_t, int64_t, int64_t, int32_t*, int32_t*, void*, void*) {
    return kReached;
}
int launch_gate_mlp(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, float, int64_t, int, int, float,
                    float*, float*, void*) { return kReached; }
int launch_gate_seqnorm(const float*, const float*, int64_t, float, float*, void*) { return kReached; }
int launch_seqnorm_select(const float*, const float*, int64_t, float, float*, const uint8_t*, int64_t, int64_t,
                          int32_t*, int32_t*, void*, void*) { return kReached; }
int launch_compact(const int32_t*, int64_t, int64_t, const uint16_t*, uint16_t*, int, const int32_t*, int32_t*,
                   const float*, float*, const tg_gather*, int, void*) { return kReached; }
int launch_rope(uint16_t*, const int32_t*, int64_t, int, int, double, void*) { return kReached; }
int launch_rope_qk(uint16_t*, uint16_t*, const int32_t*, int64_t, int, int, int, double, void*) { return kReached; }
int launch_gated_attention(const uint16_t*, const uint16_t*, const uint16_t*, const float*, const float*, float,
                           const int32_t*, int64_t, int, int, int, void*, int, float*, int, void*, void*, void*) {
    return kReached;
}
int launch_gated_attention_bwd(const uint16_t*, const uint16_t*, const uint16_t*, const float*, const float*, float,
                               const int32_t*, int64_t, int, int, int, const uint16_t*, float*, float*, float*, float*,
                               float*, float*, void*, void*) { return kReached; }
int launch_gate_score_bwd(void*, const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int, int,
                          float, float, const float*, const float*, const int32_t*, int64_t, float*, float*, float*,
                          float*, float*, void*, void*) { return kReached; }
int launch_gated_delta_rule(const uint16_t*, const uint16_t*, const uint16_t*, const float*, const float*,
                            const float*, int64_t, int, int, int, int, float*, float*, void*) { return kReached; }
size_t gdn_chunk_ws_bytes(int64_t n, int hv) { return (size_t)((n + 31) / 32 > 0 ? (n + 31) / 32 : 1) * (size_t)hv * 16384; }
int launch_gated_delta_rule_chunked(const uint16_t*, const uint16_t*, const uint16_t*, const float*, const float*,
                                    const float*, int64_t, int, int, int, int, float*, float*, void*, void*) {
    return kReached;
}
int launch_rmsnorm(const uint16_t*, const uint16_t*, uint16_t*, int64_t, int, float, void*) { return kReached; }
int launch_swiglu(const uint16_t*, uint16_t*, int64_t, int, void*) { return kReached; }
int blas_create(void** h) { *h = (void*)0x1000; return 0; }
int blas_destroy(void*) { return 0; }
int linear(void*, const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int64_t, int, int, void*) {
    return kReached;
}
}  // namespace tgi
