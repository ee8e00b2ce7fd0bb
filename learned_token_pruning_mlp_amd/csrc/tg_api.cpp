// tg_api.cpp -- the C ABI entry points: argument checks, then the launchers.
//
// Every check runs on the host before anything touches the HIP runtime, so
// an invalid call returns a negative status with nothing enqueued.
#include <stdint.h>

#include "tg_internal.h"
#include "tokengate.h"

namespace {

constexpr int kAbiVersion = 1;

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline bool finite_nonneg(float x) { return x >= 0.0f && x <= 3.4e38f; }
constexpr int64_t kMaxRows = 0x7fffffffLL;
static_assert(tgi::kNoAllocMaxTokens == TG_NOALLOC_MAX_TOKENS, "the header's limit is the scratch array's");

}  // namespace

extern "C" {

const char* tg_status_string(int status) {
    switch (status) {
        case TG_OK: return "ok";
        case TG_EINVAL: return "invalid argument (size, budget or required pointer)";
        case TG_EUNSUPPORTED: return "unsupported shape";
        case TG_EALIGN: return "pointer, row size or stride not 16-byte aligned";
        case TG_EWORKSPACE: return "workspace missing or too small";
        case TG_EDEVICE: return "HIP launch failed";
        default: return "unknown status";
    }
}

int tg_abi_version(void) { return kAbiVersion; }

size_t tg_workspace_bytes(int64_t n) { return tgi::workspace_bytes(n < 0 ? 0 : n); }

int tg_gate_score(const tg_bf16* resid, const tg_bf16* w1, const tg_bf16* b1, const tg_bf16* w2, float b2,
                  int64_t n, int32_t d, int32_t hd, float eps_row, float eps_seq, float* score_norm,
                  float* score_raw, void* workspace, size_t workspace_bytes, void* stream) {
    if (n < 0 || n > kMaxRows) return TG_EINVAL;
    if (!finite_nonneg(eps_row) || !finite_nonneg(eps_seq)) return TG_EINVAL;
    if (d <= 0 || d % 64 != 0) return TG_EUNSUPPORTED;
    if (hd != 64 && hd != 128 && hd != 256) return TG_EUNSUPPORTED;
    if (n == 0) return TG_OK;
    if (!resid || !w1 || !w2 || !score_norm) return TG_EINVAL;
    if (!aligned(resid, 16) || !aligned(w1, 16) || !aligned(score_norm, 4) ||
        (score_raw && !aligned(score_raw, 4)) || (b1 && !aligned(b1, 2)) || !aligned(w2, 2))
        return TG_EALIGN;
    if (!workspace || workspace_bytes < tgi::workspace_bytes(n)) return TG_EWORKSPACE;
    if (!aligned(workspace, 16)) return TG_EALIGN;
    return tgi::launch_gate_score(resid, w1, b1, w2, b2, n, d, hd, eps_row, eps_seq, score_norm, score_raw,
                                  workspace, stream);
}

int tg_gate_score_noalloc(const tg_bf16* resid, const tg_bf16* w1, const tg_bf16* b1, const tg_bf16* w2, float b2,
                          int64_t n, int32_t d, int32_t hd, float eps_row, float eps_seq, float* score_norm,
                          float* score_raw, void* stream) {
    if (n < 0 || n > kMaxRows) return TG_EINVAL;
    if (!finite_nonneg(eps_row) || !finite_nonneg(eps_seq)) return TG_EINVAL;
    if (d <= 0 || d % 64 != 0) return TG_EUNSUPPORTED;
    if (hd != 64 && hd != 128 && hd != 256) return TG_EUNSUPPORTED;
    if (n > tgi::kNoAllocMaxTokens) return TG_EUNSUPPORTED;  // beyond the fixed scratch
    if (n == 0) return TG_OK;
    if (!resid || !w1 || !w2 || !score_norm) return TG_EINVAL;
    if (!aligned(resid, 16) || !aligned(w1, 16) || !aligned(score_norm, 4) ||
        (score_raw && !aligned(score_raw, 4)) || (b1 && !aligned(b1, 2)) || !aligned(w2, 2))
        return TG_EALIGN;
    return tgi::launch_gate_score_noalloc(resid, w1, b1, w2, b2, n, d, hd, eps_row, eps_seq, score_norm, score_raw,
                                          stream);
}

int tg_select_topk(const float* score, const uint8_t* forced, int64_t n, int64_t n_forced, int64_t k,
                   int32_t* kept_idx, int32_t* dev_status, void* workspace, size_t workspace_bytes,
                   void* stream) {
    if (n < 1 || n > kMaxRows || k < 1 || k > n || n_forced < 0 || n_forced > k) return TG_EINVAL;
    if (!forced && n_forced != 0) return TG_EINVAL;
    if (!score || !kept_idx) return TG_EINVAL;
    if (!aligned(score, 16) || (forced && !aligned(forced, 4)) || !aligned(kept_idx, 4) ||
        (dev_status && !aligned(dev_status, 4)))
        return TG_EALIGN;
    if (!workspace || workspace_bytes < tgi::workspace_bytes(n)) return TG_EWORKSPACE;
    if (!aligned(workspace, 16)) return TG_EALIGN;
    return tgi::launch_select_topk(score, forced, n, n_forced, k, kept_idx, dev_status, workspace, stream);
}

int tg_gate_score_select(const tg_bf16* resid, const tg_bf16* w1, const tg_bf16* b1, const tg_bf16* w2, float b2,
                         int64_t n, int32_t d, int32_t hd, float eps_row, float eps_seq, const uint8_t* forced,
                         int64_t n_forced, int64_t k, float* score_norm, float* score_raw, int32_t* kept_idx,
                         int32_t* dev_status, void* workspace, size_t workspace_bytes, void* stream) {
    // the checks of tg_gate_score and of tg_select_topk together
    if (n < 1 || n > kMaxRows || k < 1 || k > n || n_forced < 0 || n_forced > k) return TG_EINVAL;
    if (!forced && n_forced != 0) return TG_EINVAL;
    if (!finite_nonneg(eps_row) || !finite_nonneg(eps_seq)) return TG_EINVAL;
    if (d <= 0 || d % 64 != 0) return TG_EUNSUPPORTED;
    if (hd != 64 && hd != 128 && hd != 256) return TG_EUNSUPPORTED;
    if (!resid || !w1 || !w2 || !score_norm || !kept_idx) return TG_EINVAL;
    if (!aligned(resid, 16) || !aligned(w1, 16) || !aligned(score_norm, 16) ||
        (score_raw && !aligned(score_raw, 4)) || (b1 && !aligned(b1, 2)) || !aligned(w2, 2) ||
        (forced && !aligned(forced, 4)) || !aligned(kept_idx, 4) || (dev_status && !aligned(dev_status, 4)))
        return TG_EALIGN;
    if (!workspace || workspace_bytes < tgi::workspace_bytes(n)) return TG_EWORKSPACE;
    if (!aligned(workspace, 16)) return TG_EALIGN;
    float* block_ss = static_cast<float*>(workspace);
    float* s_raw = score_raw ? score_raw : score_norm;
    int rc = tgi::launch_gate_mlp(resid, w1, b1, w2, b2, n, d, hd, eps_row, s_raw, block_ss, stream);
    if (rc != TG_OK) return rc;
    if (n <= tgi::kSelectOneWgMax || tgi::select_kpt(n) > 0)
        return tgi::launch_seqnorm_select(s_raw, block_ss, n, eps_seq, score_norm, forced, n_forced, k, kept_idx,
                                          dev_status, workspace, stream);
    rc = tgi::launch_gate_seqnorm(s_raw, block_ss, n, eps_seq, score_norm, stream);
    if (rc != TG_OK) return rc;
    return tgi::launch_select_topk(score_norm, forced, n, n_forced, k, kept_idx, dev_status, workspace, stream);
}

int tg_compact(const int32_t* kept_idx, int64_t k, int64_t n, const tg_bf16* resid, tg_bf16* resid_out,
               int32_t d, const int32_t* pos, int32_t* pos_out, const float* score, float* score_out,
               const tg_gather* extra, int32_t n_extra, void* stream) {
    if (k < 0 || k > kMaxRows || n < 1 || n > kMaxRows) return TG_EINVAL;
    if (n_extra < 0 || n_extra > TG_MAX_GATHER || (n_extra > 0 && !extra)) return TG_EINVAL;
    if (!kept_idx) return TG_EINVAL;
    if (resid) {
        if (!resid_out || d <= 0) return TG_EINVAL;
        if (d % 8 != 0) return TG_EALIGN;
        if (!aligned(resid, 16) || !aligned(resid_out, 16)) return TG_EALIGN;
    }
    if (score_out && !score) return TG_EINVAL;
    if (!aligned(kept_idx, 4) || (pos && !aligned(pos, 4)) || (pos_out && !aligned(pos_out, 4)) ||
        (score && !aligned(score, 4)) || (score_out && !aligned(score_out, 4)))
        return TG_EALIGN;
    for (int e = 0; e < n_extra; ++e) {
        const tg_gather& g = extra[e];
        if (g.row_bytes < 0) return TG_EINVAL;
        if (g.row_bytes == 0) continue;
        if (!g.src || !g.dst || g.src_stride < g.row_bytes || g.dst_stride < g.row_bytes) return TG_EINVAL;
        if (g.row_bytes % 16 || g.src_stride % 16 || g.dst_stride % 16 || !aligned(g.src, 16) ||
            !aligned(g.dst, 16))
            return TG_EALIGN;
    }
    if (k == 0) return TG_OK;
    return tgi::launch_compact(kept_idx, k, n, resid, resid_out, d, pos, pos_out, score, score_out, extra,
                               n_extra, stream);
}

int tg_rope(tg_bf16* x, const int32_t* pos, int64_t rows, int32_t heads, int32_t head_dim, double theta,
            void* stream) {
    if (rows < 0 || rows > kMaxRows || heads < 1 || head_dim < 2 || head_dim > 256 || head_dim % 2 != 0)
        return TG_EINVAL;
    if (!(theta > 0.0) || theta > 1e300) return TG_EINVAL;
    if (rows == 0) return TG_OK;
    if (!x || !pos) return TG_EINVAL;
    if (!aligned(x, 2) || !aligned(pos, 4)) return TG_EALIGN;
    return tgi::launch_rope(x, pos, rows, heads, head_dim, theta, stream);
}

int tg_rope_qk(tg_bf16* q, tg_bf16* k, const int32_t* pos, int64_t rows, int32_t hq, int32_t hk,
               int32_t head_dim, double theta, void* stream) {
    if (rows < 0 || rows > kMaxRows || hq < 1 || hk < 1 || head_dim < 2 || head_dim > 256 || head_dim % 2 != 0)
        return TG_EINVAL;
    if (!(theta > 0.0) || theta > 1e300) return TG_EINVAL;
    if (rows == 0) return TG_OK;
    if (!q || !k || !pos) return TG_EINVAL;
    if (!aligned(q, 2) || !aligned(k, 2) || !aligned(pos, 4)) return TG_EALIGN;
    return tgi::launch_rope_qk(q, k, pos, rows, hq, hk, head_dim, theta, stream);
}

int tg_gated_attention(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* key_score,
                       const float* gains, float temp_coef, const int32_t* pos, int64_t n_kept, int32_t hq,
                       int32_t hkv, int32_t head_dim, void* out, int32_t out_dtype, void* stream) {
    return tg_gated_attention_timed(q, k, v, key_score, gains, temp_coef, pos, n_kept, hq, hkv, head_dim, out,
                                    out_dtype, stream, nullptr, nullptr);
}

int tg_gated_attention_timed(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* key_score,
                             const float* gains, float temp_coef, const int32_t* pos, int64_t n_kept, int32_t hq,
                             int32_t hkv, int32_t head_dim, void* out, int32_t out_dtype, void* stream,
                             void* start_event, void* stop_event) {
    if (n_kept < 0 || n_kept > kMaxRows || hq < 1 || hkv < 1 || hq % hkv != 0) return TG_EINVAL;
    if (out_dtype != 0 && out_dtype != 1) return TG_EINVAL;
    if (!(temp_coef == temp_coef) || temp_coef > 3.4e38f || temp_coef < -3.4e38f) return TG_EINVAL;
    if (head_dim != 64 && head_dim != 128) return TG_EUNSUPPORTED;
    // K and V are read through 32-bit buffer offsets: each must stay under 2 GiB
    if (n_kept * (int64_t)hkv * head_dim * 2 >= (int64_t(1) << 31)) return TG_EUNSUPPORTED;
    if (n_kept == 0) return TG_OK;
    if (!q || !k || !v || !key_score || !gains || !pos || !out) return TG_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(key_score, 4) ||
        !aligned(gains, 4) || !aligned(pos, 4))
        return TG_EALIGN;
    return tgi::launch_gated_attention(q, k, v, key_score, gains, temp_coef, pos, n_kept, hq, hkv, head_dim, out,
                                       out_dtype, nullptr, 0, stream, start_event, stop_event);
}

size_t tg_attention_bwd_workspace_bytes(int64_t n_kept, int32_t hq, int32_t hkv, int32_t head_dim) {
    if (n_kept < 0 || hq < 1 || hkv < 1 || head_dim < 1) return 0;
    return tgi::attn_bwd_ws_bytes(n_kept, hq, hkv, head_dim);
}

int tg_gated_attention_bwd(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* key_score,
                           const float* gains, float temp_coef, const int32_t* pos, int64_t n_kept, int32_t hq,
                           int32_t hkv, int32_t head_dim, const tg_bf16* dout, float* dq, float* dk, float* dv,
                           float* dscore, float* dgains, float* dtemp, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (n_kept < 0 || n_kept > kMaxRows || hq < 1 || hkv < 1 || hq % hkv != 0) return TG_EINVAL;
    if (!(temp_coef == temp_coef) || temp_coef > 3.4e38f || temp_coef < -3.4e38f) return TG_EINVAL;
    if (head_dim != 64 && head_dim != 128) return TG_EUNSUPPORTED;
    // K and V, and Q and dout (read by the key pass), go through 32-bit buffer offsets
    if (n_kept * (int64_t)hkv * head_dim * 2 >= (int64_t)1 << 31) return TG_EUNSUPPORTED;
    if (n_kept * (int64_t)hq * head_dim * 2 >= (int64_t)1 << 31) return TG_EUNSUPPORTED;
    if (n_kept == 0) return TG_OK;
    if (!q || !k || !v || !key_score || !gains || !pos || !dout || !dq || !dk || !dv || !dscore || !dgains || !dtemp)
        return TG_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
        !aligned(dk, 16) || !aligned(dv, 16))
        return TG_EALIGN;
    if (!workspace || workspace_bytes < tgi::attn_bwd_ws_bytes(n_kept, hq, hkv, head_dim)) return TG_EWORKSPACE;
    if (!aligned(workspace, 256)) return TG_EALIGN;
    return tgi::launch_gated_attention_bwd(q, k, v, key_score, gains, temp_coef, pos, n_kept, hq, hkv, head_dim, dout,
                                           dq, dk, dv, dscore, dgains, dtemp, workspace, stream);
}

size_t tg_gate_score_bwd_workspace_bytes(int64_t n, int32_t d, int32_t hd) {
    if (n < 0 || d < 1 || hd < 1) return 0;
    return tgi::gate_bwd_ws_bytes(n, hd, d);
}

int tg_gate_score_bwd(void* blas, const tg_bf16* resid, const tg_bf16* w1, const tg_bf16* b1, const tg_bf16* w2,
                      int64_t n, int32_t d, int32_t hd, float eps_row, float eps_seq, const float* score_raw,
                      const float* dscore_kept, const int32_t* kept_idx, int64_t k, float* dresid, float* dw1,
                      float* db1, float* dw2, float* db2, void* workspace, size_t workspace_bytes, void* stream) {
    if (!blas) return TG_EINVAL;
    if (n < 0 || n > kMaxRows || k < 0 || k > n) return TG_EINVAL;
    if (!finite_nonneg(eps_row) || !finite_nonneg(eps_seq)) return TG_EINVAL;
    if (hd != 64 && hd != 128 && hd != 256) return TG_EUNSUPPORTED;
    if (d < 64 || d % 64 != 0 || d > 4096) return TG_EUNSUPPORTED;
    if (n == 0) return TG_OK;
    if (!resid || !w1 || !w2 || !score_raw || !dresid || !dw1 || !db1 || !dw2 || !db2) return TG_EINVAL;
    if (k > 0 && (!dscore_kept || !kept_idx)) return TG_EINVAL;
    if (!aligned(resid, 16) || !aligned(dresid, 16) || !aligned(dw1, 16)) return TG_EALIGN;
    if (!workspace || workspace_bytes < tgi::gate_bwd_ws_bytes(n, hd, d)) return TG_EWORKSPACE;
    if (!aligned(workspace, 256)) return TG_EALIGN;
    return tgi::launch_gate_score_bwd(blas, resid, w1, b1, w2, n, d, hd, eps_row, eps_seq, score_raw, dscore_kept,
                                      kept_idx, k, dresid, dw1, db1, dw2, db2, workspace, stream);
}

// The checks shared by both forms of the gated delta rule; 1 = nothing to do.
static int gdn_checks(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* alpha, const float* beta,
                      const float* state_in, int64_t n, int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                      const float* out, const float* state_out) {
    if (n < 0 || n > kMaxRows || hk < 1 || hv < 1 || hv % hk != 0) return TG_EINVAL;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return TG_EUNSUPPORTED;
    // (token rows are read through 32-bit buffer offsets)
    if (n * (int64_t)hk * dk * 2 >= (int64_t)1 << 31 || n * (int64_t)hv * dv * 2 >= (int64_t)1 << 31)
        return TG_EUNSUPPORTED;
    if (n == 0 && !state_out) return 1;
    if (n > 0 && (!q || !k || !v || !alpha || !beta || !out)) return TG_EINVAL;
    if ((n > 0 && (!aligned(q, 16) || !aligned(k, 16))) || !aligned(state_in, 16) || !aligned(state_out, 16))
        return TG_EALIGN;
    return TG_OK;
}

int tg_gated_delta_rule(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* alpha, const float* beta,
                        const float* state_in, int64_t n, int32_t hk, int32_t hv, int32_t dk, int32_t dv, float* out,
                        float* state_out, void* stream) {
    const int rc = gdn_checks(q, k, v, alpha, beta, state_in, n, hk, hv, dk, dv, out, state_out);
    if (rc != TG_OK) return rc == 1 ? TG_OK : rc;
    return tgi::launch_gated_delta_rule(q, k, v, alpha, beta, state_in, n, hk, hv, dk, dv, out, state_out, stream);
}

size_t tg_gated_delta_rule_workspace_bytes(int64_t n, int32_t hv) {
    if (n < 0 || hv < 1) return 0;
    return tgi::gdn_chunk_ws_bytes(n, hv);
}

int tg_gated_delta_rule_chunked(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* alpha,
                                const float* beta, const float* state_in, int64_t n, int32_t hk, int32_t hv,
                                int32_t dk, int32_t dv, float* out, float* state_out, void* workspace,
                                size_t workspace_bytes, void* stream) {
    const int rc = gdn_checks(q, k, v, alpha, beta, state_in, n, hk, hv, dk, dv, out, state_out);
    if (rc != TG_OK) return rc == 1 ? TG_OK : rc;
    if (n > 0) {
        if (!workspace || workspace_bytes < tgi::gdn_chunk_ws_bytes(n, hv)) return TG_EWORKSPACE;
        if (!aligned(workspace, 16)) return TG_EALIGN;
    }
    return tgi::launch_gated_delta_rule_chunked(q, k, v, alpha, beta, state_in, n, hk, hv, dk, dv, out, state_out,
                                                workspace, stream);
}

int tg_rmsnorm(const tg_bf16* x, const tg_bf16* weight, tg_bf16* y, int64_t rows, int32_t dim, float eps,
               void* stream) {
    if (rows < 0 || rows > kMaxRows || dim < 8 || dim > 4096 || dim % 8 != 0) return TG_EINVAL;
    if (!finite_nonneg(eps)) return TG_EINVAL;
    if (rows == 0) return TG_OK;
    if (!x || !weight || !y) return TG_EINVAL;
    if (!aligned(x, 16) || !aligned(weight, 16) || !aligned(y, 16)) return TG_EALIGN;
    return tgi::launch_rmsnorm(x, weight, y, rows, dim, eps, stream);
}

int tg_swiglu(const tg_bf16* gate_up, tg_bf16* out, int64_t rows, int32_t inter, void* stream) {
    if (rows < 0 || rows > kMaxRows || inter < 8 || inter % 8 != 0) return TG_EINVAL;
    if (rows * (int64_t)(inter / 8) > kMaxRows) return TG_EUNSUPPORTED;
    if (rows == 0) return TG_OK;
    if (!gate_up || !out) return TG_EINVAL;
    if (!aligned(gate_up, 16) || !aligned(out, 16)) return TG_EALIGN;
    return tgi::launch_swiglu(gate_up, out, rows, inter, stream);
}

int tg_blas_create(void** handle) {
    if (!handle) return TG_EINVAL;
    return tgi::blas_create(handle);
}

int tg_blas_destroy(void* handle) {
    if (!handle) return TG_EINVAL;
    return tgi::blas_destroy(handle);
}

int tg_linear(void* handle, const tg_bf16* x, const tg_bf16* w, const tg_bf16* residual, tg_bf16* y, int64_t rows,
              int32_t in_dim, int32_t out_dim, void* stream) {
    if (rows < 1 || rows > kMaxRows || in_dim < 1 || out_dim < 1) return TG_EINVAL;
    if (!handle || !x || !w || !y) return TG_EINVAL;
    return tgi::linear(handle, x, w, residual, y, rows, in_dim, out_dim, stream);
}

}  // extern "C"
