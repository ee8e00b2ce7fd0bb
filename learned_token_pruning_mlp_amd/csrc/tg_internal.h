// tg_internal.h -- host-side interface between the C ABI entry points
// (tg_api.cpp: argument checks) and the kernel launchers (*.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "tokengate.h"

namespace tgi {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Rows of the residual handled by one scorer workgroup (fixed for every hd).
constexpr int kGateRowsPerBlock = 64;

// Workspace layout, shared by tg_gate_score and tg_select_topk:
//   [0, gate_bytes)        per-block sums of squared raw scores (fp32)
//   [select_off, ...)      select: histograms, counters, per-chunk counts
inline int64_t gate_blocks(int64_t n) { return (n + kGateRowsPerBlock - 1) / kGateRowsPerBlock; }
// Rows per scorer workgroup actually used for a prompt of n tokens (128 once
// that still gives each of the 256 CUs a workgroup, else 64), and the number
// of per-workgroup partial sums the scorer writes (at most gate_blocks(n)).
inline int gate_rows_per_block(int64_t n) { return n >= (int64_t)256 * 128 ? 128 : 64; }
inline int64_t gate_partials(int64_t n) { return (n + gate_rows_per_block(n) - 1) / gate_rows_per_block(n); }
inline size_t gate_bytes(int64_t n) { return align_up(sizeof(float) * (size_t)(gate_blocks(n) > 0 ? gate_blocks(n) : 1)); }

// The many-workgroup select (prompts of kSelectMultiMin tokens and more):
// chunks of 256 * kpt consecutive tokens, one workgroup each, kpt the
// smallest of 8, 16, 32 that keeps the chunk count at or below
// kSelectMaxChunks (0: the prompt is too long for it, one workgroup selects).
constexpr int kSelectThreads = 256;
constexpr int kSelectMaxChunks = 64;
constexpr int64_t kSelectMultiMin = 16385;
inline int select_kpt(int64_t n) {
    if (n < kSelectMultiMin) return 0;
    for (int kpt = 8; kpt <= 32; kpt *= 2)
        if ((n + (int64_t)kSelectThreads * kpt - 1) / ((int64_t)kSelectThreads * kpt) <= kSelectMaxChunks) return kpt;
    return 0;
}
inline int64_t select_chunk_tokens(int64_t n) { return (int64_t)kSelectThreads * select_kpt(n); }
inline int64_t select_chunks(int64_t n) {
    const int64_t ch = select_chunk_tokens(n);
    return ch > 0 ? (n + ch - 1) / ch : 0;
}
// Its workspace: per chunk a 2048-bin u16 histogram of the keys' top 11 bits
// and its 64 sums of 32 consecutive bins, the forced count, the count of
// prunable keys above the first round's bin and where its keys in that bin
// start among all chunks' (the candidates, at most n keys), plus the control
// words of the first round.
struct SelectWs {
    uint16_t* hist;    // [chunks][2048]
    uint16_t* coarse;  // [chunks][64]: sums of 32 consecutive bins of hist
    uint32_t* forced;  // [chunks]
    uint32_t* above;   // [chunks]
    uint32_t* cstart;  // [chunks]: where a chunk's candidates start in cand
    uint32_t* ctl;     // [8]: first-round bin, rank left in it, forced total, prunable to choose, candidates
    uint32_t* cand;    // the keys in the first round's bin, chunk after chunk, each chunk in index order
};
// Sized for kSelectMaxChunks chunks and for the candidates of min(n, the
// largest prompt of the many-workgroup form) tokens rounded up to a chunk of
// the largest size, so the size never shrinks as n grows (a workspace sized
// for a prompt serves every shorter one).
constexpr int64_t kSelectMultiMax = (int64_t)kSelectMaxChunks * kSelectThreads * 32;
inline size_t select_bytes(int64_t n) {
    if (n < kSelectMultiMin) return kAlign;
    const int64_t m = n < kSelectMultiMax ? n : kSelectMultiMax;
    const int64_t big = (int64_t)kSelectThreads * 32;
    const size_t g = (size_t)kSelectMaxChunks;
    return align_up(sizeof(uint16_t) * 2048 * g) + align_up(sizeof(uint16_t) * 64 * g) +
           3 * align_up(sizeof(uint32_t) * g) + align_up(8 * sizeof(uint32_t)) +
           align_up(sizeof(uint32_t) * (size_t)((m + big - 1) / big * big));
}
inline SelectWs select_ws(void* base, int64_t n) {
    (void)n;
    const size_t g = (size_t)kSelectMaxChunks;
    char* p = (char*)base;
    SelectWs w;
    w.hist = (uint16_t*)p;
    p += align_up(sizeof(uint16_t) * 2048 * g);
    w.coarse = (uint16_t*)p;
    p += align_up(sizeof(uint16_t) * 64 * g);
    w.forced = (uint32_t*)p;
    p += align_up(sizeof(uint32_t) * g);
    w.above = (uint32_t*)p;
    p += align_up(sizeof(uint32_t) * g);
    w.cstart = (uint32_t*)p;
    p += align_up(sizeof(uint32_t) * g);
    w.ctl = (uint32_t*)p;
    p += align_up(8 * sizeof(uint32_t));
    w.cand = (uint32_t*)p;
    return w;
}
inline size_t workspace_bytes(int64_t n) { return gate_bytes(n) + select_bytes(n); }

// Largest prompt tg_gate_score_noalloc takes: its per-workgroup partial sums
// live in a fixed device array of kNoAllocMaxTokens / kGateRowsPerBlock floats.
constexpr int64_t kNoAllocMaxTokens = int64_t(1) << 22;

// Launchers: return 0 on success, TG_EDEVICE on a launch error.
int launch_gate_score_noalloc(const uint16_t* resid, const uint16_t* w1, const uint16_t* b1, const uint16_t* w2,
                              float b2, int64_t n, int d, int hd, float eps_row, float eps_seq, float* score_norm,
                              float* score_raw, void* stream);

int launch_gate_score(const uint16_t* resid, const uint16_t* w1, const uint16_t* b1,
                      const uint16_t* w2, float b2, int64_t n, int d, int hd, float eps_row,
                      float eps_seq, float* score_norm, float* score_raw, void* ws, void* stream);

// The scorer's two launches on their own: the MLP (raw scores and the
// per-workgroup partial sums of their squares, gate_partials(n) of them) and
// the sequence norm.
int launch_gate_mlp(const uint16_t* resid, const uint16_t* w1, const uint16_t* b1, const uint16_t* w2, float b2,
                    int64_t n, int d, int hd, float eps_row, float* s_raw, float* block_ss, void* stream);
int launch_gate_seqnorm(const float* s_raw, const float* block_ss, int64_t n, float eps_seq, float* score_norm,
                        void* stream);

// Largest prompt whose select runs in one workgroup; up to it the sequence
// norm can run inside that workgroup (tg_gate_score_select).
constexpr int64_t kSelectOneWgMax = 16384;

// Sequence norm and select together, from the raw scores and their partial
// sums to the normalised scores and the kept set: one launch up to
// kSelectOneWgMax tokens, the norm inside the first of the many-workgroup
// select's launches from there up to its limit (ws: the whole workspace, as
// for launch_select_topk); TG_EUNSUPPORTED beyond.
int launch_seqnorm_select(const float* s_raw, const float* block_ss, int64_t n, float eps_seq,
                          float* score_norm, const uint8_t* forced, int64_t n_forced, int64_t k,
                          int32_t* kept_idx, int32_t* dev_status, void* ws, void* stream);

int launch_select_topk(const float* score, const uint8_t* forced, int64_t n, int64_t n_forced,
                       int64_t k, int32_t* kept_idx, int32_t* dev_status, void* ws, void* stream);

int launch_compact(const int32_t* kept_idx, int64_t k, int64_t n, const uint16_t* resid,
                   uint16_t* resid_out, int d, const int32_t* pos, int32_t* pos_out,
                   const float* score, float* score_out, const tg_gather* extra, int n_extra,
                   void* stream);

int launch_rope(uint16_t* x, const int32_t* pos, int64_t rows, int heads, int head_dim,
                double theta, void* stream);

int launch_rope_qk(uint16_t* q, uint16_t* k, const int32_t* pos, int64_t rows, int hq, int hk, int head_dim,
                   double theta, void* stream);

// start_event / stop_event (hipEvent_t, may be null): recorded at the
// attention kernel's own start and end (an extended launch).
int launch_gated_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const float* key_score, const float* gains, float temp_coef,
                           const int32_t* pos, int64_t n_kept, int hq, int hkv, int head_dim,
                           void* out, int out_dtype, float* lse, int lse_ld, void* stream,
                           void* start_event = nullptr, void* stop_event = nullptr);

// Workspace of the attention backward (fp32 arrays; row arrays padded to kp =
// n_kept rounded up to 32 rows): the recomputed forward output [n, hq, D], the
// per-row log2-sum-exp2 [hq, kp], D_t = dO.O [hq, kp], lambda_t and its exp2
// scale [kp], per-row partials of dc and dg [hq, kp], per-key partials of ds
// [hkv, kp].
struct AttnBwdWs {
    float* out;     // [n, hq, d] forward output, fp32
    float* lse;     // [hq][kp] forward per-row log2-sum-exp2
    float* rowv;    // [hq][kp] float4 per row: a_t, lse, D_t = dO.O, lambda_t
    float* dlamc;   // [hq][kp / 32] per-block partial of the temperature gradient
    float* dgp;     // [hq][kp / 32] per-block partial of the gain gradient
    float* dsp;     // [hkv][kp] per-kv-head partial of the score gradient
    int kp;
};
inline int64_t attn_bwd_kp(int64_t n) { return (n + 31) / 32 * 32; }
inline size_t attn_bwd_ws_bytes(int64_t n, int hq, int hkv, int d) {
    const size_t kp = (size_t)attn_bwd_kp(n);
    return align_up(sizeof(float) * (size_t)n * hq * d) + align_up(sizeof(float) * hq * kp) +
           align_up(4 * sizeof(float) * hq * kp) + 2 * align_up(sizeof(float) * hq * (kp / 32)) +
           align_up(sizeof(float) * hkv * kp);
}
inline AttnBwdWs attn_bwd_ws(void* base, int64_t n, int hq, int hkv, int d) {
    const size_t kp = (size_t)attn_bwd_kp(n);
    char* p = (char*)base;
    AttnBwdWs w;
    w.kp = (int)kp;
    w.out = (float*)p;
    p += align_up(sizeof(float) * (size_t)n * hq * d);
    w.lse = (float*)p;
    p += align_up(sizeof(float) * hq * kp);
    w.rowv = (float*)p;
    p += align_up(4 * sizeof(float) * hq * kp);
    w.dlamc = (float*)p;
    p += align_up(sizeof(float) * hq * (kp / 32));
    w.dgp = (float*)p;
    p += align_up(sizeof(float) * hq * (kp / 32));
    w.dsp = (float*)p;
    (void)hkv;
    return w;
}

int launch_gated_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* key_score,
                               const float* gains, float temp_coef, const int32_t* pos, int64_t n_kept, int hq,
                               int hkv, int head_dim, const uint16_t* dout, float* dq, float* dk, float* dv,
                               float* dscore, float* dgains, float* dtemp, void* workspace, void* stream);

// Backward of the scorer: per-wave row count and the workspace layout.
constexpr int kGateBwdRowsPerWave = 16;
inline int64_t gate_bwd_waves(int64_t n) { return (n + kGateBwdRowsPerWave - 1) / kGateBwdRowsPerWave; }
// dW1 = dz^T h is split over the tokens into this many equal chunks (plus a
// remainder chunk), summed afterwards in a fixed order.
inline int gate_bwd_splits(int64_t n) {
    const int64_t s = n / 2048;
    return (int)(s < 1 ? 1 : (s > 16 ? 16 : s));
}
struct GateBwdWs {
    float* dsh;     // [n] dense dshat
    float* sc;      // {1/rho, sequence-norm coefficient}
    float* z;       // [n, hd] h W1^T, fp32
    uint16_t* dz;   // [n, hd] bf16
    float* dw2p;    // [waves, hd] partials
    float* db1p;    // [waves, hd]
    float* db2p;    // [waves]
    float* w1p;     // [splits + 1, hd, d] partial dW1
};
inline size_t gate_bwd_ws_bytes(int64_t n, int hd, int d) {
    const size_t nw = (size_t)gate_bwd_waves(n);
    return align_up(sizeof(float) * (size_t)n) + align_up(2 * sizeof(float)) + align_up(sizeof(float) * (size_t)n * hd) +
           align_up(sizeof(uint16_t) * (size_t)n * hd) + 2 * align_up(sizeof(float) * nw * hd) +
           align_up(sizeof(float) * nw) + align_up(sizeof(float) * (size_t)(gate_bwd_splits(n) + 1) * hd * d);
}
inline GateBwdWs gate_bwd_ws(void* base, int64_t n, int hd, int d) {
    const size_t nw = (size_t)gate_bwd_waves(n);
    char* p = (char*)base;
    GateBwdWs w;
    w.dsh = (float*)p;
    p += align_up(sizeof(float) * (size_t)n);
    w.sc = (float*)p;
    p += align_up(2 * sizeof(float));
    w.z = (float*)p;
    p += align_up(sizeof(float) * (size_t)n * hd);
    w.dz = (uint16_t*)p;
    p += align_up(sizeof(uint16_t) * (size_t)n * hd);
    w.dw2p = (float*)p;
    p += align_up(sizeof(float) * nw * hd);
    w.db1p = (float*)p;
    p += align_up(sizeof(float) * nw * hd);
    w.db2p = (float*)p;
    p += align_up(sizeof(float) * nw);
    w.w1p = (float*)p;
    (void)d;
    return w;
}

int launch_gate_score_bwd(void* blas, const uint16_t* resid, const uint16_t* w1, const uint16_t* b1,
                          const uint16_t* w2, int64_t n, int d, int hd, float eps_row, float eps_seq,
                          const float* score_raw, const float* dscore_kept, const int32_t* kept_idx, int64_t k,
                          float* dresid, float* dw1, float* db1, float* dw2, float* db2, void* workspace,
                          void* stream);

// Column-major rocBLAS GEMM, bf16 A and B, fp32 C = D (in place when beta != 0):
// D[m x n] = op(A) op(B) + beta D, op = transpose when the flag is set.
int gemm_bf16_f32(void* handle, bool trans_a, bool trans_b, int m, int n, int k, const uint16_t* a, int lda,
                  const uint16_t* b, int ldb, float beta, float* d, int ldd, void* stream);
// The same with beta = 0 over `batch` equal problems at fixed strides.
int gemm_bf16_f32_batched(void* handle, bool trans_a, bool trans_b, int m, int n, int k, const uint16_t* a,
                          int lda, int64_t stride_a, const uint16_t* b, int ldb, int64_t stride_b, float* d, int ldd,
                          int64_t stride_d, int batch, void* stream);

int launch_gated_delta_rule(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha,
                            const float* beta, const float* state_in, int64_t n, int hk, int hv, int dk, int dv,
                            float* out, float* state_out, void* stream);

// The chunked form: a pre-pass writes each (v head, chunk of 32 tokens)'s
// state-independent transform into a 16 KB record of ws, then the state walks
// the chunks (gdn_chunk_ws_bytes(n, hv) bytes of workspace).
size_t gdn_chunk_ws_bytes(int64_t n, int hv);
int launch_gated_delta_rule_chunked(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha,
                                    const float* beta, const float* state_in, int64_t n, int hk, int hv, int dk,
                                    int dv, float* out, float* state_out, void* ws, void* stream);

int launch_rmsnorm(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t rows, int dim, float eps,
                   void* stream);

int launch_swiglu(const uint16_t* gu, uint16_t* out, int64_t rows, int inter, void* stream);

int blas_create(void** handle);
int blas_destroy(void* handle);
int linear(void* handle, const uint16_t* x, const uint16_t* w, const uint16_t* residual, uint16_t* y, int64_t rows,
           int in_dim, int out_dim, void* stream);

}  // namespace tgi
