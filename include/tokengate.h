/*
 * tokengate.h -- C ABI of the TokenGate gated-prefill hot path on MI355X (gfx950).
 *
 * The path runs at the gate layer L of a decoder and in the layers above it:
 *   tg_gate_score      -> a small MLP scores every token's normalised residual,
 *                         and the scores are RMS-normalised along the sequence;
 *   tg_select_topk     -> forced-keep top-K picks the tokens that continue
 *                         (tg_gate_score_select: scorer and select in one call);
 *   tg_compact         -> the kept rows, their original positions, their scores
 *                         and any extra per-token streams (KV rows) are gathered;
 *   tg_rope, tg_rope_qk -> (auxiliary) rotary embedding at the original positions;
 *   tg_gated_attention -> causal attention over the kept tokens only, with a
 *                         per-key importance bias and a per-query temperature.
 * Training-side gradients: tg_gated_attention_bwd, tg_gate_score_bwd.  The
 * hybrid backbone's recurrent mixer over the kept tokens: tg_gated_delta_rule
 * (a scan over the tokens) and tg_gated_delta_rule_chunked (in chunks on the
 * matrix cores, with a workspace).
 * The rest of an upper decoder layer on the kept rows (see the section at the
 * end): tg_rmsnorm, tg_swiglu, and tg_linear (a rocBLAS GEMM through a handle
 * from tg_blas_create).
 *
 * Sources (web pages on the method; cited by the key in brackets):
 *  [P1] fluxbbs.com, "TokenGate 长上下文预填充提速 11.3 倍，斯坦福伯克利开源门控剪枝":
 *       section "门控到底插在模型的哪个位置" (where the gate sits) and section
 *       "端到端训练的关键在 token 门控注意力" (token-gated attention).
 *  [P2] slinene.github.io paper digest, "TokenGate: Adapting LLMs for Fast and
 *       Memory-Efficient Prefill with Learned Token Pruning": "方法关键点".
 *  [P3] news.farwalk.ai, "斯坦福与 UC Berkeley 提出 TokenGate ...": "How does
 *       TokenGate learned token pruning work?", "What is token-gated attention?",
 *       "How do you deploy TokenGate?".
 *  [P5] aiwillknow.com, "TokenGate：让模型学会跳读，而不只压缩 KV 缓存":
 *       Figure 1(a)(b) and Figure 1(c) descriptions.
 *
 * Conventions for every entry point:
 *  - bf16 tensors are passed as uint16_t bit patterns (tg_bf16).
 *  - Every tensor pointer is DEVICE memory owned by the caller; the library
 *    allocates nothing, keeps no state between calls, never synchronises the
 *    stream and never reads device data back to the host.  (The one
 *    exception is the rocBLAS handle of tg_linear and tg_gate_score_bwd, which the caller creates
 *    and destroys explicitly with tg_blas_create / tg_blas_destroy.)  Work is enqueued on
 *    `stream` (a hipStream_t passed as void*; NULL = the null stream) and is
 *    complete when the stream reaches that point.
 *  - Arguments are checked on the host before anything is enqueued; a
 *    negative status means nothing was enqueued (except TG_EDEVICE, which
 *    reports a launch failure).
 *  - Layouts are row-major and dense unless a stride is given.
 *  - Outputs must not overlap inputs, the workspace or each other, except
 *    where an entry point says otherwise (in-place RoPE, tg_linear's
 *    residual, tg_gated_delta_rule's state).
 *  - Batch size is 1 (one prompt per call), as in the pages' measurements.
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t tg_bf16;

/* Status codes. */
#define TG_OK 0
#define TG_EINVAL (-1)        /* a size, budget or required pointer is invalid */
#define TG_EUNSUPPORTED (-2)  /* a shape the kernels do not implement */
#define TG_EALIGN (-3)        /* a pointer, row size or stride is not 16-byte aligned */
#define TG_EWORKSPACE (-4)    /* workspace missing or smaller than tg_workspace_bytes */
#define TG_EDEVICE (-5)       /* the HIP runtime rejected a launch */

/* Bits written to the optional device status word of tg_select_topk. */
#define TG_STATUS_FORCED_MISMATCH 1  /* forced-mask count differs from n_forced */
#define TG_STATUS_FORCED_OVER_K 2    /* more forced tokens than k: only k kept */

/* Upper limit on extra gather streams in one tg_compact call. */
#define TG_MAX_GATHER 16

/* Human-readable text for a status code (static storage; never NULL). */
const char* tg_status_string(int status);

/* ABI version of this header (incremented on incompatible change). */
int tg_abi_version(void);

/* Bytes of device workspace that tg_gate_score and tg_select_topk need for a
 * prompt of n tokens.  Both take the same size; one buffer may serve both
 * (not concurrently).  Alignment: 256 bytes. */
size_t tg_workspace_bytes(int64_t n);

/*
 * tg_gate_score -- gate scoring network plus sequence RMSNorm
 * [P1 gate][P2 method][P3 how][P5 Fig 1(a)(b)].
 *   r_i  = 1 / sqrt(mean_k resid_ik^2 + eps_row)
 *   a_ij = r_i * sum_k resid_ik w1_jk + b1_j
 *   s_i  = sum_j w2_j GELU(a_ij) + b2
 *   GELU is the erf form a/2 (1 + erf(a/sqrt 2)); erf is evaluated to an
 *   absolute error of at most 1.5e-7 (not correctly rounded).
 *   score_norm_i = s_i / sqrt(mean_i s_i^2 + eps_seq)
 * resid      [n, d] bf16: post-attention residual of layer L (row stride d).
 * w1         [hd, d] bf16: first scorer layer, with the elementwise weight of
 *            the normalisation folded in by the caller (w1_jk * gamma_k).
 * b1         [hd] bf16 or NULL (= 0).   w2 [hd] bf16.   b2: output bias.
 * score_norm [n] fp32 out: normalised scores.
 * score_raw  [n] fp32 out: raw scores s, or NULL.
 * Supported: d % 64 == 0, hd in {64, 128, 256}; resid, w1 16-byte aligned.
 * n == 0 is a no-op.  Workspace: tg_workspace_bytes(n).
 * Results are deterministic (fixed reduction order, no float atomics).
 */
int tg_gate_score(const tg_bf16* resid, const tg_bf16* w1, const tg_bf16* b1, const tg_bf16* w2,
                  float b2, int64_t n, int32_t d, int32_t hd, float eps_row, float eps_seq,
                  float* score_norm, float* score_raw, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * tg_gate_score_noalloc -- tg_gate_score for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): same arguments, results and checks, bit for bit,
 * without the workspace.  Its scratch (the per-workgroup partial sums) is a
 * fixed device array inside the library, one per device, located on the
 * first call on each device (with that device current; the stream must
 * belong to it).  Limit: n <= TG_NOALLOC_MAX_TOKENS, else TG_EUNSUPPORTED.
 * Every call on one device shares that device's array: calls that overlap on
 * one device (concurrent streams or threads) race and must not be issued;
 * calls ordered on one stream are safe (each overwrites the array).  Returns
 * TG_EDEVICE if the array's address cannot be obtained.
 */
#define TG_NOALLOC_MAX_TOKENS (1 << 22)
int tg_gate_score_noalloc(const tg_bf16* resid, const tg_bf16* w1, const tg_bf16* b1, const tg_bf16* w2,
                          float b2, int64_t n, int32_t d, int32_t hd, float eps_row, float eps_seq,
                          float* score_norm, float* score_raw, void* stream);

/*
 * tg_select_topk -- forced-keep top-K [P1 gate][P2 method][P3 how][P5 Fig 1(a)(b)].
 * Keeps every token with forced[i] != 0 and, among the others, the
 * k - F with the largest score (ties to the lower index; -0.0 equals +0.0;
 * NaN ranks below -inf).  k counts all kept tokens, forced ones included.
 * score    [n] fp32, 16-byte aligned.  forced [n] uint8 (4-byte aligned) or NULL
 *          (no forced tokens).
 * n_forced host-known number of forced tokens F (checked: 0 <= F <= k <= n, k >= 1).
 * kept_idx [k] int32 out: kept indices in ascending order.
 * dev_status optional device int32: receives TG_STATUS_* bits (0 = consistent).
 *   The kernels use the forced count they find on the device; if it exceeds
 *   k, the first k forced tokens are kept and TG_STATUS_FORCED_OVER_K is set.
 * Workspace: tg_workspace_bytes(n).
 */
int tg_select_topk(const float* score, const uint8_t* forced, int64_t n, int64_t n_forced,
                   int64_t k, int32_t* kept_idx, int32_t* dev_status, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * tg_gate_score_select -- tg_gate_score, then tg_select_topk on its
 * normalised scores, in one call [P1 gate][P2 method][P3 how][P5 Fig 1(a)(b)]:
 * the same score_norm, score_raw, kept_idx and dev_status as the two calls,
 * bit for bit.  Up to 524288 tokens the sequence norm runs inside the
 * select's first launch (one launch fewer: the one-workgroup select up to
 * 16384 tokens, the first of the many-workgroup select's three launches
 * above); longer prompts take the two calls' kernels.  Arguments: those of
 * tg_gate_score and tg_select_topk
 * (score_norm must also be 16-byte aligned); checks: both calls' checks
 * (n >= 1).  Workspace: tg_workspace_bytes(n).
 */
int tg_gate_score_select(const tg_bf16* resid, const tg_bf16* w1, const tg_bf16* b1, const tg_bf16* w2, float b2,
                         int64_t n, int32_t d, int32_t hd, float eps_row, float eps_seq, const uint8_t* forced,
                         int64_t n_forced, int64_t k, float* score_norm, float* score_raw, int32_t* kept_idx,
                         int32_t* dev_status, void* workspace, size_t workspace_bytes, void* stream);

/* One extra per-token row stream for tg_compact: dst row t = src row kept_idx[t]. */
typedef struct tg_gather {
    const void* src;     /* device, src_stride bytes between rows, >= n rows */
    void* dst;           /* device, dst_stride bytes between rows, >= k rows */
    int64_t row_bytes;   /* bytes copied per row (multiple of 16) */
    int64_t src_stride;  /* multiple of 16 */
    int64_t dst_stride;  /* multiple of 16 */
} tg_gather;

/*
 * tg_compact -- residual truncation and compaction [P1 gate][P3 how][P5 Fig 1(a)(b)]:
 * pruned tokens stop at layer L; the kept ones continue with their original
 * position ids, and KV rows are kept for them only.
 *   resid_out[t] = resid[kept_idx[t]]   ([k, d] bf16; skipped if resid is NULL)
 *   pos_out[t]   = pos[kept_idx[t]]     (pos NULL = identity: pos_out[t] = kept_idx[t])
 *   score_out[t] = score[kept_idx[t]]   (skipped if score is NULL)
 *   extra[e]: row gather as described by tg_gather (host array of n_extra <= 16).
 * kept_idx values must lie in [0, n); a row whose index does not is left unwritten.
 * Copies are bit-exact.  k == 0 is a no-op.
 */
int tg_compact(const int32_t* kept_idx, int64_t k, int64_t n, const tg_bf16* resid,
               tg_bf16* resid_out, int32_t d, const int32_t* pos, int32_t* pos_out,
               const float* score, float* score_out, const tg_gather* extra, int32_t n_extra,
               void* stream);

/*
 * tg_rope -- rotary embedding at original positions, in place (auxiliary;
 * [P5 Fig 1(a)(b)]: kept tokens keep their original position encoding).
 * x [rows, heads, head_dim] bf16, pos [rows] int32 >= 0.  Half-split pairs
 * (j, j + head_dim/2), angle pos * theta^(-2j/head_dim), evaluated in fp64 and
 * rounded to bf16 (nearest-even) once.  head_dim even, <= 256.
 */
int tg_rope(tg_bf16* x, const int32_t* pos, int64_t rows, int32_t heads, int32_t head_dim,
            double theta, void* stream);

/*
 * tg_rope_qk -- tg_rope on the query and key rows of one upper layer in one
 * launch (auxiliary; [P5 Fig 1(a)(b)]): q [rows, hq, head_dim] and
 * k [rows, hk, head_dim] bf16, both rotated in place at the same original
 * positions pos [rows] int32 >= 0.  Same convention, precision and limits as
 * tg_rope (hq, hk >= 1); the results equal two tg_rope calls bit for bit.
 * q and k must not overlap.
 */
int tg_rope_qk(tg_bf16* q, tg_bf16* k, const int32_t* pos, int64_t rows, int32_t hq, int32_t hk,
               int32_t head_dim, double theta, void* stream);

/*
 * tg_gated_attention -- token-gated causal attention over the kept list, one
 * upper layer [P1 tga][P2 method][P3 tga][P5 Fig 1(c)].  For q head h (kv head
 * h / (hq/hkv)), query row t and keys j <= t:
 *   z_tj     = lambda_t * (q_t . k_j / sqrt(head_dim) + gains[h] * key_score[j])
 *   lambda_t = 1 + temp_coef * ln((t + 1) / (pos[t] + 1))
 *   out_t    = sum_j softmax_j(z_tj) v_j
 * q [n_kept, hq, head_dim], k / v [n_kept, hkv, head_dim] bf16 (16-byte aligned);
 * key_score [n_kept] fp32 (normalised score of each kept token); gains [hq] fp32;
 * pos [n_kept] int32 original positions (>= 0, increasing).
 * out [n_kept, hq, head_dim]: bf16 if out_dtype == 0, fp32 if out_dtype == 1.
 * Supported: head_dim in {64, 128}, hq % hkv == 0, and K and V each under
 * 2 GiB (n_kept * hkv * head_dim * 2 < 2^31; else TG_EUNSUPPORTED).
 * n_kept == 0 is a no-op.
 * bf16 matrix-core products with fp32 accumulation; softmax in fp32.
 */
int tg_gated_attention(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v,
                       const float* key_score, const float* gains, float temp_coef,
                       const int32_t* pos, int64_t n_kept, int32_t hq, int32_t hkv,
                       int32_t head_dim, void* out, int32_t out_dtype, void* stream);

/*
 * tg_gated_attention_timed -- tg_gated_attention (same arguments, checks and
 * results, bit for bit) for measuring the attention kernel alone: the launch
 * also records start_event and stop_event (hipEvent_t, created by the caller
 * with timing enabled, owned by the caller; either may be NULL) at the
 * kernel's own start and end, so hipEventElapsedTime(start, stop) leaves out
 * the queue's dispatch gap that events recorded around the call take in.
 * Nothing is recorded when n_kept == 0 or a check fails.
 */
int tg_gated_attention_timed(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v,
                             const float* key_score, const float* gains, float temp_coef,
                             const int32_t* pos, int64_t n_kept, int32_t hq, int32_t hkv,
                             int32_t head_dim, void* out, int32_t out_dtype, void* stream,
                             void* start_event, void* stop_event);

/*
 * tg_attention_bwd_workspace_bytes -- device workspace of tg_gated_attention_bwd
 * (256-byte aligned): about 4 * n_kept * hq * head_dim bytes plus per-row
 * arrays.
 */
size_t tg_attention_bwd_workspace_bytes(int64_t n_kept, int32_t hq, int32_t hkv, int32_t head_dim);

/*
 * tg_gated_attention_bwd -- gradients of tg_gated_attention [P1 tga][P2 method]
 * [P3 tga][P5 Fig 1(c)]: the gate is trained through the upper layers'
 * attention, whose key bias and gains carry the score gradient.  With
 * U_tj = q_t.k_j/sqrt(head_dim) + gains[h] key_score[j], Z = lambda_t U and
 * P = softmax_j(Z) (the forward above), given dout = dL/dO:
 *   dq [n_kept, hq, head_dim], dk / dv [n_kept, hkv, head_dim]  (fp32 out)
 *   dscore [n_kept]  = dL/dkey_score   (fp32 out; sums over all heads)
 *   dgains [hq]      = dL/dgains       (fp32 out)
 *   dtemp  [1]       = dL/dtemp_coef   (fp32 out)
 * Inputs as in tg_gated_attention (q, k, v, key_score, gains, temp_coef, pos,
 * same shapes and limits); dout [n_kept, hq, head_dim] bf16 (16-byte
 * aligned).  Q and dout must also each stay under 2 GiB
 * (n_kept * hq * head_dim * 2 < 2^31; else TG_EUNSUPPORTED).  Every output
 * is overwritten (nothing accumulates across calls).
 * The forward is recomputed (fp32, with its per-row log-sum-exp) into the
 * workspace; probabilities are rebuilt per 32x32 block, never stored.
 * bf16 matrix-core products with fp32 accumulation; deterministic (fixed
 * reduction orders, no atomics).  n_kept == 0 is a no-op.
 */
int tg_gated_attention_bwd(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* key_score,
                           const float* gains, float temp_coef, const int32_t* pos, int64_t n_kept, int32_t hq,
                           int32_t hkv, int32_t head_dim, const tg_bf16* dout, float* dq, float* dk, float* dv,
                           float* dscore, float* dgains, float* dtemp, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * tg_gate_score_bwd_workspace_bytes -- device workspace of tg_gate_score_bwd
 * (256-byte aligned): about 6 * n * hd bytes, per-row arrays and up to 17
 * partial copies of dw1 (4 * hd * d bytes each).
 */
size_t tg_gate_score_bwd_workspace_bytes(int64_t n, int32_t d, int32_t hd);

/*
 * tg_gate_score_bwd -- gradients of tg_gate_score's normalised scores with
 * respect to the residual and the scorer's weights [P1 gate][P1 tga]
 * [P2 method][P5 Fig 1(a)(b)]: the gate is trained end to end through the
 * attention bias of the kept tokens, so the incoming gradient is
 * dscore_kept[t] = dL/dscore_norm[kept_idx[t]] (what tg_gated_attention_bwd
 * returns as dscore, in kept order) and zero for every pruned token.
 * With the forward of tg_gate_score (r_i, a_ij, s_i, rho as documented there):
 *   ds_i   = dshat_i / rho - s_i (sum_m dshat_m s_m) / (n rho^3)
 *   dw2_j  = sum_i ds_i GELU(a_ij),   db2 = sum_i ds_i
 *   da_ij  = ds_i w2_j GELU'(a_ij),   db1_j = sum_i da_ij
 *   dw1    = (r da)^T resid
 *   dresid_i = (r_i da_i) w1 - (sum_j da_ij (resid_i . w1_j)) r_i^3 resid_i / d
 * blas: a handle from tg_blas_create (three rocBLAS GEMMs run through it:
 *   resid w1^T again, the w1 product of dresid and dw1).
 * resid, w1, b1 (or NULL), w2, n, d, hd, eps_row, eps_seq: as given to
 *   tg_gate_score.  score_raw [n] fp32: its raw-score output.
 * dscore_kept [k] fp32, kept_idx [k] int32: distinct indices in [0, n)
 *   (entries outside are skipped); k may be 0 (then only the pruned-token
 *   paths remain and every gradient is zero).
 * dresid [n, d] fp32 out, dw1 [hd, d] fp32 out (both 16-byte aligned), db1 [hd],
 *   dw2 [hd], db2 [1] fp32 out; all overwritten.  db1 is written also when
 *   b1 is NULL (the gradient of a zero bias).
 * Supported: hd in {64, 128, 256}; d % 64 == 0, 64 <= d <= 4096; resid
 * 16-byte aligned.  n == 0 is a no-op.  dz = r da enters the two gradient
 * GEMMs in bf16 (fp32 accumulation); the rest is fp32 with fp64 sums.
 * Deterministic: fixed reduction orders, and the handle's GEMMs run with
 * atomics disabled.
 */
int tg_gate_score_bwd(void* blas, const tg_bf16* resid, const tg_bf16* w1, const tg_bf16* b1, const tg_bf16* w2,
                      int64_t n, int32_t d, int32_t hd, float eps_row, float eps_seq, const float* score_raw,
                      const float* dscore_kept, const int32_t* kept_idx, int64_t k, float* dresid, float* dw1,
                      float* db1, float* dw2, float* db2, void* workspace, size_t workspace_bytes, void* stream);

/*
 * tg_gated_delta_rule -- the recurrent mixer of the hybrid backbone over a
 * token sequence [P1 hybrid][P3 hybrid FAQ][P5 hybrid state]: in a hybrid
 * (Gated-DeltaNet + attention) backbone the gate may follow a recurrent
 * layer, and above it the recurrent mixers see only the kept tokens, in
 * order, while the lower layers' state has read every token.  The mixer's
 * core is the gated delta rule (Yang, Kautz and Hatamizadeh, "Gated Delta
 * Networks", 2024), per v head h with state S [dv, dk]:
 *   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *   out_t = S_t q_t.
 * q, k   [n, hk, dk] bf16 (16-byte aligned); v head h uses q/k head
 *        h / (hv / hk).  The mixer normalises q and k before this step; keys
 *        with |k| > 1 make the recurrence expansive.
 * v      [n, hv, dv] bf16.   alpha, beta [n, hv] fp32 (decay in (0, 1],
 *        write strength in [0, 1]).
 * state_in  [hv, dv, dk] fp32 or NULL (= zeros); state_out [hv, dv, dk] fp32
 *        or NULL (the state after the last token; may equal state_in).
 *        Both 16-byte aligned.
 * out    [n, hv, dv] fp32.
 * Supported: dk, dv in {64, 128}; hv % hk == 0; n * hk * dk and n * hv * dv
 * below 2^30.  n == 0 copies state_in (or zeros) to state_out if given.  fp32
 * state and arithmetic; deterministic.  The scan is sequential over tokens:
 * one workgroup per 8 rows of a head's state, tokens staged through LDS in
 * chunks of 32.
 */
int tg_gated_delta_rule(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* alpha, const float* beta,
                        const float* state_in, int64_t n, int32_t hk, int32_t hv, int32_t dk, int32_t dv, float* out,
                        float* state_out, void* stream);

/*
 * tg_gated_delta_rule_chunked -- tg_gated_delta_rule in chunks of 32 tokens on
 * the matrix cores (the chunkwise WY / UT form of the Gated Delta Networks
 * paper): the same arguments, checks and definition, plus a workspace.  A
 * pre-pass forms every chunk's state-independent transform at once (Gram
 * products, decay table, the inverse of the chunk's unit lower-triangular
 * system) and writes it to the workspace, one 16 KB record per (v head,
 * chunk); then the state walks the chunks, one workgroup per 16 rows of a
 * head's state.  fp32 operands enter the bf16 matrix cores split into three
 * parts (fp32-level products); the results agree with tg_gated_delta_rule to
 * rounding, not bit for bit.  Deterministic.  A run split at a multiple of 32
 * tokens with the state carried over equals one run bit for bit.
 * workspace: tg_gated_delta_rule_workspace_bytes(n, hv) bytes, 16-byte
 * aligned, overwritten (no contents need clearing); not needed when n == 0.
 */
size_t tg_gated_delta_rule_workspace_bytes(int64_t n, int32_t hv);
int tg_gated_delta_rule_chunked(const tg_bf16* q, const tg_bf16* k, const tg_bf16* v, const float* alpha,
                                const float* beta, const float* state_in, int64_t n, int32_t hk, int32_t hv,
                                int32_t dk, int32_t dv, float* out, float* state_out, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * ---- Upper decoder layer on the kept rows ----
 * Above the gate only the kept tokens go through the backbone's layers
 * [P1 gate][P5 Fig 1(a)(b)].  With a Qwen3-shaped backbone a layer is:
 *   x = rmsnorm(h, w_in); q, k, v = linear(x, Wq / Wk / Wv);
 *   q, k = rmsnorm per head (w_qn, w_kn); rope at the original positions;
 *   a = gated attention; h2 = linear(a, Wo) + h;
 *   x2 = rmsnorm(h2, w_post); h3 = linear(swiglu(linear(x2, Wgu)), Wdown) + h2.
 * These three entry points are the pieces not covered above; a caller chains
 * them with tg_rope_qk and tg_gated_attention.
 */

/*
 * tg_rmsnorm -- y_r = x_r / sqrt(mean_k x_rk^2 + eps) * weight, per row.
 * x, y [rows, dim] bf16 (y may equal x); weight [dim] bf16.  fp32 arithmetic,
 * one rounding to bf16 (nearest-even).  A per-head norm is the same call with
 * rows = tokens * heads and dim = head_dim.
 * Supported: dim % 8 == 0 and 8 <= dim <= 4096; x, y, weight 16-byte aligned.
 * rows == 0 is a no-op.
 */
int tg_rmsnorm(const tg_bf16* x, const tg_bf16* weight, tg_bf16* y, int64_t rows, int32_t dim, float eps,
               void* stream);

/*
 * tg_swiglu -- out_r = silu(g_r) * u_r with silu(g) = g / (1 + e^-g), where
 * g_r and u_r are the first and second halves of row r of gate_up.
 * gate_up [rows, 2 * inter] bf16, out [rows, inter] bf16 (no overlap).  fp32
 * arithmetic, one rounding to bf16.  Supported: inter % 8 == 0; both 16-byte
 * aligned.  rows == 0 is a no-op.
 */
int tg_swiglu(const tg_bf16* gate_up, tg_bf16* out, int64_t rows, int32_t inter, void* stream);

/*
 * tg_blas_create / tg_blas_destroy -- a rocBLAS handle for tg_linear (and
 * tg_gate_score_bwd), created with atomics disabled.  The
 * handle is the one piece of library-side state and allocation: the caller
 * creates it once per device (with that device current), owns it, and
 * destroys it; calls that share a handle must not run concurrently from
 * several host threads.  Returns TG_EDEVICE if rocBLAS fails.
 */
int tg_blas_create(void** handle);
int tg_blas_destroy(void* handle);

/*
 * tg_linear -- y = x . W^T (+ residual): x [rows, in_dim], W [out_dim, in_dim]
 * (row-major, the usual weight layout), residual NULL or [rows, out_dim], y
 * [rows, out_dim], all bf16; fp32 accumulation, one rounding of the sum (with
 * the residual) to bf16.  A library GEMM (rocBLAS gemm_ex) on `stream`.
 * y must not overlap x or W; it may equal residual.  rows, in_dim, out_dim
 * >= 1 and below 2^31.
 */
int tg_linear(void* handle, const tg_bf16* x, const tg_bf16* w, const tg_bf16* residual, tg_bf16* y,
              int64_t rows, int32_t in_dim, int32_t out_dim, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_H */
