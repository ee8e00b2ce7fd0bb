/*
 * tg_oracle.c -- plain fp64 CPU reference of the TokenGate gated-prefill path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP
 * library: the two meet only in the seeded inputs.
 *
 * Arithmetic is IEEE double on the exact values of the bf16/fp32 inputs, in
 * plain loops, one output element at a time, with no blocking or reordering.
 * Threads only split independent rows; a row's arithmetic does not depend on
 * the thread count.  Build with -ffp-contract=off and without -ffast-math.
 *
 * Sources (web pages on the method; cited by the key in brackets):
 *  [P1] fluxbbs.com, "TokenGate 长上下文预填充提速 11.3 倍，斯坦福伯克利开源门控剪枝":
 *       section "门控到底插在模型的哪个位置" (where the gate sits) and section
 *       "端到端训练的关键在 token 门控注意力" (token-gated attention).
 *  [P2] slinene.github.io paper digest, "TokenGate: Adapting LLMs for Fast and
 *       Memory-Efficient Prefill with Learned Token Pruning": section "方法关键点".
 *  [P3] news.farwalk.ai, "斯坦福与 UC Berkeley 提出 TokenGate ...": sections
 *       "How does TokenGate learned token pruning work?" and
 *       "What is token-gated attention?".
 *  [P5] aiwillknow.com, "TokenGate：让模型学会跳读，而不只压缩 KV 缓存":
 *       Figure 1(a)(b) and Figure 1(c) descriptions.
 *
 * Readings where the pages leave the arithmetic open (each is a spec choice,
 * "parity unpinned" against the pages, which print no worked example):
 *  - row RMSNorm epsilon and sequence RMSNorm epsilon are arguments (1e-6 in
 *    the workloads); the norm's elementwise weight is folded into W1;
 *  - the sequence RMSNorm has no learnable scale;
 *  - GELU is the exact-erf form;
 *  - temperature: lambda_t = 1 + c * ln((t+1)/(pos_t+1)), scaling the whole
 *    logit (dot-product term and bias);
 *  - forced-keep keys get their own normalised score as bias;
 *  - top-K ties go to the lower index; NaN ranks below -inf; -0 equals +0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ threads */

typedef void (*tgo_range_fn)(void* ctx, int64_t begin, int64_t end);

typedef struct {
    tgo_range_fn fn;
    void* ctx;
    int64_t total, chunk;
    int64_t next; /* shared work counter */
} tgo_pool;

static void* tgo_worker(void* p) {
    tgo_pool* pool = (tgo_pool*)p;
    for (;;) {
        int64_t b = __atomic_fetch_add(&pool->next, pool->chunk, __ATOMIC_RELAXED);
        if (b >= pool->total) break;
        int64_t e = b + pool->chunk < pool->total ? b + pool->chunk : pool->total;
        pool->fn(pool->ctx, b, e);
    }
    return NULL;
}

/* Run fn over [0, total) in small chunks handed out to nthreads workers.
 * Each unit of work is computed by exactly one call, the same way whatever
 * the thread count, so results do not depend on it. */
static void tgo_parallel(tgo_range_fn fn, void* ctx, int64_t total, int nthreads) {
    if (total <= 0) return;
    if (nthreads < 1) nthreads = 1;
    tgo_pool pool = {fn, ctx, total, 1, 0};
    pool.chunk = total / ((int64_t)nthreads * 16);
    if (pool.chunk < 1) pool.chunk = 1;
    if (nthreads == 1) {
        fn(ctx, 0, total);
        return;
    }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, tgo_worker, &pool) != 0) break;
        ++started;
    }
    tgo_worker(&pool); /* the caller works too; also covers a failed start */
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    free(th);
}

/* ------------------------------------------------------- S1-S3: the scorer */
/*
 * Gate scoring network [P1 gate][P2 method][P5 Fig 1(a)(b)]: each token's
 * post-attention residual h_i at the gate layer is RMS-normalised and fed to
 * a small MLP that returns one scalar.
 *   r_i  = 1 / sqrt( (1/d) sum_k h_ik^2 + eps_row )
 *   a_ij = r_i * sum_k h_ik W1_jk + b1_j
 *   u_ij = GELU(a_ij) = a_ij * (1 + erf(a_ij / sqrt 2)) / 2
 *   s_i  = sum_j w2_j u_ij + b2
 */
typedef struct {
    const double *h, *w1, *b1, *w2;
    double b2, eps_row;
    int64_t d, hd;
    double* s;
} tgo_score_ctx;

static void tgo_score_rows(void* p, int64_t begin, int64_t end) {
    const tgo_score_ctx* c = (const tgo_score_ctx*)p;
    for (int64_t i = begin; i < end; ++i) {
        const double* hi = c->h + i * c->d;
        double ss = 0.0;
        for (int64_t k = 0; k < c->d; ++k) ss += hi[k] * hi[k];
        double r = 1.0 / sqrt(ss / (double)c->d + c->eps_row);
        double acc = 0.0;
        for (int64_t j = 0; j < c->hd; ++j) {
            const double* wj = c->w1 + j * c->d;
            double dot = 0.0;
            for (int64_t k = 0; k < c->d; ++k) dot += hi[k] * wj[k];
            double a = r * dot + (c->b1 ? c->b1[j] : 0.0);
            double u = 0.5 * a * (1.0 + erf(a / sqrt(2.0)));
            acc += c->w2[j] * u;
        }
        c->s[i] = acc + c->b2;
    }
}

void tgo_score_mlp(const double* h, const double* w1, const double* b1, const double* w2,
                   double b2, int64_t n, int64_t d, int64_t hd, double eps_row,
                   double* s_out, int nthreads) {
    tgo_score_ctx c = {h, w1, b1, w2, b2, eps_row, d, hd, s_out};
    tgo_parallel(tgo_score_rows, &c, n, nthreads);
}

/* --------------------------------------------- S4: sequence-wise RMSNorm */
/*
 * The scores are RMSNorm-normalised along the sequence [P1 gate][P2 method]:
 *   rho = sqrt( (1/n) sum_i s_i^2 + eps_seq ),   s^_i = s_i / rho.
 * Reading: all n tokens (forced-keep included) enter the mean; no learnable
 * scale (a scalar gain would be absorbed by the per-head attention gains).
 */
double tgo_seq_rmsnorm(const double* s, int64_t n, double eps_seq, double* out) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += s[i] * s[i];
    double rho = sqrt(ss / (double)n + eps_seq);
    for (int64_t i = 0; i < n; ++i) out[i] = s[i] / rho;
    return rho;
}

/* ------------------------------------------------- S5: forced-keep top-K */
/*
 * Top-K selector with a forced-keep set [P1 gate][P2 method][P3 how][P5 Fig 1(a)(b)]:
 * question / instruction tokens are never pruned; among the prunable tokens
 * the K - F best by score are kept.  K counts every kept token.
 * Order: score descending, then index ascending (ties to the lower index).
 * NaN ranks below every number; -0.0 and +0.0 compare equal.
 * Output: the kept indices, ascending (sequence order).
 * Returns 0, or -1 when the budget is infeasible (k < 1, k > n, or more
 * forced tokens than k).
 */
typedef struct {
    double s;
    int64_t i;
} tgo_scored;

static int tgo_rank_cmp(const void* pa, const void* pb) {
    const tgo_scored* a = (const tgo_scored*)pa;
    const tgo_scored* b = (const tgo_scored*)pb;
    int an = isnan(a->s), bn = isnan(b->s);
    if (an != bn) return an ? 1 : -1;
    if (!an) {
        if (a->s > b->s) return -1;
        if (a->s < b->s) return 1;
    }
    return (a->i < b->i) ? -1 : (a->i > b->i ? 1 : 0);
}

int tgo_select_topk(const double* score, const uint8_t* forced, int64_t n, int64_t k,
                    int32_t* kept) {
    if (n < 1 || k < 1 || k > n) return -1;
    int64_t n_forced = 0;
    for (int64_t i = 0; i < n; ++i) n_forced += (forced && forced[i]) ? 1 : 0;
    if (n_forced > k) return -1;
    int64_t n_prunable = n - n_forced;
    tgo_scored* cand = (tgo_scored*)malloc(sizeof(tgo_scored) * (size_t)(n_prunable > 0 ? n_prunable : 1));
    uint8_t* keep = (uint8_t*)calloc((size_t)n, 1);
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (forced && forced[i]) {
            keep[i] = 1;
        } else {
            cand[m].s = score[i];
            cand[m].i = i;
            ++m;
        }
    }
    qsort(cand, (size_t)m, sizeof(tgo_scored), tgo_rank_cmp);
    int64_t take = k - n_forced;
    for (int64_t r = 0; r < take; ++r) keep[cand[r].i] = 1;
    int64_t t = 0;
    for (int64_t i = 0; i < n; ++i)
        if (keep[i]) kept[t++] = (int32_t)i;
    free(cand);
    free(keep);
    return 0;
}

/* ------------------------------------------------------- S6: compaction */
/*
 * Pruned tokens stop at the gate layer; kept rows continue with their
 * original position ids [P1 gate][P3 how][P5 Fig 1(a)(b)]:
 * dst[t] = src[idx[t]], row by row, byte for byte.
 */
void tgo_gather_rows(const void* src, int64_t src_stride, int64_t row_bytes,
                     const int32_t* idx, int64_t k, void* dst, int64_t dst_stride) {
    const unsigned char* s = (const unsigned char*)src;
    unsigned char* o = (unsigned char*)dst;
    for (int64_t t = 0; t < k; ++t)
        memcpy(o + t * dst_stride, s + (int64_t)idx[t] * src_stride, (size_t)row_bytes);
}

/* ------------------------------------------------------------- S7: RoPE */
/*
 * Rotary embedding at the original positions of the kept tokens
 * ([P5 Fig 1(a)(b)]: original position encoding kept).  Half-split pairing
 * (x_j, x_{j+D/2}), frequency theta^(-2j/D), angle = pos * frequency.
 * Unrounded fp64 output; tgo_to_bf16 rounds it.
 */
void tgo_rope(const double* x, const int32_t* pos, int64_t rows, int64_t heads, int64_t D,
              double theta, double* out) {
    int64_t half = D / 2;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t h = 0; h < heads; ++h) {
            const double* xi = x + (r * heads + h) * D;
            double* yo = out + (r * heads + h) * D;
            for (int64_t j = 0; j < half; ++j) {
                double f = pow(theta, -2.0 * (double)j / (double)D);
                double phi = (double)pos[r] * f;
                double c = cos(phi), s = sin(phi);
                yo[j] = xi[j] * c - xi[j + half] * s;
                yo[j + half] = xi[j + half] * c + xi[j] * s;
            }
        }
    }
}

/* Round to the nearest bfloat16, ties to even, directly from double. */
static uint16_t tgo_bf16_of(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    int e;
    double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    if (e >= -125) {          /* a >= 2^-126: normal bf16 range */
        double r = nearbyint(ldexp(m, 8)); /* 8 significant bits, in [128, 256] */
        if (r == 256.0) {
            r = 128.0;
            e += 1;
        }
        int biased = (e - 1) + 127;
        if (biased >= 255) return (uint16_t)(sign | 0x7F80);
        return (uint16_t)(sign | (uint16_t)(biased << 7) | (uint16_t)((int)r - 128));
    }
    double q = nearbyint(ldexp(a, 133)); /* subnormal quantum 2^-133 */
    return (uint16_t)(sign | (uint16_t)q);
}

void tgo_to_bf16(const double* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = tgo_bf16_of(x[i]);
}

/* ------------------------------------------ S8: token-gated attention */
/*
 * Causal attention over the K kept tokens of one upper layer
 * [P1 tga][P2 method][P3 tga][P5 Fig 1(c)].  For query row t of q head h
 * (kv head h / (hq/hkv)) and every kept key j <= t:
 *   z_tj   = lambda_t * ( q_t . k_j / sqrt(D) + g_h * s^_j )
 *   lambda_t = 1 + c * ln( (t+1) / (pos_t+1) )
 *   O_t    = sum_j exp(z_tj) v_j / sum_j exp(z_tj)
 * The per-head gain g_h scales the key's importance score, which is added
 * to the logit (a softmax gate multiplying the weights is the same thing:
 * its normaliser cancels).  The exponentials are taken after subtracting the
 * row maximum, which leaves the quotient unchanged.
 * rows == NULL computes every query row; otherwise only rows[0..nrows) and
 * out holds nrows x hq x D values in that order.
 */
typedef struct {
    const double *q, *k, *v, *ks, *gains;
    double c;
    const int32_t* pos;
    int64_t K, hq, hkv, D;
    const int64_t* rows;
    double* out;
} tgo_attn_ctx;

static void tgo_attn_rows(void* p, int64_t begin, int64_t end) {
    const tgo_attn_ctx* a = (const tgo_attn_ctx*)p;
    int64_t G = a->hq / a->hkv;
    double* z = (double*)malloc(sizeof(double) * (size_t)a->K);
    for (int64_t w = begin; w < end; ++w) {
        int64_t ri = w / a->hq;      /* which output row */
        int64_t h = w % a->hq;       /* which q head */
        int64_t t = a->rows ? a->rows[ri] : ri;
        int64_t hk = h / G;
        double lam = 1.0 + a->c * log(((double)t + 1.0) / ((double)a->pos[t] + 1.0));
        const double* qt = a->q + (t * a->hq + h) * a->D;
        double zmax = -INFINITY;
        for (int64_t j = 0; j <= t; ++j) {
            const double* kj = a->k + (j * a->hkv + hk) * a->D;
            double dot = 0.0;
            for (int64_t e = 0; e < a->D; ++e) dot += qt[e] * kj[e];
            z[j] = lam * (dot / sqrt((double)a->D) + a->gains[h] * a->ks[j]);
            if (z[j] > zmax) zmax = z[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j <= t; ++j) {
            z[j] = exp(z[j] - zmax);
            den += z[j];
        }
        double* o = a->out + (ri * a->hq + h) * a->D;
        for (int64_t e = 0; e < a->D; ++e) {
            double num = 0.0;
            for (int64_t j = 0; j <= t; ++j) num += z[j] * a->v[(j * a->hkv + hk) * a->D + e];
            o[e] = num / den;
        }
    }
    free(z);
}

void tgo_gated_attention(const double* q, const double* k, const double* v,
                         const double* key_score, const double* gains, double c,
                         const int32_t* pos, int64_t K, int64_t hq, int64_t hkv, int64_t D,
                         const int64_t* rows, int64_t nrows, double* out, int nthreads) {
    tgo_attn_ctx a = {q, k, v, key_score, gains, c, pos, K, hq, hkv, D, rows, out};
    int64_t nr = rows ? nrows : K;
    tgo_parallel(tgo_attn_rows, &a, nr * hq, nthreads);
}
