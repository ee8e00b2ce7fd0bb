/* Drives every entry point of the fp64 oracle (oracle/tg_oracle.c) on small
 * seeded inputs, single- and multi-threaded, for an AddressSanitizer /
 * UndefinedBehaviorSanitizer build.  Exit status 0 when the runs agree. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void tgo_score_mlp(const double*, const double*, const double*, const double*, double, int64_t, int64_t, int64_t,
                   double, double*, int);
double tgo_seq_rmsnorm(const double*, int64_t, double, double*);
int tgo_select_topk(const double*, const uint8_t*, int64_t, int64_t, int32_t*);
void tgo_gather_rows(const void*, int64_t, int64_t, const int32_t*, int64_t, void*, int64_t);
void tgo_rope(const double*, const int32_t*, int64_t, int64_t, int64_t, double, double*);
void tgo_to_bf16(const double*, int64_t, uint16_t*);
void tgo_gated_attention(const double*, const double*, const double*, const double*, const double*, double,
                         const int32_t*, int64_t, int64_t, int64_t, int64_t, const int64_t*, int64_t, double*, int);

static uint64_t st = 88172645463325252ull;
static double rnd(void) { /* xorshift64, uniform in [-1, 1) */
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return (double)(st >> 11) / 4503599627370496.0 - 1.0;
}
static double* vec(int64_t n) {
    double* p = malloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}

int main(void) {
    const int64_t n = 97, d = 64, hd = 16, K = 41, hq = 4, hkv = 2, D = 8;
    double *h = vec(n * d), *w1 = vec(hd * d), *b1 = vec(hd), *w2 = vec(hd);
    double *s1 = malloc(sizeof(double) * n), *s3 = malloc(sizeof(double) * n), *sh = malloc(sizeof(double) * n);
    tgo_score_mlp(h, w1, b1, w2, 0.1, n, d, hd, 1e-6, s1, 1);
    tgo_score_mlp(h, w1, NULL, w2, 0.1, n, d, hd, 1e-6, s3, 3);
    tgo_score_mlp(h, w1, b1, w2, 0.1, n, d, hd, 1e-6, s3, 3);
    if (memcmp(s1, s3, sizeof(double) * n)) return 1;
    if (!(tgo_seq_rmsnorm(s1, n, 1e-6, sh) > 0.0)) return 2;
    uint8_t* forced = calloc((size_t)n, 1);
    forced[n - 1] = forced[n - 5] = 1;
    int32_t kept[97];
    for (int64_t k = 2; k <= n; k += 19) {
        if (tgo_select_topk(sh, forced, n, k, kept) != 0) return 3;
        for (int64_t t = 1; t < k; ++t)
            if (kept[t] <= kept[t - 1]) return 4;
    }
    if (tgo_select_topk(sh, forced, n, 1, kept) == 0) return 5; /* fewer slots than forced tokens */
    if (tgo_select_topk(sh, NULL, n, 0, kept) == 0) return 6;
    int64_t k = K;
    if (tgo_select_topk(sh, forced, n, k, kept) != 0) return 7;
    uint16_t* rows = malloc(sizeof(uint16_t) * (size_t)(n * d));
    for (int64_t i = 0; i < n * d; ++i) rows[i] = (uint16_t)(i * 2654435761u);
    uint16_t* g = malloc(sizeof(uint16_t) * (size_t)(k * d));
    tgo_gather_rows(rows, d * 2, d * 2, kept, k, g, d * 2);
    for (int64_t t = 0; t < k; ++t)
        if (memcmp(g + t * d, rows + (int64_t)kept[t] * d, (size_t)d * 2)) return 8;
    double *q = vec(K * hq * D), *kk = vec(K * hkv * D), *v = vec(K * hkv * D), *gains = vec(hq);
    double* qr = malloc(sizeof(double) * (size_t)(K * hq * D));
    tgo_rope(q, kept, K, hq, D, 1e6, qr);
    uint16_t* qb = malloc(sizeof(uint16_t) * (size_t)(K * hq * D));
    tgo_to_bf16(qr, K * hq * D, qb);
    double ks[41];
    for (int64_t t = 0; t < K; ++t) ks[t] = sh[kept[t]];
    double *o1 = malloc(sizeof(double) * (size_t)(K * hq * D)), *o3 = malloc(sizeof(double) * (size_t)(K * hq * D));
    tgo_gated_attention(qr, kk, v, ks, gains, 0.3, kept, K, hq, hkv, D, NULL, 0, o1, 1);
    tgo_gated_attention(qr, kk, v, ks, gains, 0.3, kept, K, hq, hkv, D, NULL, 0, o3, 3);
    if (memcmp(o1, o3, sizeof(double) * (size_t)(K * hq * D))) return 9;
    const int64_t sel[3] = {0, 17, 40};
    double* os = malloc(sizeof(double) * (size_t)(3 * hq * D));
    tgo_gated_attention(qr, kk, v, ks, gains, 0.3, kept, K, hq, hkv, D, sel, 3, os, 2);
    for (int r = 0; r < 3; ++r)
        if (memcmp(os + r * hq * D, o1 + sel[r] * hq * D, sizeof(double) * (size_t)(hq * D))) return 10;
    free(h); free(w1); free(b1); free(w2); free(s1); free(s3); free(sh); free(forced); free(rows); free(g);
    free(q); free(kk); free(v); free(gains); free(qr); free(qb); free(o1); free(o3); free(os);
    puts("oracle driver ok");
    return 0;
}
