// k_attn_bwd.hip -- backward of token-gated causal attention.
//
// The gate is trained through the upper layers' attention: each kept token's
// score, times a per-head gain, is a bias on that token's attention logits,
// and a per-query temperature rescales the logits (fluxbbs.com TokenGate
// article, section on token-gated attention; slinene.github.io digest, method
// key points; news.farwalk.ai, "What is token-gated attention?";
// aiwillknow.com, Figure 1(c)).  With U_tj = q_t.k_j/sqrt(D) + g_h s_j,
// Z = lambda_t U, P = softmax_j(Z) and dO given, the gradients are
//   dP_tj = dO_t.v_j,  D_t = dO_t.O_t,  dZ_tj = P_tj (dP_tj - D_t),
//   dU = lambda_t dZ,  dlambda_t = sum_j dZ_tj U_tj,
//   dq_t = sum_j dU_tj k_j / sqrt(D),  dk_j = sum_t dU_tj q_t / sqrt(D),
//   dv_j = sum_t P_tj dO_t,  ds_j = sum_h g_h sum_t dU_tj,
//   dg_h = sum_tj dU_tj s_j,  dc = sum_ht dlambda_t ln((t+1)/(pos_t+1)).
//
// Flash-style: the probabilities are rebuilt block by block from the
// forward's per-row log2-sum-exp2 (P = 2^(a_t S - lse_t), S = q.k + sqrt(D)
// g s, a_t = lambda_t log2(e)/sqrt(D)), never stored.  Three passes:
//  * bwd_prep: D_t, lambda_t and a_t per row.
//  * bwd_dq: one wave per (q head, 32-query block) walks the key blocks up
//    to the diagonal: S^T = K.Q^T and dP^T = V.dO^T on the matrix cores (a
//    lane owns a query column, so the row values are per-lane scalars), then
//    dq^T += K^T.dU^T with K^T read from LDS by the transposing read, and the
//    per-row partials of dlambda and of sum_j dU s_j.
//  * bwd_dkv: one wave per (kv head, 32-key block) walks the query blocks
//    from the diagonal on, for every q head of the group: S = Q.K^T and
//    dP = dO.V^T (a lane owns a key column), then dv^T += dO^T.P and
//    dk^T += Q^T.dU with Q^T and dO^T read transposed from LDS, and the
//    per-key partial of ds.
//  * bwd_reduce: the per-row and per-key partials summed in a fixed order.
// No atomics: results are deterministic.  P and dU enter the matrix cores as
// bf16 (fp32 accumulation).  Each wave stages its blocks in LDS of its own.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::f32x16;
using tgd::u32x2;
using tgd::u32x4;

#define TG_LDS __attribute__((address_space(3)))
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;

constexpr int kWavesPerBlock = 4;
constexpr float kLog2e = 1.44269504088896340736f;

// XOR permutation of the 16-byte pieces of a row by the row (bank-conflict-free
// 16-byte reads of 16 consecutive rows and transposing reads of 4-row groups).
template <int PIECES>
__device__ __forceinline__ int swz(int r) {
    if (PIECES == 16) {
        const int x = r & 15;
        return ((x << 2) | (x >> 2)) & 15;
    }
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
}

template <int D>
struct Geo {
    static constexpr int PIECES = D / 8;
    static constexpr int ROW_BYTES = 2 * D;
    static constexpr int BLOCK_BYTES = 32 * ROW_BYTES;
    static constexpr int QS = D / 16;  // k-steps over head_dim
    static constexpr int DB = D / 32;  // 32-row blocks of head_dim
};

// 32 rows (row0 .. row0+31, rows past nrows as zeros) of a [rows, heads, D]
// bf16 tensor, head hh, into a wave's LDS block with swizzled pieces.
template <int D>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ src, int heads, int hh, int row0, int nrows,
                                           TG_LDS uint8_t* blk, int lane) {
    using G = Geo<D>;
#pragma unroll
    for (int it = 0; it < G::PIECES / 2; ++it) {
        const int e = it * 64 + lane;
        const int r = e / G::PIECES, c = e % G::PIECES;
        const int row = row0 + r;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (row < nrows) v = *reinterpret_cast<const u32x4*>(src + ((int64_t)row * heads + hh) * D + 8 * c);
        *reinterpret_cast<TG_LDS u32x4*>(blk + r * G::ROW_BYTES + 16 * (c ^ swz<G::PIECES>(r))) = v;
    }
}

// Row-major operand of a product over head_dim (lane holds 8 consecutive
// values of row l32 at k-step s, half g) from an LDS block.
template <int D>
__device__ __forceinline__ u32x4 row_operand(const TG_LDS uint8_t* blk, int l32, int g, int s) {
    using G = Geo<D>;
    return *reinterpret_cast<const TG_LDS u32x4*>(blk + l32 * G::ROW_BYTES + 16 * ((2 * s + g) ^ swz<G::PIECES>(l32)));
}

// Transposed operand (head_dim rows x 16 block rows, k-step s over the block
// rows) of the products that contract over the block's rows: the transposing
// read hands lane jj of each 16-lane group four consecutive block rows of
// one head_dim column, matching the row order of a 32x32 accumulator used
// as the B operand.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const TG_LDS uint8_t* blk, int lane, int db, int s) {
    using G = Geo<D>;
    const int quad = lane >> 4, jj = lane & 15;
    u32x4 a;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int row = 16 * s + 4 * (quad >> 1) + 8 * half + (jj >> 2);
        const int dcol = db * 32 + 16 * (quad & 1) + 4 * (jj & 3);
        const int off = row * G::ROW_BYTES + 16 * ((dcol >> 3) ^ swz<G::PIECES>(row)) + 8 * ((dcol >> 2) & 1);
        const bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((TG_LDS bf16x4_t*)(blk + off));
        const u32x2 w = __builtin_bit_cast(u32x2, x);
        a[2 * half] = w[0];
        a[2 * half + 1] = w[1];
    }
    return a;
}

// Register operand of a product over head_dim from global memory: lane holds
// 8 consecutive values of row `row` (zeros past nrows) at k-step s, half g.
template <int D>
__device__ __forceinline__ u32x4 global_operand(const uint16_t* __restrict__ src, int heads, int hh, int row,
                                                int nrows, int g, int s) {
    if (row >= nrows) return u32x4{0u, 0u, 0u, 0u};
    return *reinterpret_cast<const u32x4*>(src + ((int64_t)row * heads + hh) * D + 16 * s + 8 * g);
}

// A 32x32 accumulator as the bf16 B operand of a product over its rows
// (two k-steps of 16 rows).
__device__ __forceinline__ void pack_b(const f32x16& x, u32x4 (&b)[2]) {
#pragma unroll
    for (int i = 0; i < 16; i += 2) b[i >> 3][(i & 7) >> 1] = tgd::cvt_pk_bf16(x[i], x[i + 1]);
}

// ---- per-row values: D_t = dO_t . O_t, lambda_t, a_t
template <int D>
__global__ __launch_bounds__(256) void bwd_prep(const float* __restrict__ O, const uint16_t* __restrict__ dO,
                                                const int32_t* __restrict__ pos, float temp_coef, int nk, int hq,
                                                int kp, float* __restrict__ dvec, float* __restrict__ lam,
                                                float* __restrict__ acoef) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // row = t * hq + h
    if (r >= (int64_t)nk * hq) return;
    const int t = (int)(r / hq), h = (int)(r % hq);
    float acc = 0.0f;
    for (int d = lane; d < D; d += 64) acc = fmaf(O[r * D + d], tgd::bf16lo(dO[r * D + d]), acc);
    acc = tgd::wave_sum(acc);
    if (lane == 0) {
        dvec[(int64_t)h * kp + t] = acc;
        if (h == 0) {
            const float l = 1.0f + temp_coef * logf((float)(t + 1) / ((float)pos[t] + 1.0f));
            lam[t] = l;
            acoef[t] = l * kLog2e * (1.0f / sqrtf((float)D));
        }
    }
}

// ---- dq, and the per-row partials of dlambda and of sum_j dU_tj s_j
template <int D>
__global__ __launch_bounds__(64 * kWavesPerBlock) void bwd_dq(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ gains, const int32_t* __restrict__ pos,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ dvec,
    const float* __restrict__ lam, const float* __restrict__ acoef, int nk, int hq, int hkv, int kp,
    float* __restrict__ dq, float* __restrict__ dlamc, float* __restrict__ dgp) {
    using G = Geo<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t sK[kWavesPerBlock][G::BLOCK_BYTES];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int nqb = (nk + 31) / 32;
    const int item = blockIdx.x * kWavesPerBlock + w;
    if (item >= hq * nqb) return;
    const int h = item / nqb, qb = item % nqb;
    const int hk = h / (hq / hkv);
    const int t = qb * 32 + l32;
    const bool ok = t < nk;
    const float rs = 1.0f / sqrtf((float)D);
    const float sg = sqrtf((float)D) * gains[h];
    TG_LDS uint8_t* blk = (TG_LDS uint8_t*)sK[w];

    u32x4 qreg[G::QS], doreg[G::QS];
#pragma unroll
    for (int s = 0; s < G::QS; ++s) {
        qreg[s] = global_operand<D>(q, hq, h, t, nk, g, s);
        doreg[s] = global_operand<D>(dO, hq, h, t, nk, g, s);
    }
    const float a_t = ok ? acoef[t] : 0.0f;
    const float lse_t = ok ? lse[(int64_t)h * kp + t] : 0.0f;
    const float d_t = ok ? dvec[(int64_t)h * kp + t] : 0.0f;
    const float lam_t = ok ? lam[t] : 0.0f;

    f32x16 dqa[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) dqa[db] = f32x16{};
    float dl = 0.0f, dgs = 0.0f;

    for (int kb = 0; kb <= qb; ++kb) {
        const int j0 = kb * 32;
        // (one wave writes and reads its own LDS block; LDS executes a wave's
        // instructions in order, the barriers keep the compiler from moving
        // reads across the writes)
        __builtin_amdgcn_wave_barrier();
        stage_rows<D>(k, hkv, hk, j0, nk, blk, lane);
        __builtin_amdgcn_wave_barrier();
        // this lane's 16 key rows of the accumulators: j0 + 8 (i/4) + 4 g + i%4
        float sv[16];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + 8 * i4 + 4 * g + e;
                sv[4 * i4 + e] = j < nk ? key_score[j] : 0.0f;
            }
        }
        f32x16 sacc, dpacc = f32x16{};
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = sg * sv[i];
#pragma unroll
        for (int s = 0; s < G::QS; ++s) {
            sacc = tgd::mfma32(row_operand<D>(blk, l32, g, s), qreg[s], sacc);
            dpacc = tgd::mfma32(global_operand<D>(v, hkv, hk, j0 + l32, nk, g, s), doreg[s], dpacc);
        }
        f32x16 du;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = j0 + 8 * (i >> 2) + 4 * g + (i & 3);
            const bool vis = ok && j <= t;
            const float p = vis ? __builtin_amdgcn_exp2f(fmaf(a_t, sacc[i], -lse_t)) : 0.0f;
            const float dz = p * (dpacc[i] - d_t);
            du[i] = lam_t * dz;
            dl = fmaf(dz, sacc[i] * rs, dl);
            dgs = fmaf(du[i], sv[i], dgs);
        }
        u32x4 pb[2];
        pack_b(du, pb);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int db = 0; db < G::DB; ++db) dqa[db] = tgd::mfma32(tr_operand<D>(blk, lane, db, s), pb[s], dqa[db]);
    }
    // dq_t[d]: accumulator unit u holds head_dim rows 32 (u/4) + 8 (u%4) + 4 g .. +3
    if (ok) {
#pragma unroll
        for (int u = 0; u < 4 * G::DB; ++u) {
            const int i = 4 * (u % 4);
            const int dd = (u / 4) * 32 + 8 * (u % 4) + 4 * g;
            *reinterpret_cast<float4*>(dq + ((int64_t)t * hq + h) * D + dd) =
                float4{dqa[u / 4][i] * rs, dqa[u / 4][i + 1] * rs, dqa[u / 4][i + 2] * rs, dqa[u / 4][i + 3] * rs};
        }
    }
    dl = tgd::half_sum(dl);
    dgs = tgd::half_sum(dgs);
    if (ok && g == 0) {
        dlamc[(int64_t)h * kp + t] = dl * logf((float)(t + 1) / ((float)pos[t] + 1.0f));
        dgp[(int64_t)h * kp + t] = dgs;
    }
}

// ---- dk, dv, and the per-key partial of ds (this kv head's q heads)
template <int D>
__global__ __launch_bounds__(64 * kWavesPerBlock) void bwd_dkv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ gains, const uint16_t* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ dvec, const float* __restrict__ lam,
    const float* __restrict__ acoef, int nk, int hq, int hkv, int kp, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dsp) {
    using G = Geo<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t sQ[kWavesPerBlock][G::BLOCK_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sO[kWavesPerBlock][G::BLOCK_BYTES];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int nkb = (nk + 31) / 32;
    const int item = blockIdx.x * kWavesPerBlock + w;
    if (item >= hkv * nkb) return;
    const int hk = item / nkb, kb = item % nkb;
    const int grp = hq / hkv;
    const int j = kb * 32 + l32;  // this lane's key column
    const float rs = 1.0f / sqrtf((float)D);
    TG_LDS uint8_t* bq = (TG_LDS uint8_t*)sQ[w];
    TG_LDS uint8_t* bo = (TG_LDS uint8_t*)sO[w];

    u32x4 kreg[G::QS], vreg[G::QS];
#pragma unroll
    for (int s = 0; s < G::QS; ++s) {
        kreg[s] = global_operand<D>(k, hkv, hk, j, nk, g, s);
        vreg[s] = global_operand<D>(v, hkv, hk, j, nk, g, s);
    }
    const float sj = j < nk ? key_score[j] : 0.0f;
    f32x16 dka[G::DB], dva[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) dka[db] = dva[db] = f32x16{};
    float dsj = 0.0f;
    const int nqb = (nk + 31) / 32;

    for (int hh = 0; hh < grp; ++hh) {
        const int h = hk * grp + hh;
        const float gh = gains[h];
        const float bias = sqrtf((float)D) * gh * sj;
        for (int qb = kb; qb < nqb; ++qb) {
            const int t0 = qb * 32;
            __builtin_amdgcn_wave_barrier();
            stage_rows<D>(q, hq, h, t0, nk, bq, lane);
            stage_rows<D>(dO, hq, h, t0, nk, bo, lane);
            __builtin_amdgcn_wave_barrier();
            // this lane's 16 query rows: t0 + 8 (i/4) + 4 g + i%4 (arrays padded to 32 rows)
            float ar[16], lr[16], dr[16], mr[16];
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int tr = t0 + 8 * i4 + 4 * g;
                const float4 a4 = *reinterpret_cast<const float4*>(acoef + tr);
                const float4 l4 = *reinterpret_cast<const float4*>(lse + (int64_t)h * kp + tr);
                const float4 d4 = *reinterpret_cast<const float4*>(dvec + (int64_t)h * kp + tr);
                const float4 m4 = *reinterpret_cast<const float4*>(lam + tr);
                ar[4 * i4] = a4.x, ar[4 * i4 + 1] = a4.y, ar[4 * i4 + 2] = a4.z, ar[4 * i4 + 3] = a4.w;
                lr[4 * i4] = l4.x, lr[4 * i4 + 1] = l4.y, lr[4 * i4 + 2] = l4.z, lr[4 * i4 + 3] = l4.w;
                dr[4 * i4] = d4.x, dr[4 * i4 + 1] = d4.y, dr[4 * i4 + 2] = d4.z, dr[4 * i4 + 3] = d4.w;
                mr[4 * i4] = m4.x, mr[4 * i4 + 1] = m4.y, mr[4 * i4 + 2] = m4.z, mr[4 * i4 + 3] = m4.w;
            }
            f32x16 sacc, dpacc = f32x16{};
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = bias;
#pragma unroll
            for (int s = 0; s < G::QS; ++s) {
                sacc = tgd::mfma32(row_operand<D>(bq, l32, g, s), kreg[s], sacc);
                dpacc = tgd::mfma32(row_operand<D>(bo, l32, g, s), vreg[s], dpacc);
            }
            f32x16 p, du;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = t0 + 8 * (i >> 2) + 4 * g + (i & 3);
                const bool vis = t < nk && j <= t;
                // (rows past the last query read the padding of the row arrays: never used)
                p[i] = vis ? __builtin_amdgcn_exp2f(fmaf(ar[i], sacc[i], -lr[i])) : 0.0f;
                du[i] = vis ? mr[i] * p[i] * (dpacc[i] - dr[i]) : 0.0f;
                dsj = fmaf(gh, du[i], dsj);
            }
            u32x4 pp[2], pu[2];
            pack_b(p, pp);
            pack_b(du, pu);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int db = 0; db < G::DB; ++db) {
                    dva[db] = tgd::mfma32(tr_operand<D>(bo, lane, db, s), pp[s], dva[db]);
                    dka[db] = tgd::mfma32(tr_operand<D>(bq, lane, db, s), pu[s], dka[db]);
                }
            }
        }
    }
    if (j < nk) {
#pragma unroll
        for (int u = 0; u < 4 * G::DB; ++u) {
            const int i = 4 * (u % 4);
            const int dd = (u / 4) * 32 + 8 * (u % 4) + 4 * g;
            const int64_t off = ((int64_t)j * hkv + hk) * D + dd;
            *reinterpret_cast<float4*>(dk + off) =
                float4{dka[u / 4][i] * rs, dka[u / 4][i + 1] * rs, dka[u / 4][i + 2] * rs, dka[u / 4][i + 3] * rs};
            *reinterpret_cast<float4*>(dv + off) = float4{dva[u / 4][i], dva[u / 4][i + 1], dva[u / 4][i + 2],
                                                          dva[u / 4][i + 3]};
        }
    }
    dsj = tgd::half_sum(dsj);
    if (j < nk && g == 0) dsp[(int64_t)hk * kp + j] = dsj;
}

// ---- fixed-order sums: dscore[j] over the kv heads; dgains[h] over the rows;
// dtemp over heads and rows (workgroup hq)
__global__ __launch_bounds__(256) void bwd_reduce_score(const float* __restrict__ dsp, int nk, int hkv, int kp,
                                                        float* __restrict__ dscore) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= nk) return;
    float s = 0.0f;
    for (int hk = 0; hk < hkv; ++hk) s += dsp[(int64_t)hk * kp + j];
    dscore[j] = s;
}

__global__ __launch_bounds__(256) void bwd_reduce_rows(const float* __restrict__ dgp, const float* __restrict__ dlamc,
                                                       int nk, int hq, int kp, float* __restrict__ dgains,
                                                       float* __restrict__ dtemp) {
    __shared__ double red[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int b = blockIdx.x;  // 0 .. hq-1: gains; hq: temperature
    double acc = 0.0;
    if (b < hq) {
        for (int t = tid; t < nk; t += 256) acc += (double)dgp[(int64_t)b * kp + t];
    } else {
        for (int hh = 0; hh < hq; ++hh)
            for (int t = tid; t < nk; t += 256) acc += (double)dlamc[(int64_t)hh * kp + t];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) red[w] = acc;
    __syncthreads();
    if (tid == 0) {
        const double tot = red[0] + red[1] + red[2] + red[3];
        if (b < hq)
            dgains[b] = (float)tot;
        else
            *dtemp = (float)tot;
    }
}

template <int D>
int launch_bwd_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* key_score, const float* gains,
                 float temp_coef, const int32_t* pos, int nk, int hq, int hkv, const uint16_t* dout, float* dq,
                 float* dk, float* dv, float* dscore, float* dgains, float* dtemp, const tgi::AttnBwdWs& ws,
                 hipStream_t s) {
    const int kp = ws.kp;
    // forward again, in fp32 with the per-row log2-sum-exp2
    int rc = tgi::launch_gated_attention(q, k, v, key_score, gains, temp_coef, pos, nk, hq, hkv, D, ws.out, 1, ws.lse,
                                         kp, s);
    if (rc != TG_OK) return rc;
    const int64_t rows = (int64_t)nk * hq;
    hipLaunchKernelGGL(bwd_prep<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, ws.out, dout, pos, temp_coef,
                       nk, hq, kp, ws.dvec, ws.lam, ws.acoef);
    const int nqb = (nk + 31) / 32;
    hipLaunchKernelGGL(bwd_dq<D>, dim3((unsigned)((hq * nqb + kWavesPerBlock - 1) / kWavesPerBlock)),
                       dim3(64 * kWavesPerBlock), 0, s, q, k, v, key_score, gains, pos, dout, ws.lse, ws.dvec, ws.lam,
                       ws.acoef, nk, hq, hkv, kp, dq, ws.dlamc, ws.dgp);
    hipLaunchKernelGGL(bwd_dkv<D>, dim3((unsigned)((hkv * nqb + kWavesPerBlock - 1) / kWavesPerBlock)),
                       dim3(64 * kWavesPerBlock), 0, s, q, k, v, key_score, gains, dout, ws.lse, ws.dvec, ws.lam,
                       ws.acoef, nk, hq, hkv, kp, dk, dv, ws.dsp);
    hipLaunchKernelGGL(bwd_reduce_score, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, s, ws.dsp, nk, hkv, kp,
                       dscore);
    hipLaunchKernelGGL(bwd_reduce_rows, dim3((unsigned)(hq + 1)), dim3(256), 0, s, ws.dgp, ws.dlamc, nk, hq, kp, dgains,
                       dtemp);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace

namespace tgi {

int launch_gated_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* key_score,
                               const float* gains, float temp_coef, const int32_t* pos, int64_t n_kept, int hq,
                               int hkv, int head_dim, const uint16_t* dout, float* dq, float* dk, float* dv,
                               float* dscore, float* dgains, float* dtemp, void* workspace, void* stream) {
    const AttnBwdWs ws = attn_bwd_ws(workspace, n_kept, hq, hkv, head_dim);
    hipStream_t s = (hipStream_t)stream;
    switch (head_dim) {
        case 64:
            return launch_bwd_d<64>(q, k, v, key_score, gains, temp_coef, pos, (int)n_kept, hq, hkv, dout, dq, dk, dv,
                                    dscore, dgains, dtemp, ws, s);
        case 128:
            return launch_bwd_d<128>(q, k, v, key_score, gains, temp_coef, pos, (int)n_kept, hq, hkv, dout, dq, dk,
                                     dv, dscore, dgains, dtemp, ws, s);
        default:
            return TG_EUNSUPPORTED;
    }
}

}  // namespace tgi
