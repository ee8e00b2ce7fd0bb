// k_attn.hip -- token-gated causal attention over the kept tokens.
//
// Above the gate layer only the K kept tokens exist.  Each kept key's
// normalised importance score, times a per-head gain, is added to the
// attention logits, and a per-query temperature rescales the logits by the
// log ratio of the query's rank in the kept list to its original position
// (fluxbbs.com TokenGate article, section on token-gated attention;
// slinene.github.io digest, method key points; news.farwalk.ai, "What is
// token-gated attention?"; aiwillknow.com, Figure 1(c)):
//     z_tj = lambda_t * (q_t . k_j / sqrt(D) + g_h * s_j),  j <= t
//     lambda_t = 1 + c * ln((t + 1) / (pos_t + 1))
//     O_t = softmax_j(z_tj) V
//
// Flash-style, one pass over the keys with an online softmax, on CDNA4
// matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//  * S^T = K . Q^T is computed transposed, so a lane owns one query column
//    and 16 keys per 32x32 block: lambda_t, the running max and the running
//    sum are per-lane scalars, and the max needs one exchange between the
//    two half-waves.
//  * The accumulator of S^T starts at sqrt(D) * g_h * s_j (from LDS), so the
//    matrix core adds the key bias for free; the logit in the exp2 domain is
//    then a single multiply by lambda_t * log2(e) / sqrt(D) per element.
//  * The S^T accumulator layout is exactly the B-operand layout of the
//    O^T = V^T . P^T product (keys along k), so P goes from registers to the
//    matrix core with only a conversion to bf16; V is stored transposed in
//    LDS to serve the A operand.
//  * A workgroup is 4 waves of 32 query rows each; when the q heads of a GQA
//    group allow it, the waves of one workgroup cover 2 or 4 heads of the
//    same kv head so every K/V tile in LDS is used by all of them.
//  * Work items are laid out so all workgroups of one kv head run on the same
//    XCD (workgroups go round-robin over the 8 XCDs), keeping that head's K/V
//    in one L2; within an XCD the longest (latest) query tiles start first.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::f32x16;
using tgd::u32x2;
using tgd::u32x4;

constexpr int kThreads = 256;  // 4 waves
constexpr int kBK = 64;        // keys per LDS tile
constexpr int kXcds = 8;
constexpr float kLog2e = 1.44269504088896340736f;

template <int D, int HPW>
struct AttnCfg {
    static constexpr int RB = 4 / HPW;        // 32-row blocks per workgroup
    static constexpr int QROWS = 32 * RB;     // query rows per workgroup
    static constexpr int LDK = D + 8;         // K tile row (bf16), padded
    static constexpr int LDV = kBK + 8;       // V^T tile row (bf16), padded
    static constexpr int KP = kBK * D / 8 / kThreads;        // K 16-byte loads per thread
    static constexpr int VP = kBK * D / 8 / 2 / kThreads;    // V key-pair items per thread
    static constexpr int DB = D / 32;         // 32-row blocks of head_dim in O^T
    static constexpr int QS = D / 16;         // k-steps of the QK^T product
    static_assert(KP >= 1 && VP >= 1, "tile shape");
};

template <int D, int HPW, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void gated_attn(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ kk,
                                                       const uint16_t* __restrict__ v,
                                                       const float* __restrict__ key_score,
                                                       const float* __restrict__ gains, float temp_coef,
                                                       const int32_t* __restrict__ pos, int nk, int hq,
                                                       int hkv, int n_qtiles, int per_xcd, int n_items,
                                                       void* __restrict__ out) {
    using C = AttnCfg<D, HPW>;
    __shared__ __attribute__((aligned(16))) uint16_t sK[kBK * C::LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[D * C::LDV];
    __shared__ __attribute__((aligned(16))) float sBias[HPW][kBK];

    // ---- work item: (kv head, head group, query tile), XCD-aware
    const int lin = blockIdx.x;
    const int item = (lin % kXcds) * per_xcd + lin / kXcds;
    if (item >= n_items) return;
    const int G = hq / hkv;
    const int n_hg = G / HPW;
    const int per_head = n_hg * n_qtiles;
    const int kvh = item / per_head;
    const int rem = item % per_head;
    const int hg = rem / n_qtiles;
    const int qt = n_qtiles - 1 - rem % n_qtiles;  // latest (longest) tiles first

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int hl = wave % HPW, rb = wave / HPW;
    const int h = kvh * G + hg * HPW + hl;
    const int q0 = qt * C::QROWS + rb * 32;  // this wave's first query row
    const int t = q0 + l32;                   // this lane's query row
    const int wg_last = min(nk, qt * C::QROWS + C::QROWS) - 1;
    const int wave_last = min(nk - 1, q0 + 31);

    // ---- this lane's query row (B operand of S^T), temperature and scale
    u32x4 qreg[C::QS];
    {
        const bool ok = t < nk;
        const uint16_t* qp = q + ((int64_t)t * hq + h) * D;
#pragma unroll
        for (int s = 0; s < C::QS; ++s)
            qreg[s] = ok ? *reinterpret_cast<const u32x4*>(qp + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
    }
    float lam = 1.0f;
    if (t < nk) lam = 1.0f + temp_coef * logf((float)(t + 1) / ((float)pos[t] + 1.0f));
    const float a_t = lam * kLog2e * (1.0f / sqrtf((float)D));
    const float sqrt_d = sqrtf((float)D);

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;

    // ---- K/V tile staging (registers -> LDS)
    u32x4 kreg[C::KP];
    u32x4 vreg[C::VP][2];
    auto load_tile = [&](int j0) {
#pragma unroll
        for (int r = 0; r < C::KP; ++r) {
            const int p = tid + kThreads * r, row = p / (D / 8), col = (p % (D / 8)) * 8;
            const int j = j0 + row;
            kreg[r] = j < nk ? *reinterpret_cast<const u32x4*>(kk + ((int64_t)j * hkv + kvh) * D + col)
                             : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < C::VP; ++r) {
            const int p = tid + kThreads * r, kp = p % (kBK / 2), dc = p / (kBK / 2);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int j = j0 + 2 * kp + e;
                vreg[r][e] = j < nk ? *reinterpret_cast<const u32x4*>(v + ((int64_t)j * hkv + kvh) * D + dc * 8)
                                    : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&](int j0) {
#pragma unroll
        for (int r = 0; r < C::KP; ++r) {
            const int p = tid + kThreads * r, row = p / (D / 8), col = (p % (D / 8)) * 8;
            *reinterpret_cast<u32x4*>(&sK[row * C::LDK + col]) = kreg[r];
        }
#pragma unroll
        for (int r = 0; r < C::VP; ++r) {
            const int p = tid + kThreads * r, kp = p % (kBK / 2), dc = p / (kBK / 2);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a = vreg[r][0][w], b = vreg[r][1][w];
                // d = dc*8 + 2w (low halves) and dc*8 + 2w + 1 (high halves); keys 2kp, 2kp+1
                *reinterpret_cast<uint32_t*>(&sVt[(dc * 8 + 2 * w) * C::LDV + 2 * kp]) =
                    (a & 0xffffu) | (b << 16);
                *reinterpret_cast<uint32_t*>(&sVt[(dc * 8 + 2 * w + 1) * C::LDV + 2 * kp]) =
                    (a >> 16) | (b & 0xffff0000u);
            }
        }
        if (tid < HPW * kBK) {
            const int hh = tid / kBK, j = tid % kBK;
            const int jj = j0 + j;
            const float gh = gains[kvh * G + hg * HPW + hh];
            sBias[hh][j] = jj < nk ? sqrt_d * gh * key_score[jj] : 0.0f;
        }
    };

    load_tile(0);
    for (int j0 = 0; j0 <= wg_last; j0 += kBK) {
        __syncthreads();  // previous tile fully consumed
        store_tile(j0);
        __syncthreads();
        if (j0 + kBK <= wg_last) load_tile(j0 + kBK);  // next tile's loads overlap this tile's math
        if (j0 > wave_last) continue;                 // every key of this tile is in this wave's future

        // S^T for 64 keys x 32 queries: two 32x32 blocks, started at the key bias.
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const float4 bv = *reinterpret_cast<const float4*>(&sBias[hl][kb * 32 + 8 * i4 + 4 * g]);
                sacc[kb][4 * i4 + 0] = bv.x;
                sacc[kb][4 * i4 + 1] = bv.y;
                sacc[kb][4 * i4 + 2] = bv.z;
                sacc[kb][4 * i4 + 3] = bv.w;
            }
        }
#pragma unroll
        for (int s = 0; s < C::QS; ++s) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(&sK[(kb * 32 + l32) * C::LDK + s * 16 + g * 8]);
                sacc[kb] = tgd::mfma32(a, qreg[s], sacc[kb]);
            }
        }

        // logits in the exp2 domain, causal mask, tile max
        const bool diag = j0 + kBK - 1 > q0;
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float z = sacc[kb][i] * a_t;
                if (diag) {
                    const int j = j0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (j > t) z = -INFINITY;
                }
                sacc[kb][i] = z;
                mt = fmaxf(mt, z);
            }
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float ls = 0.0f;
        u32x4 pb[2][2];  // P^T as bf16, [key block][k-step]
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                const float p0 = exp2f(sacc[kb][i] - m_new);
                const float p1 = exp2f(sacc[kb][i + 1] - m_new);
                ls += p0 + p1;
                pb[kb][i >> 3][(i & 7) >> 1] = tgd::pack_bf16x2(p0, p1);
            }
        }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] *= alpha;

        // O^T += V^T . P^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int key = kb * 32 + 16 * s + 4 * g;
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    const uint16_t* vr = &sVt[(db * 32 + l32) * C::LDV];
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(vr + key);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + key + 8);
                    const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
                    o[db] = tgd::mfma32(a, pb[kb][s], o[db]);
                }
            }
        }
    }

    // ---- normalise and write this lane's query row
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (t >= nk) return;
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int dd = db * 32 + 8 * i4 + 4 * g;
            const int64_t off = ((int64_t)t * hq + h) * D + dd;
            const float y0 = o[db][4 * i4] * inv, y1 = o[db][4 * i4 + 1] * inv;
            const float y2 = o[db][4 * i4 + 2] * inv, y3 = o[db][4 * i4 + 3] * inv;
            if (OUT_F32) {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + off) = float4{y0, y1, y2, y3};
            } else {
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + off) =
                    u32x2{tgd::pack_bf16x2(y0, y1), tgd::pack_bf16x2(y2, y3)};
            }
        }
    }
}

template <int D, int HPW>
int launch_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* ks, const float* gains,
                float c, const int32_t* pos, int64_t nk, int hq, int hkv, void* out, int out_dtype,
                hipStream_t s) {
    using C = AttnCfg<D, HPW>;
    const int n_qtiles = (int)((nk + C::QROWS - 1) / C::QROWS);
    const int n_items = hkv * (hq / hkv / HPW) * n_qtiles;
    const int per_xcd = (n_items + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(per_xcd * kXcds));
    if (out_dtype == 1)
        hipLaunchKernelGGL((gated_attn<D, HPW, true>), grid, dim3(kThreads), 0, s, q, k, v, ks, gains, c, pos,
                           (int)nk, hq, hkv, n_qtiles, per_xcd, n_items, out);
    else
        hipLaunchKernelGGL((gated_attn<D, HPW, false>), grid, dim3(kThreads), 0, s, q, k, v, ks, gains, c, pos,
                           (int)nk, hq, hkv, n_qtiles, per_xcd, n_items, out);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

template <int D>
int launch_attn_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* ks, const float* gains,
                  float c, const int32_t* pos, int64_t nk, int hq, int hkv, void* out, int out_dtype,
                  hipStream_t s) {
    const int G = hq / hkv;
    if (G % 4 == 0) return launch_attn<D, 4>(q, k, v, ks, gains, c, pos, nk, hq, hkv, out, out_dtype, s);
    if (G % 2 == 0) return launch_attn<D, 2>(q, k, v, ks, gains, c, pos, nk, hq, hkv, out, out_dtype, s);
    return launch_attn<D, 1>(q, k, v, ks, gains, c, pos, nk, hq, hkv, out, out_dtype, s);
}

}  // namespace

namespace tgi {

int launch_gated_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const float* key_score, const float* gains, float temp_coef,
                           const int32_t* pos, int64_t n_kept, int hq, int hkv, int head_dim,
                           void* out, int out_dtype, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    switch (head_dim) {
        case 64:
            return launch_attn_d<64>(q, k, v, key_score, gains, temp_coef, pos, n_kept, hq, hkv, out, out_dtype, s);
        case 128:
            return launch_attn_d<128>(q, k, v, key_score, gains, temp_coef, pos, n_kept, hq, hkv, out, out_dtype, s);
        default:
            return TG_EUNSUPPORTED;
    }
}

}  // namespace tgi
