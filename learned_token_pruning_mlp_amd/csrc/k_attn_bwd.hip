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
//    per-(head, query block) partials of dlambda and of sum_j dU s_j.  The
//    four waves of a workgroup (two q heads of a kv group x two adjacent
//    query blocks) share one stream of K/V blocks, and two workgroups fit a
//    CU (two waves a SIMD).
//  * bwd_dkv: one wave per (kv head, 32-key block, share of the group's q
//    heads) walks the query blocks from the diagonal on: S = Q.K^T and
//    dP = dO.V^T (a lane owns a key column), then dv^T += dO^T.P and
//    dk^T += Q^T.dU with Q^T and dO^T read transposed from LDS, and the
//    per-key partial of ds; the waves sharing a key block add their partial
//    dk, dv and ds in LDS in a fixed order.
//  * bwd_reduce: the per-kv-head and per-block partials summed in a fixed
//    order.
// No atomics: results are deterministic.  P and dU enter the matrix cores as
// bf16 (fp32 accumulation).  Blocks stream through two LDS stages (per
// workgroup in the dq pass, per wave in the dk/dv pass), filled by direct
// loads one block ahead; rows past the end read as zeros through the buffer
// bounds.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::f32x16;
using tgd::u32x2;
using tgd::u32x4;

#define TG_LDS __attribute__((address_space(3)))
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef float lf4 __attribute__((ext_vector_type(4)));  // LDS-side float4

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

// ---- per-(head, row) values packed for the two passes: a_t, the forward's
// lse, D_t = dO_t . O_t and lambda_t (rows past the last one: zeros)
template <int D>
__global__ __launch_bounds__(256) void bwd_prep(const float* __restrict__ O, const uint16_t* __restrict__ dO,
                                                const float* __restrict__ lse, const int32_t* __restrict__ pos,
                                                float temp_coef, int nk, int hq, int kp, float4* __restrict__ rowv) {
    constexpr int LPR = D / 8;        // lanes per (head, row): 8 values each
    constexpr int RPB = 256 / LPR;    // (head, row) pairs per workgroup
    const int tid = threadIdx.x, sub = tid % LPR;
    const int64_t rr = (int64_t)blockIdx.x * RPB + tid / LPR;  // h * kp + t
    if (rr >= (int64_t)hq * kp) return;
    const int h = (int)(rr / kp), t = (int)(rr % kp);
    float acc = 0.0f;
    if (t < nk) {
        const int64_t off = ((int64_t)t * hq + h) * D + 8 * sub;
        const float4 o0 = *reinterpret_cast<const float4*>(O + off);
        const float4 o1 = *reinterpret_cast<const float4*>(O + off + 4);
        const u32x4 d = *reinterpret_cast<const u32x4*>(dO + off);
        acc = o0.x * tgd::bf16lo(d[0]) + o0.y * tgd::bf16hi(d[0]) + o0.z * tgd::bf16lo(d[1]) +
              o0.w * tgd::bf16hi(d[1]) + o1.x * tgd::bf16lo(d[2]) + o1.y * tgd::bf16hi(d[2]) +
              o1.z * tgd::bf16lo(d[3]) + o1.w * tgd::bf16hi(d[3]);
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (sub == 0) {
        float4 out = float4{0.0f, 0.0f, 0.0f, 0.0f};
        if (t < nk) {
            const float l = 1.0f + temp_coef * logf((float)(t + 1) / ((float)pos[t] + 1.0f));
            out = float4{l * kLog2e * (1.0f / sqrtf((float)D)), lse[(int64_t)h * kp + t], acc, l};
        }
        rowv[rr] = out;
    }
}

// Direct loads from memory into LDS: `SIZE` bytes per lane from base + voff
// land at lds + SIZE * lane, through a raw buffer resource covering `bytes`
// bytes, so offsets at or past the end read as zero (rows past the last one).
constexpr int kBufferWord3 = 0x00020000;

template <int SIZE>
__device__ __forceinline__ void lds_load(const void* base, uint32_t bytes, TG_LDS uint8_t* lds, uint32_t voff) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
    static_assert(SIZE == 16 || SIZE == 4, "direct-load size");
    if constexpr (SIZE == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TG_LDS void*)lds, 16, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TG_LDS void*)lds, 4, voff, 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define TG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// 32 rows (row0 ..) of head hh of a [rows, heads, D] bf16 tensor into an LDS
// block: instruction `it` fills bytes it*1024 .. +1023, lane L the 16-byte slot
// (it*64 + L) of the block, i.e. row r, slot c'; it reads piece c' ^ swz(r) of
// that row, which gives the swizzled layout the operand reads expect.
template <int D>
__device__ __forceinline__ void load_block(const uint16_t* src, uint32_t bytes, int heads, int hh, int row0,
                                           TG_LDS uint8_t* blk, int lane) {
    using G = Geo<D>;
#pragma unroll
    for (int it = 0; it < G::PIECES / 2; ++it) {
        const int e = it * 64 + lane;
        const int r = e / G::PIECES, c = (e % G::PIECES) ^ swz<G::PIECES>(r);
        const uint32_t voff = ((uint32_t)(row0 + r) * (uint32_t)heads + (uint32_t)hh) * (uint32_t)G::ROW_BYTES + 16u * c;
        lds_load<16>(src, bytes, blk + it * 1024, voff);
    }
}

// The direct loads of load_block<D> numbered it0, it0 + step, ... (a share of
// them, for a wave of a workgroup that loads a block together).
template <int D>
__device__ __forceinline__ void load_block_share(const uint16_t* src, uint32_t bytes, int heads, int hh, int row0,
                                                 TG_LDS uint8_t* blk, int lane, int it0, int step) {
    using G = Geo<D>;
#pragma unroll
    for (int it = 0; it < G::PIECES / 2; ++it) {
        if ((it - it0) % step != 0 || it < it0) continue;
        const int e = it * 64 + lane;
        const int r = e / G::PIECES, c = (e % G::PIECES) ^ swz<G::PIECES>(r);
        const uint32_t voff = ((uint32_t)(row0 + r) * (uint32_t)heads + (uint32_t)hh) * (uint32_t)G::ROW_BYTES + 16u * c;
        lds_load<16>(src, bytes, blk + it * 1024, voff);
    }
}

// Workgroup barrier that no LDS access moves across (the compiler sees a
// memory clobber on both sides).
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// ---- dq, and per-(head, query block) partials of dlambda and of sum dU s
// A workgroup's four waves take HPW q heads of one kv head x 4 / HPW
// adjacent query blocks, so they all need the same key blocks: each K and V
// block (and its 32 key scores) is streamed once into a two-stage LDS ring
// that the four waves fill together and read together; the loads of block
// kb+1 fly while block kb is multiplied.  A wave multiplies the key blocks up
// to its own query block.
template <int D, int HPW>
__global__ __launch_bounds__(64 * kWavesPerBlock, 2) void bwd_dq(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ gains, const int32_t* __restrict__ pos,
    const uint16_t* __restrict__ dO, const float4* __restrict__ rowv, int nk, int hq, int hkv, int kp,
    float* __restrict__ dq, float* __restrict__ dlamc, float* __restrict__ dgp) {
    using G = Geo<D>;
    constexpr int QBW = kWavesPerBlock / HPW;         // query blocks per workgroup
    constexpr int STAGE = 2 * G::BLOCK_BYTES + 256;   // K block, V block, 64 key scores (32 used)
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int grp = hq / hkv;
    const int nqb = (nk + 31) / 32;
    const int ngq = (nqb + QBW - 1) / QBW;            // query-block groups
    const int nhg = grp / HPW;                        // head groups of a kv head
    // work item: (query-block group, kv head, head group); the groups of the
    // last query blocks (the longest walks) first
    const int item = blockIdx.x;
    const int gq = ngq - 1 - item / (hkv * nhg);
    const int hk = (item / nhg) % hkv, hg = item % nhg;
    const int h = hk * grp + hg * HPW + w % HPW;
    const int qb = gq * QBW + w / HPW;                 // this wave's query block
    const int qb_last = min(gq * QBW + QBW - 1, nqb - 1);
    const bool live = qb < nqb;
    const int t = qb * 32 + l32;
    const bool ok = live && t < nk;
    const float rs = 1.0f / sqrtf((float)D);
    const float sg = sqrtf((float)D) * gains[h];
    TG_LDS uint8_t* st0 = (TG_LDS uint8_t*)smem;
    TG_LDS uint8_t* st1 = st0 + STAGE;
    const uint32_t kv_bytes = (uint32_t)nk * (uint32_t)hkv * (uint32_t)G::ROW_BYTES;

    u32x4 qreg[G::QS], doreg[G::QS];
#pragma unroll
    for (int s = 0; s < G::QS; ++s) {
        qreg[s] = global_operand<D>(q, hq, h, t, nk, g, s);
        doreg[s] = global_operand<D>(dO, hq, h, t, nk, g, s);
    }
    const float4 rv = live ? rowv[(int64_t)h * kp + t] : float4{0.0f, 0.0f, 0.0f, 0.0f};  // t < kp
    const float a_t = rv.x, lse_t = rv.y, d_t = rv.z, lam_t = rv.w;

    f32x16 dqa[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) dqa[db] = f32x16{};
    float dl = 0.0f, dgs = 0.0f;

    // block kb into a stage: each wave issues its share of the K and V loads;
    // wave 0 also the scores
    auto issue = [&](int kb, TG_LDS uint8_t* __restrict__ nb) {
        const int j0 = kb * 32;
        load_block_share<D>(k, kv_bytes, hkv, hk, j0, nb, lane, w, kWavesPerBlock);
        load_block_share<D>(v, kv_bytes, hkv, hk, j0, nb + G::BLOCK_BYTES, lane, w, kWavesPerBlock);
        if (w == 0) lds_load<4>(key_score, (uint32_t)nk * 4u, nb + 2 * G::BLOCK_BYTES, (uint32_t)(j0 + lane) * 4u);
    };
    auto step = [&](int kb, TG_LDS uint8_t* __restrict__ cb, TG_LDS uint8_t* __restrict__ nb) {
        TG_WAIT_VMCNT(0);  // this wave's share of block kb is in LDS ...
        lds_barrier();     // ... and every wave's; every wave is done with the other stage
        if (kb < qb_last) issue(kb + 1, nb);
        if (!live || kb > qb) return;  // (wave-uniform) this block is in this wave's future
        const int j0 = kb * 32;
        TG_LDS uint8_t* kblk = cb;
        TG_LDS uint8_t* vblk = cb + G::BLOCK_BYTES;
        const TG_LDS lf4* sblk = (const TG_LDS lf4*)(cb + 2 * G::BLOCK_BYTES);
        // this lane's 16 key rows of the accumulators: j0 + 8 (i/4) + 4 g + i%4
        float sv[16];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const lf4 x = sblk[2 * i4 + g];
            sv[4 * i4] = x.x, sv[4 * i4 + 1] = x.y, sv[4 * i4 + 2] = x.z, sv[4 * i4 + 3] = x.w;
        }
        f32x16 sacc, dpacc = f32x16{};
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = sg * sv[i];
#pragma unroll
        for (int s = 0; s < G::QS; ++s) {
            sacc = tgd::mfma32(row_operand<D>(kblk, l32, g, s), qreg[s], sacc);
            dpacc = tgd::mfma32(row_operand<D>(vblk, l32, g, s), doreg[s], dpacc);
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
            for (int db = 0; db < G::DB; ++db)
                dqa[db] = tgd::mfma32(tr_operand<D>(kblk, lane, db, s), pb[s], dqa[db]);
    };
    issue(0, st0);
    for (int kb = 0; kb <= qb_last; kb += 2) {
        step(kb, st0, st1);
        if (kb + 1 <= qb_last) step(kb + 1, st1, st0);
    }
    if (!live) return;
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
    // block partials: both halves of a row carry the same log ratio
    const float lr = ok ? logf((float)(t + 1) / ((float)pos[t] + 1.0f)) : 0.0f;
    const float xl = tgd::wave_sum(dl * lr);
    const float xg = tgd::wave_sum(dgs);
    if (lane == 0) {
        dlamc[(int64_t)h * nqb + qb] = xl;
        dgp[(int64_t)h * nqb + qb] = xg;
    }
}

// ---- dk, dv, and the per-key partial of ds (this kv head's q heads)
// A workgroup holds kWavesPerBlock / wsplit key blocks; the wsplit waves of a
// key block share its q heads (wave r takes heads r, r + wsplit, ...) and
// their partial sums are added in LDS in the order r = 0, 1, ...
template <int D>
__global__ __launch_bounds__(64 * kWavesPerBlock) void bwd_dkv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ gains, const uint16_t* __restrict__ dO,
    const float4* __restrict__ rowv, int nk, int hq, int hkv, int kp, int wsplit, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dsp) {
    using G = Geo<D>;
    constexpr int STAGE = 2 * G::BLOCK_BYTES + 1024;  // Q block, dO block, 64 row values (32 used)
    constexpr int XCH = G::DB * 16 * 64 * 4;          // one wave's accumulator set, bytes
    static_assert(3 * XCH <= kWavesPerBlock * 2 * STAGE, "exchange fits the staging memory");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kWavesPerBlock * 2 * STAGE];
    __shared__ float sds[kWavesPerBlock][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int grp = hq / hkv;
    const int W = wsplit, S = kWavesPerBlock / wsplit;
    const int sidx = w / W, r = w % W;
    const int nkb = (nk + 31) / 32;
    const int hk = blockIdx.x % hkv;
    const int kb = (int)(blockIdx.x / hkv) * S + sidx;  // the longest walks (first key blocks) first
    const bool valid = kb < nkb;
    const int j = kb * 32 + l32;  // this lane's key column
    const int jc = min(j, nk - 1);
    const float rs = 1.0f / sqrtf((float)D);
    TG_LDS uint8_t* st0 = (TG_LDS uint8_t*)smem + w * 2 * STAGE;
    TG_LDS uint8_t* st1 = st0 + STAGE;
    const uint32_t q_bytes = (uint32_t)nk * (uint32_t)hq * (uint32_t)G::ROW_BYTES;
    const uint32_t row_bytes = (uint32_t)hq * (uint32_t)kp * 16u;

    u32x4 kreg[G::QS], vreg[G::QS];
#pragma unroll
    for (int s = 0; s < G::QS; ++s) {
        kreg[s] = *reinterpret_cast<const u32x4*>(k + ((int64_t)jc * hkv + hk) * D + 16 * s + 8 * g);
        vreg[s] = *reinterpret_cast<const u32x4*>(v + ((int64_t)jc * hkv + hk) * D + 16 * s + 8 * g);
    }
    const float sj = key_score[jc];
    f32x16 dka[G::DB], dva[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) dka[db] = dva[db] = f32x16{};
    float dsj = 0.0f;

    // (head, query block) pairs of this wave: heads r, r + W, ..., query
    // blocks kb .. nkb-1, streamed through two LDS stages of its own
    const int nq = valid ? nkb - kb : 0;
    const int nh = valid ? (grp - r + W - 1) / W : 0;
    const int iters = nq * nh;
    int ch = r, cq = kb;  // the current pair
    float gh_c = 0.0f, gh_n = 0.0f;
    auto issue = [&](int hh, int qb, TG_LDS uint8_t* __restrict__ nb) -> float {
        const int h = hk * grp + hh;
        load_block<D>(q, q_bytes, hq, h, qb * 32, nb, lane);
        load_block<D>(dO, q_bytes, hq, h, qb * 32, nb + G::BLOCK_BYTES, lane);
        lds_load<16>(rowv, row_bytes, nb + 2 * G::BLOCK_BYTES, ((uint32_t)h * (uint32_t)kp + qb * 32 + lane) * 16u);
        return gains[h];
    };
    auto step = [&](int it, TG_LDS uint8_t* __restrict__ cb, TG_LDS uint8_t* __restrict__ nb) {
        TG_WAIT_VMCNT(0);  // this pair's blocks are in LDS
        int hn = ch, qn = cq + 1;
        if (qn == nkb) {
            qn = kb;
            hn = ch + W;
        }
        if (it + 1 < iters) gh_n = issue(hn, qn, nb);
        const float gh = gh_c;
        const int t0 = cq * 32;
        TG_LDS uint8_t* bq = cb;
        TG_LDS uint8_t* bo = cb + G::BLOCK_BYTES;
        const TG_LDS lf4* brow = (const TG_LDS lf4*)(cb + 2 * G::BLOCK_BYTES);

        // this lane's 16 query rows: t0 + 8 (i/4) + 4 g + i%4
        float ar[16], lr[16], dr[16], mr[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const lf4 x = brow[8 * (i >> 2) + 4 * g + (i & 3)];
            ar[i] = x.x, lr[i] = x.y, dr[i] = x.z, mr[i] = x.w;
        }
        const float bias = sqrtf((float)D) * gh * sj;
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
        ch = hn;
        cq = qn;
        gh_c = gh_n;
    };
    if (iters > 0) gh_c = issue(ch, cq, st0);
    for (int it = 0; it < iters; it += 2) {
        step(it, st0, st1);
        if (it + 1 < iters) step(it + 1, st1, st0);
    }
    dsj = tgd::half_sum(dsj);

    // add the head-split partials: slot of wave (sidx, r >= 1) = sidx * (W - 1) + r - 1
    TG_LDS lf4* xs = (TG_LDS lf4*)smem;
    const int slot = sidx * (W - 1) + r - 1;
    __syncthreads();
    if (r > 0) {
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                xs[slot * (XCH / 16) + (db * 4 + i4) * 64 + lane] =
                    lf4{dka[db][4 * i4], dka[db][4 * i4 + 1], dka[db][4 * i4 + 2], dka[db][4 * i4 + 3]};
        sds[w][lane] = dsj;
    }
    __syncthreads();
    if (r == 0) {
        for (int rr = 1; rr < W; ++rr) {
            const int sl = sidx * (W - 1) + rr - 1;
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const lf4 x = xs[sl * (XCH / 16) + (db * 4 + i4) * 64 + lane];
                    dka[db][4 * i4] += x.x, dka[db][4 * i4 + 1] += x.y, dka[db][4 * i4 + 2] += x.z,
                        dka[db][4 * i4 + 3] += x.w;
                }
            dsj += sds[w + rr][lane];
        }
    }
    __syncthreads();
    if (r > 0) {
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                xs[slot * (XCH / 16) + (db * 4 + i4) * 64 + lane] =
                    lf4{dva[db][4 * i4], dva[db][4 * i4 + 1], dva[db][4 * i4 + 2], dva[db][4 * i4 + 3]};
    }
    __syncthreads();
    if (r == 0) {
        for (int rr = 1; rr < W; ++rr) {
            const int sl = sidx * (W - 1) + rr - 1;
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const lf4 x = xs[sl * (XCH / 16) + (db * 4 + i4) * 64 + lane];
                    dva[db][4 * i4] += x.x, dva[db][4 * i4 + 1] += x.y, dva[db][4 * i4 + 2] += x.z,
                        dva[db][4 * i4 + 3] += x.w;
                }
        }
        if (valid && j < nk) {
#pragma unroll
            for (int u = 0; u < 4 * G::DB; ++u) {
                const int i = 4 * (u % 4);
                const int dd = (u / 4) * 32 + 8 * (u % 4) + 4 * g;
                const int64_t off = ((int64_t)j * hkv + hk) * D + dd;
                *reinterpret_cast<float4*>(dk + off) = float4{dka[u / 4][i] * rs, dka[u / 4][i + 1] * rs,
                                                              dka[u / 4][i + 2] * rs, dka[u / 4][i + 3] * rs};
                *reinterpret_cast<float4*>(dv + off) =
                    float4{dva[u / 4][i], dva[u / 4][i + 1], dva[u / 4][i + 2], dva[u / 4][i + 3]};
            }
            if (g == 0) dsp[(int64_t)hk * kp + j] = dsj;
        }
    }
}

// ---- fixed-order sums: dscore[j] over the kv heads; dgains[h] over the query
// blocks; dtemp over heads and query blocks (workgroup hq)
__global__ __launch_bounds__(256) void bwd_reduce_score(const float* __restrict__ dsp, int nk, int hkv, int kp,
                                                        float* __restrict__ dscore) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= nk) return;
    float s = 0.0f;
    for (int hk = 0; hk < hkv; ++hk) s += dsp[(int64_t)hk * kp + j];
    dscore[j] = s;
}

__global__ __launch_bounds__(256) void bwd_reduce_rows(const float* __restrict__ dgp, const float* __restrict__ dlamc,
                                                       int nqb, int hq, float* __restrict__ dgains,
                                                       float* __restrict__ dtemp) {
    __shared__ double red[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int b = blockIdx.x;  // 0 .. hq-1: gains; hq: temperature
    const float* src = b < hq ? dgp + (int64_t)b * nqb : dlamc;
    const int n = b < hq ? nqb : hq * nqb;
    double acc = 0.0;
#pragma unroll 8
    for (int i = tid; i < n; i += 256) acc += (double)src[i];
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
    float4* rowv = reinterpret_cast<float4*>(ws.rowv);
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL(bwd_prep<D>, dim3((unsigned)(((int64_t)hq * kp + RPB - 1) / RPB)), dim3(256), 0, s, ws.out,
                       dout, ws.lse, pos, temp_coef, nk, hq, kp, rowv);
    const int nqb = (nk + 31) / 32;
    const int grp = hq / hkv;
    // dq: two heads of a kv group x two query blocks per workgroup (one head x
    // four query blocks when the group has one head)
    if (grp % 2 == 0) {
        const int items = hkv * (grp / 2) * ((nqb + 1) / 2);
        hipLaunchKernelGGL((bwd_dq<D, 2>), dim3((unsigned)items), dim3(64 * kWavesPerBlock), 0, s, q, k, v, key_score,
                           gains, pos, dout, rowv, nk, hq, hkv, kp, dq, ws.dlamc, ws.dgp);
    } else {
        const int items = hkv * grp * ((nqb + 3) / 4);
        hipLaunchKernelGGL((bwd_dq<D, 1>), dim3((unsigned)items), dim3(64 * kWavesPerBlock), 0, s, q, k, v, key_score,
                           gains, pos, dout, rowv, nk, hq, hkv, kp, dq, ws.dlamc, ws.dgp);
    }
    const int wsplit = grp >= 4 ? 4 : (grp >= 2 ? 2 : 1);
    const int kbs = kWavesPerBlock / wsplit;
    hipLaunchKernelGGL(bwd_dkv<D>, dim3((unsigned)(hkv * ((nqb + kbs - 1) / kbs))), dim3(64 * kWavesPerBlock), 0, s,
                       q, k, v, key_score, gains, dout, rowv, nk, hq, hkv, kp, wsplit, dk, dv, ws.dsp);
    hipLaunchKernelGGL(bwd_reduce_score, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, s, ws.dsp, nk, hkv, kp,
                       dscore);
    hipLaunchKernelGGL(bwd_reduce_rows, dim3((unsigned)(hq + 1)), dim3(256), 0, s, ws.dgp, ws.dlamc, nqb, hq, dgains,
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
