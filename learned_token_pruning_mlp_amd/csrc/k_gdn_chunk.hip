// k_gdn_chunk.hip -- the gated delta rule over the kept tokens in chunks on
// the matrix cores, the chunks' state-independent transforms formed first by
// a parallel pre-pass.
//
// The recurrent mixer of the hybrid backbone runs above the gate on the kept
// tokens only (fluxbbs.com TokenGate article, section on the hybrid
// architecture; aiwillknow.com, section on the two kinds of state in hybrid
// models).  Its core is the gated delta rule (Yang, Kautz and Hatamizadeh,
// "Gated Delta Networks", 2024): per v head, with S in R^{dv x dk},
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
// With w_t = beta_t (v_t - alpha_t S_{t-1} k_t) the rule reads
// S_t = alpha_t S_{t-1} + w_t k_t^T, and over a chunk of C tokens from the
// state S0, with R(t, i) = prod_{i<j<=t} alpha_j and gamma_t = prod_{j<=t}
// alpha_j (the chunkwise WY / UT form of the same paper),
//   (I + L) W = diag(beta) (V - diag(gamma) K S0^T),  L_ti = beta_t R(t,i) k_t.k_i  (i < t)
//   O   = diag(gamma) Q S0^T + M W,                    M_ti = R(t,i) q_t.k_i        (i <= t)
//   S_C = gamma_{C-1} S0 + W^T diag(R(C-1, .)) K.
// Everything but the products with S0 and W is independent of the state:
//  * gdn_prep, one workgroup per (v head, chunk), all chunks at once: the
//    Gram products K K^T and Q K^T, the decay table, L, M and
//    T = (I + L)^{-1} (16 x 16 diagonal blocks by forward substitution, then
//    T10 = -T11 L10 T00); it writes T and M as the matrix-core operands of
//    the two products that use them, already split, and gamma, beta and
//    R(C-1, .), into one record of the workspace per (v head, chunk);
//  * gdn_seq, one workgroup per 16 rows of a head's state, walks the chunks
//    in order with one barrier each.  Each of DK/32 owner waves holds a
//    32-column band of the rows in registers and forms its band's share of
//    K S0^T; after the barrier every owner sums the shares and forms all of
//    U = diag(beta)(V - diag(gamma) K S0^T) and W = T U itself, with the
//    tokens of the k dimension in the order the matrix cores leave them, so
//    W goes from the product straight into its band's state update; its
//    band's share of Q S0^T runs on the matrix cores meanwhile.  Two helper
//    waves form the outputs one chunk late, off the state's chain.  Each
//    chunk's k, q and v rows and its record go through LDS by direct loads,
//    three stages, issued two chunks ahead.
// The products run on 16x16x32 bf16 MFMA with fp32 accumulation.  k, q and v
// are bf16 already; every fp32 operand (the state, T, U, M, W) is split into
// three bf16 parts (hi + mid + lo, each the nearest bf16 to what the ones
// before it leave), a state product takes three MFMAs and an fp32 x fp32
// product the six terms above 2^-24 (the bf16x3 scheme of Henry, Tang and
// Heinecke, "Leveraging the bfloat16 Artificial Intelligence Datatype For
// Higher-Precision Computations", 2019).  Tokens past the last take
// alpha = 1, beta = 0 and zero rows, which leaves the state unchanged.
// Deterministic.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::f32x4;
using tgd::u32x2;
using tgd::u32x4;

#define TG_LDS __attribute__((address_space(3)))
typedef float lf4 __attribute__((ext_vector_type(4)));  // LDS-side float4
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;

constexpr int kCC = 32;  // tokens per chunk
constexpr int kRS = 16;  // state rows per workgroup of the sequential pass

// One record per (v head, chunk), in bytes: the A operands of W = T U and of
// M W (per 16-token row block tb, per part hi / mid / lo, per lane: 16 bytes),
// then, per 16-token half of the chunk, gamma, beta (0 past the last token)
// and R(C-1, i) of its tokens, 16 floats each (each half in 256 bytes).
constexpr int kRecT = 0;
constexpr int kRecM = 2 * 3 * 64 * 16;
constexpr int kRecTail = 2 * kRecM;
constexpr int kRecBytes = 16384;
constexpr int kTailGam = 0, kTailBet = 1, kTailRl = 2;
// byte offset in the record of gamma (a = kTailGam), beta or R(C-1, t) of token t
__host__ __device__ constexpr int rec_tail(int a, int t) { return kRecTail + 256 * (t >> 4) + 64 * a + 4 * (t & 15); }
static_assert(kRecTail + 512 <= kRecBytes, "record layout");

constexpr int kBufferWord3 = 0x00020000;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Direct load of SIZE bytes per lane from base + voff into LDS at
// lds + SIZE * lane (lds wave-uniform), through a raw buffer resource over
// `bytes` bytes (offsets at or past the end read as zero).  Issued from
// inline assembly so the compiler does not track these LDS writes: it would
// otherwise make the reads of one stage (and other LDS writes) wait for the
// loads in flight into the other.  The instruction writes no register; the
// kernels order it with explicit vector-memory waits and barriers written as
// inline assembly with a memory clobber.  (m0 is set right before each use.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int SIZE>
__device__ __forceinline__ void lds_load(const void* base, uint32_t bytes, TG_LDS uint8_t* lds, uint32_t voff) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const i32x4 rs = i32x4{(int32_t)(uint32_t)a, (int32_t)((uint32_t)(a >> 32) & 0xffffu), (int32_t)bytes,
                           kBufferWord3};
    const uint32_t m = (uint32_t)(uintptr_t)lds;
    if constexpr (SIZE == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(m), "v"(voff), "s"(rs)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                     :
                     : "s"(m), "v"(voff), "s"(rs)
                     : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define TG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Workgroup barrier that waits only for this wave's LDS accesses (the phases
// of a chunk talk through LDS): the next chunk's loads and this chunk's
// output stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(tgd::as_bf16x8(a), tgd::as_bf16x8(b), c, 0, 0, 0);
}

// eight fp32 values into three packed bf16 parts: x = hi + mid + lo
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& mid, u32x4& lo) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t h = tgd::cvt_pk_bf16(x[2 * p], x[2 * p + 1]);
        const float r0 = x[2 * p] - tgd::bf16lo(h), r1 = x[2 * p + 1] - tgd::bf16hi(h);
        const uint32_t m = tgd::cvt_pk_bf16(r0, r1);
        const uint32_t l = tgd::cvt_pk_bf16(r0 - tgd::bf16lo(m), r1 - tgd::bf16hi(m));
        hi[p] = h, mid[p] = m, lo[p] = l;
    }
}

// fp32 x fp32 product of 8-wide operands on a 16x16x32 tile, both split:
// the six cross terms above 2^-24, smallest first
__device__ __forceinline__ f32x4 mfma16_x6p(u32x4 ah, u32x4 am, u32x4 al, u32x4 bh, u32x4 bm, u32x4 bl,
                                            f32x4 acc) {
    acc = mfma16(am, bm, acc);
    acc = mfma16(al, bh, acc);
    acc = mfma16(ah, bl, acc);
    acc = mfma16(am, bh, acc);
    acc = mfma16(ah, bm, acc);
    return mfma16(ah, bh, acc);
}

// the same with the A operand split and B given as fp32
__device__ __forceinline__ f32x4 mfma16_x6s(u32x4 ah, u32x4 am, u32x4 al, const float* b, f32x4 acc) {
    u32x4 bh, bm, bl;
    split8(b, bh, bm, bl);
    return mfma16_x6p(ah, am, al, bh, bm, bl, acc);
}

// The token order of the k dimension in the products over a chunk's tokens
// that use T or M: k-slot e (0..7) of k-group g4 is token 4 g4 + e for e < 4
// and 16 + 4 g4 + e - 4 above, the order in which a 16x16 product leaves a
// lane's values of two 16-token blocks (D rows 4 g4 .. 4 g4 + 3 of each).
// So W, formed as two such blocks, is the B operand of the state update and
// of M W as it leaves the matrix cores, without a trip through LDS.
__host__ __device__ constexpr int kslot(int g4, int e) { return e < 4 ? 4 * g4 + e : 12 + 4 * g4 + e; }

__device__ __forceinline__ f32x4 mfma16_x6(const float* a, const float* b, f32x4 acc) {
    u32x4 ah, am, al;
    split8(a, ah, am, al);
    return mfma16_x6s(ah, am, al, b, acc);
}

// k and q rows of a chunk in LDS: the 16-byte pieces of row t at slot
// t * NP + (piece ^ t % NP), so the rows a tile's lanes read hit distinct banks.
template <int DK>
struct Rows {
    static constexpr int NP = DK / 8;
    static constexpr int KQ = kCC * DK * 2;  // bytes of the chunk's k (or q) rows
    static_assert(KQ % 4096 == 0, "k/q chunk in whole rounds of direct loads");
    __device__ static int boff(int row, int col) { return 16 * (row * NP + ((col >> 3) ^ (row % NP))) + 2 * (col & 7); }
    // k and q rows of tokens t0 .. t0 + kCC - 1 of q/k head hq into kb, qb
    __device__ static void issue(const uint16_t* k, const uint16_t* q, uint32_t qk_bytes, int64_t t0, int hk, int hq,
                                 TG_LDS uint8_t* kb, TG_LDS uint8_t* qb) {
        const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
#pragma unroll
        for (int it = 0; it < KQ / 4096; ++it) {
            const int e = it * 256 + tid;  // piece slot
            const int t = e / NP, p = (e % NP) ^ (t % NP);
            const uint32_t go = ((uint32_t)(t0 + t) * (uint32_t)hk + (uint32_t)hq) * (DK * 2u) + 16u * p;
            lds_load<16>(k, qk_bytes, kb + it * 4096 + w * 1024, go);
            lds_load<16>(q, qk_bytes, qb + it * 4096 + w * 1024, go);
        }
    }
    // 16-byte operand piece of k-step s (32 columns) for this lane's k-group
    __device__ static u32x4 rowop(const TG_LDS uint8_t* base, int row, int s, int g4) {
        return *(const TG_LDS u32x4*)(base + boff(row, 32 * s + 8 * g4));
    }
};

// ---- the pre-pass: one workgroup (4 waves) per (v head, chunk)
template <int DK>
__global__ __launch_bounds__(256) void gdn_prep(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                const float* __restrict__ alpha, const float* __restrict__ beta,
                                                int64_t n, int hk, int hv, int64_t nch, uint8_t* __restrict__ rec) {
    using RW = Rows<DK>;
    // LDS reused as the phases go (so that six workgroups fit on a CU): the
    // chunk's k and q rows, then T and L10 T00 over them; the Gram products,
    // then L and M in place
    __shared__ __attribute__((aligned(1024))) uint8_t stg[2 * RW::KQ + 2 * kCC * 4];
    __shared__ __attribute__((aligned(16))) float gkk[kCC][36];  // k_t . k_i, then L
    __shared__ __attribute__((aligned(16))) float gqk[kCC][36];  // q_t . k_i, then M
    __shared__ __attribute__((aligned(16))) float gam[kCC], bet[kCC], rl[kCC];
    static_assert(kCC * 36 * 4 + 16 * 20 * 4 <= 2 * RW::KQ, "T and L10 T00 over the k and q rows");
    float(*const lm)[36] = gkk;
    float(*const mm)[36] = gqk;
    float(*const tm)[36] = reinterpret_cast<float(*)[36]>(stg);
    float(*const xx)[20] = reinterpret_cast<float(*)[20]>(stg + kCC * 36 * 4);
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i16 = lane & 15, g4 = lane >> 4;
    const int h = (int)(blockIdx.x / nch);
    const int64_t ch = blockIdx.x % nch;
    const int hq = h / (hv / hk);
    const int64_t t0 = ch * kCC;
    const int tn = n - t0 < kCC ? (int)(n - t0) : kCC;
    TG_LDS uint8_t* kb = (TG_LDS uint8_t*)stg;
    TG_LDS uint8_t* qb = kb + RW::KQ;
    TG_LDS float* ab = (TG_LDS float*)(kb + 2 * RW::KQ);
    TG_LDS float* bb = ab + kCC;

    RW::issue(k, q, (uint32_t)n * (uint32_t)hk * DK * 2u, t0, hk, hq, kb, qb);
    if (w == 0 && lane < kCC) {
        const uint32_t g_bytes = (uint32_t)n * (uint32_t)hv * 4u;
        const uint32_t go = ((uint32_t)(t0 + lane) * (uint32_t)hv + (uint32_t)h) * 4u;
        lds_load<4>(alpha, g_bytes, (TG_LDS uint8_t*)ab, go);
        lds_load<4>(beta, g_bytes, (TG_LDS uint8_t*)bb, go);
    }
    TG_WAIT_VMCNT(0);
    lds_barrier();

    // Gram products, two 16 x 16 tiles a wave: K K^T blocks (0,0), (1,0),
    // (1,1), then Q K^T's (the blocks L and M need)
    if (w < 3) {
        const int ga = 2 * w, gb = 2 * w + 1;
        const int ra0 = ga % 3 == 0 ? 0 : 1, rb0 = ga % 3 == 2 ? 1 : 0;
        const int ra1 = gb % 3 == 0 ? 0 : 1, rb1 = gb % 3 == 2 ? 1 : 0;
        const TG_LDS uint8_t* xa = ga >= 3 ? qb : kb;
        const TG_LDS uint8_t* xg = gb >= 3 ? qb : kb;
        f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sk = 0; sk < DK / 32; ++sk) {
            acc0 = mfma16(RW::rowop(xa, 16 * ra0 + i16, sk, g4), RW::rowop(kb, 16 * rb0 + i16, sk, g4), acc0);
            acc1 = mfma16(RW::rowop(xg, 16 * ra1 + i16, sk, g4), RW::rowop(kb, 16 * rb1 + i16, sk, g4), acc1);
        }
        float(*g0)[36] = ga >= 3 ? gqk : gkk;
        float(*g1)[36] = gb >= 3 ? gqk : gkk;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            g0[16 * ra0 + 4 * g4 + j][16 * rb0 + i16] = acc0[j];
            g1[16 * ra1 + 4 * g4 + j][16 * rb1 + i16] = acc1[j];
        }
    }
    // decay table, a row quad a thread: R(t, i) = alpha_t alpha_{t-1} ...
    // alpha_{i+1} (1 at i = t, 0 above); gates past the last token are
    // alpha = 1, beta = 0.  Thread (t, c4) forms R(t, c4 + 3) from t down,
    // then the three below it.
    const int rt_t = tid >> 3, rt_c = 4 * (tid & 7);
    float rq[4];
    {
        float al[kCC];
#pragma unroll
        for (int m4 = 0; m4 < kCC / 4; ++m4) {
            const lf4 a4 = *(const TG_LDS lf4*)(ab + 4 * m4);
            al[4 * m4] = a4.x, al[4 * m4 + 1] = a4.y, al[4 * m4 + 2] = a4.z, al[4 * m4 + 3] = a4.w;
        }
#pragma unroll
        for (int i = 0; i < kCC; ++i) al[i] = i < tn ? al[i] : 1.0f;
        float acc = 1.0f;
#pragma unroll
        for (int jj = kCC - 1; jj >= 4; --jj)
            if (jj <= rt_t && jj > rt_c + 3) acc *= al[jj];
        // acc = R(t, c4 + 3) when c4 + 3 < t (and is 1 otherwise)
#pragma unroll
        for (int e = 3; e >= 0; --e) {
            const int i = rt_c + e;
            rq[e] = i <= rt_t ? acc : 0.0f;
            if (i >= 1 && i <= rt_t) acc *= al[i];  // R(t, i - 1) = R(t, i) alpha_i
        }
        if (rt_t == kCC - 1) *(float4*)&rl[rt_c] = float4{rq[0], rq[1], rq[2], rq[3]};
        if (rt_c == 0) {
            gam[rt_t] = rq[0] * al[0];
            bet[rt_t] = rt_t < tn ? bb[rt_t] : 0.0f;
        }
    }
    __syncthreads();

    // L and M, a row quad a thread, each over the Gram products it is formed
    // from (a thread reads and writes only its own quad)
    {
        const int t = rt_t, c4 = rt_c;
        const float4 k4 = *(const float4*)&gkk[t][c4];
        const float4 q4 = *(const float4*)&gqk[t][c4];
        const float bt = bet[t];
        float4 l4, m4;
        l4.x = c4 + 0 < t ? bt * rq[0] * k4.x : 0.0f;
        l4.y = c4 + 1 < t ? bt * rq[1] * k4.y : 0.0f;
        l4.z = c4 + 2 < t ? bt * rq[2] * k4.z : 0.0f;
        l4.w = c4 + 3 < t ? bt * rq[3] * k4.w : 0.0f;
        m4.x = c4 + 0 <= t ? rq[0] * q4.x : 0.0f;
        m4.y = c4 + 1 <= t ? rq[1] * q4.y : 0.0f;
        m4.z = c4 + 2 <= t ? rq[2] * q4.z : 0.0f;
        m4.w = c4 + 3 <= t ? rq[3] * q4.w : 0.0f;
        *(float4*)&lm[t][c4] = l4;
        *(float4*)&mm[t][c4] = m4;
    }
    __syncthreads();

    // T = (I + L)^{-1}: the diagonal 16 x 16 blocks by forward substitution
    // (wave 0: T00, wave 1: T11; lane (p, j) = (lane / 16, lane % 16) keeps
    // rows 4 p .. 4 p + 3 of column j and sums that slice of each row's dot
    // product, the four slices added by two lane swaps, which leave the same
    // bits in all four lanes), then T10 = -T11 (L10 T00) on the matrix cores
    if (w < 2) {
        const int o = 16 * w, j = i16, pp = g4;
        lf4 lrow[16];
#pragma unroll
        for (int u = 1; u < 16; ++u) lrow[u] = *(const lf4*)&lm[o + u][o + 4 * pp];
        float cbk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) cbk[e] = 4 * pp + e == j ? 1.0f : 0.0f;
#pragma unroll
        for (int u = 1; u < 16; ++u) {
            float part = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) part = fmaf(4 * pp + e < u ? lrow[u][e] : 0.0f, cbk[e], part);
            const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part), false, false);
            float sum = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
            const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum), false, false);
            sum = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
            const float val = u > j ? -sum : (u == j ? 1.0f : 0.0f);
            if (pp == (u >> 2)) cbk[u & 3] = val;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tm[o + 4 * pp + e][o + j] = cbk[e];
            if (w == 0) tm[4 * pp + e][16 + j] = 0.0f;  // T01 = 0
        }
    }
    __syncthreads();
    if (w == 0) {
        // X = L10 T00 (k = 0..15; k-groups 2 and 3 are zero)
        float a8[8], b8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a8[e] = g4 < 2 ? lm[16 + i16][8 * g4 + e] : 0.0f;
            b8[e] = g4 < 2 ? tm[8 * g4 + e][i16] : 0.0f;
        }
        f32x4 x = mfma16_x6(a8, b8, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) xx[4 * g4 + jj][i16] = x[jj];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // T10 = -T11 X
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a8[e] = g4 < 2 ? tm[16 + i16][16 + 8 * g4 + e] : 0.0f;
            b8[e] = g4 < 2 ? xx[8 * g4 + e][i16] : 0.0f;
        }
        x = mfma16_x6(a8, b8, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) tm[16 + 4 * g4 + jj][i16] = -x[jj];
    }
    __syncthreads();

    // The record: waves 0, 1 split T's 16-token row block w, waves 2, 3 M's
    // block w - 2, as the A operands (row 16 tb + i16, k-slots of k-group g4)
    uint8_t* r = rec + ((int64_t)h * nch + ch) * kRecBytes;
    {
        const int tb = w & 1;
        float(*src)[36] = w < 2 ? tm : mm;
        float a8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a8[e] = src[16 * tb + i16][kslot(g4, e)];
        u32x4 parts[3];
        split8(a8, parts[0], parts[1], parts[2]);
        uint8_t* dst = r + (w < 2 ? kRecT : kRecM);
#pragma unroll
        for (int p = 0; p < 3; ++p) *reinterpret_cast<u32x4*>(dst + ((tb * 3 + p) * 64 + lane) * 16) = parts[p];
    }
    if (tid < kCC) {
        *reinterpret_cast<float*>(r + rec_tail(kTailGam, tid)) = gam[tid];
        *reinterpret_cast<float*>(r + rec_tail(kTailBet, tid)) = bet[tid];
        *reinterpret_cast<float*>(r + rec_tail(kTailRl, tid)) = rl[tid];
    }
}

// ---- the sequential pass: one workgroup per kRS rows of a head's state,
// DK / 32 owner waves (each holds a 32-column band of the state) and two
// helper waves, one barrier a chunk
template <int DK, int DV>
struct Seq {
    static constexpr int DW = DK / 32;         // owner waves
    static constexpr int NT = 64 * (DW + 2);   // threads: the owners', then the helpers'
    static constexpr int BAND = kCC * 32 * 2;  // bytes of a band's k (or q) values of a chunk
    static constexpr int VB = kCC * kRS * 2;   // bytes of the workgroup's v values of a chunk
    static constexpr int RECB = kRecTail + 512;  // bytes of the record taken
    static constexpr int OFF_V = DW * 2 * BAND;  // stage: the owners' bands (k, then q), v, the record
    static constexpr int OFF_R = OFF_V + VB;
    static constexpr int STAGE = OFF_R + RECB;
    static constexpr int NLOAD = 9;  // direct loads a helper wave issues per chunk
    static_assert(VB == 2 * 4 * 128, "v chunk in two 4-byte rounds of the helpers");
    static_assert(kRecM == 2 * 3 * 1024 && RECB <= kRecBytes, "a row block of T or M in three 1 KB loads");
    static_assert(DV % kRS == 0 && DW >= 1 && DW <= 4, "state slices");
    static_assert(NT == 64 * (DK / 32 + 2), "the kernel's launch bounds");
};

// A band's k (or q) values of a chunk in LDS: token t's four 16-byte pieces
// (band columns 8 p .. 8 p + 7) at slots 4 t + (p ^ (t / 4) % 4), so that the
// operand reads of a product and the transposing reads hit distinct banks.
__device__ __forceinline__ int band_off(int t, int cc) {
    return 16 * (4 * t + ((cc >> 3) ^ ((t >> 2) & 3))) + 2 * (cc & 7);
}

template <int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 32 + 2)) void gdn_seq(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v, const float* state_in,
                                                             int64_t n, int hk, int hv, int64_t nch,
                                                             const uint8_t* __restrict__ rec,
                                                             float* __restrict__ out,
                                                             float* state_out) {  // state_out may be state_in
    using C = Seq<DK, DV>;
    constexpr int DW = C::DW, BAND = C::BAND;
    // three stages, one LDS object each (so the compiler can see that reads of
    // one never alias the loads in flight into another)
    __shared__ __attribute__((aligned(1024))) uint8_t stg0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t stg1[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t stg2[C::STAGE];
    // by chunk parity, per band: (K S0^T)^T and (Q S0^T)^T; W^T
    __shared__ __attribute__((aligned(16))) float ppk[2][DW][kRS][36];
    __shared__ __attribute__((aligned(16))) float ppq[2][DW][kRS][36];
    __shared__ __attribute__((aligned(16))) float ww[2][kRS][36];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i16 = lane & 15, g4 = lane >> 4;
    const int h = blockIdx.x / (DV / kRS), r0 = (blockIdx.x % (DV / kRS)) * kRS;
    const int hq = h / (hv / hk);
    const uint32_t qk_bytes = (uint32_t)n * (uint32_t)hk * DK * 2u;
    const uint32_t v_bytes = (uint32_t)n * (uint32_t)hv * DV * 2u;
    const bool owner = w < DW;
    const int tb = w - DW;  // a helper's 16-token block

    // Loads of a chunk, two chunks ahead: each owner takes its band of the k
    // and q rows (four 1 KB direct loads into its own region of the stage,
    // read by it alone, so it waits for them by itself); the helpers take the
    // workgroup's v values and the record, and wait for them before the
    // barrier that precedes their use.  A stage is refilled while the other
    // helper may still be reading the output operands of the chunk it held
    // (M's row block and gamma of its half): each helper loads exactly those
    // parts of the record that it alone reads there (T and M's row block tb,
    // the tail of half tb).
    auto issue_band = [&](int64_t c, TG_LDS uint8_t* __restrict__ sb) {
        const int64_t t0 = c * kCC;
        TG_LDS uint8_t* bk = sb + w * 2 * BAND;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int s = 64 * it + lane, t = s >> 2, p = (s & 3) ^ ((t >> 2) & 3);
            const uint32_t go =
                ((uint32_t)(t0 + t) * (uint32_t)hk + (uint32_t)hq) * (DK * 2u) + 64u * (uint32_t)w + 16u * p;
            lds_load<16>(k, qk_bytes, bk + 1024 * it, go);
            lds_load<16>(q, qk_bytes, bk + BAND + 1024 * it, go);
        }
    };
    auto issue_rest = [&](int64_t c, TG_LDS uint8_t* __restrict__ sb) {
        const int64_t t0 = c * kCC;
        const int tg = tid - 64 * DW;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int e = it * 128 + tg, t = e >> 3, wd = e & 7;
            const uint32_t go = ((uint32_t)(t0 + t) * (uint32_t)hv + (uint32_t)h) * (DV * 2u) + r0 * 2u + 4u * wd;
            lds_load<4>(v, v_bytes, sb + C::OFF_V + 4 * (it * 128 + tb * 64), go);
        }
        const uint8_t* r = rec + ((int64_t)h * nch + c) * kRecBytes;
#pragma unroll
        for (int it = 0; it < 3; ++it) {
            const int ot = kRecT + 3072 * tb + 1024 * it, om = kRecM + 3072 * tb + 1024 * it;
            lds_load<16>(r, kRecBytes, sb + C::OFF_R + ot, ot + 16u * lane);
            lds_load<16>(r, kRecBytes, sb + C::OFF_R + om, om + 16u * lane);
        }
        const int otl = kRecTail + 256 * tb;
        lds_load<4>(r, kRecBytes, sb + C::OFF_R + otl, otl + 4u * lane);
    };

    // The state: owner w holds columns 32 w .. 32 w + 31 of the slice's rows,
    // transposed (lane: row i16, columns 32 w + 16 u + 4 g4 + j, u = 0, 1,
    // j = 0..3), and, as the B operand of the chunk's products, split into
    // three bf16 parts (k-group g4 of the band takes band columns 4 g4 .. +3
    // and 16 + 4 g4 .. +3).
    float sr[2][4];
    u32x4 sh, sm, sl;
    if (owner) {
        const int c0 = 32 * w;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float4 x = float4{0.0f, 0.0f, 0.0f, 0.0f};
            if (state_in) x = *(const float4*)&state_in[((int64_t)h * DV + r0 + i16) * DK + c0 + 16 * u + 4 * g4];
            sr[u][0] = x.x, sr[u][1] = x.y, sr[u][2] = x.z, sr[u][3] = x.w;
        }
        const float x8[8] = {sr[0][0], sr[0][1], sr[0][2], sr[0][3], sr[1][0], sr[1][1], sr[1][2], sr[1][3]};
        split8(x8, sh, sm, sl);
    }
    // a product's A operand from a band: this lane's token, k-group g4's columns
    auto band_op = [&](const TG_LDS uint8_t* b, int t) {
        const u32x2 lo = *(const TG_LDS u32x2*)(b + band_off(t, 4 * g4));
        const u32x2 hi = *(const TG_LDS u32x2*)(b + band_off(t, 16 + 4 * g4));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    // The outputs of chunk cc, O = diag(gamma) Q S0^T + M W (the helpers, one
    // 16-token block each), formed one chunk late, off the state's chain: M's
    // operands and gamma are taken into registers before cc's stage is
    // refilled, the Q S0^T partials and W are kept by chunk parity.
    struct OutOps {
        u32x4 mh, mm, ml;
        lf4 gm;  // gamma of this lane's four tokens
    };
    auto out_ops = [&](const TG_LDS uint8_t* __restrict__ stage) {
        const TG_LDS uint8_t* rbc = stage + C::OFF_R;
        const TG_LDS u32x4* mp = (const TG_LDS u32x4*)(rbc + kRecM) + tb * 3 * 64 + lane;
        OutOps o;
        o.mh = mp[0], o.mm = mp[64], o.ml = mp[128];
        o.gm = *(const TG_LDS lf4*)(rbc + rec_tail(kTailGam, 16 * tb + 4 * g4));
        return o;
    };
    auto outputs = [&](int64_t cc, const OutOps& o) {
        const int64_t tc = cc * kCC;
        const int tnc = n - tc < kCC ? (int)(n - tc) : kCC;
        const int par = (int)(cc & 1);
        float4 pq[DW];
#pragma unroll
        for (int b = 0; b < DW; ++b) pq[b] = *(const float4*)&ppq[par][b][i16][16 * tb + 4 * g4];
        const float4 w0 = *(const float4*)&ww[par][i16][4 * g4], w1 = *(const float4*)&ww[par][i16][16 + 4 * g4];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float4 p = pq[0];
#pragma unroll
        for (int b = 1; b < DW; ++b) p.x += pq[b].x, p.y += pq[b].y, p.z += pq[b].z, p.w += pq[b].w;
        f32x4 acc = {o.gm.x * p.x, o.gm.y * p.y, o.gm.z * p.z, o.gm.w * p.w};
        const float b8[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};  // W, tokens in k-slot order
        acc = mfma16_x6s(o.mh, o.mm, o.ml, b8, acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 16 * tb + 4 * g4 + j;
            if (t < tnc) out[((tc + t) * hv + h) * DV + r0 + i16] = acc[j];
        }
    };

    // One chunk.  cb: its stage; ob: the stage of the chunk before, which
    // takes the chunk two ahead.
    auto chunk = [&](int64_t ch, const TG_LDS uint8_t* __restrict__ cb, TG_LDS uint8_t* __restrict__ ob) {
        const TG_LDS uint8_t* rb = cb + C::OFF_R;
        const int par = (int)(ch & 1);
        if (owner) {
            // ---- the band's (K S0^T)^T and its operands of Q S0^T, before the barrier
            if (ch + 1 < nch)
                TG_WAIT_VMCNT(4);  // this chunk's bands have landed (the next chunk's may be in flight)
            else
                TG_WAIT_VMCNT(0);
            const TG_LDS uint8_t* bk = cb + w * 2 * BAND;
            const u32x4 ak0 = band_op(bk, i16), ak1 = band_op(bk, 16 + i16);
            const u32x4 aq0 = band_op(bk + BAND, i16), aq1 = band_op(bk + BAND, 16 + i16);
            if (ch + 2 < nch) issue_band(ch + 2, ob);  // its own reads of that stage ended a chunk ago
            f32x4 x0 = mfma16(ak0, sl, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            f32x4 x1 = mfma16(ak1, sl, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            x0 = mfma16(ak0, sm, x0), x1 = mfma16(ak1, sm, x1);
            x0 = mfma16(ak0, sh, x0), x1 = mfma16(ak1, sh, x1);
            *(float4*)&ppk[par][w][i16][4 * g4] = float4{x0[0], x0[1], x0[2], x0[3]};
            *(float4*)&ppk[par][w][i16][16 + 4 * g4] = float4{x1[0], x1[1], x1[2], x1[3]};
            lds_barrier();

            // ---- every owner forms all of U and W = T U itself, the k
            // dimension (tokens) in k-slot order, so that W as it leaves the
            // matrix cores is the B operand of the update.  All operands in one
            // round of LDS reads: the band partials, v (transposing reads as
            // for K^T), beta, gamma and R(C-1, .), T's parts, K^T of the band.
            float4 pk[DW][2];
#pragma unroll
            for (int b = 0; b < DW; ++b)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) pk[b][hh] = *(const float4*)&ppk[par][b][i16][4 * g4 + 16 * hh];
            u32x2 vw[2];
            lf4 bt[2], gm[2], rv[2];
            u32x4 kt[2];
            const TG_LDS uint8_t* vb = cb + C::OFF_V;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int t = 4 * g4 + 16 * hh + (i16 >> 2);  // the token this lane addresses
                vw[hh] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                       (TG_LDS bf16x4_t*)(vb + 2 * (t * kRS + 4 * (i16 & 3)))));
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const u32x2 xw = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                                   (TG_LDS bf16x4_t*)(bk + band_off(t, 16 * u + 4 * (i16 & 3)))));
                    kt[u][2 * hh] = xw[0], kt[u][2 * hh + 1] = xw[1];
                }
                bt[hh] = *(const TG_LDS lf4*)(rb + rec_tail(kTailBet, 4 * g4 + 16 * hh));
                gm[hh] = *(const TG_LDS lf4*)(rb + rec_tail(kTailGam, 4 * g4 + 16 * hh));
                rv[hh] = *(const TG_LDS lf4*)(rb + rec_tail(kTailRl, 4 * g4 + 16 * hh));
            }
            const float gl = *(const TG_LDS float*)(rb + rec_tail(kTailGam, kCC - 1));
            u32x4 tpt[2][3];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const TG_LDS u32x4* tp = (const TG_LDS u32x4*)(rb + kRecT) + b * 3 * 64 + lane;
                tpt[b][0] = tp[0], tpt[b][1] = tp[64], tpt[b][2] = tp[128];
            }
            // (Q S0^T)^T of the band meanwhile, for the outputs
            f32x4 y0 = mfma16(aq0, sl, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            f32x4 y1 = mfma16(aq1, sl, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            y0 = mfma16(aq0, sm, y0), y1 = mfma16(aq1, sm, y1);
            y0 = mfma16(aq0, sh, y0), y1 = mfma16(aq1, sh, y1);
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

            // U = diag(beta)(V - diag(gamma) K S0^T), this lane's eight (token, row i16)
            float u8[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                float p4[4] = {pk[0][hh].x, pk[0][hh].y, pk[0][hh].z, pk[0][hh].w};
#pragma unroll
                for (int b = 1; b < DW; ++b)
                    p4[0] += pk[b][hh].x, p4[1] += pk[b][hh].y, p4[2] += pk[b][hh].z, p4[3] += pk[b][hh].w;
                const float v4[4] = {tgd::bf16lo(vw[hh][0]), tgd::bf16hi(vw[hh][0]), tgd::bf16lo(vw[hh][1]),
                                     tgd::bf16hi(vw[hh][1])};
#pragma unroll
                for (int e = 0; e < 4; ++e) u8[4 * hh + e] = bt[hh][e] * (v4[e] - gm[hh][e] * p4[e]);
            }
            u32x4 uh, um, ul;
            split8(u8, uh, um, ul);
            // W's two 16-token blocks: lane (i16, g4) takes W(4 g4 + j, i16) and W(16 + 4 g4 + j, i16)
            f32x4 wb0 = mfma16_x6p(tpt[0][0], tpt[0][1], tpt[0][2], uh, um, ul, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            f32x4 wb1 = mfma16_x6p(tpt[1][0], tpt[1][1], tpt[1][2], uh, um, ul, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            *(float4*)&ppq[par][w][i16][4 * g4] = float4{y0[0], y0[1], y0[2], y0[3]};
            *(float4*)&ppq[par][w][i16][16 + 4 * g4] = float4{y1[0], y1[1], y1[2], y1[3]};
            if (w == 0) {
                *(float4*)&ww[par][i16][4 * g4] = float4{wb0[0], wb0[1], wb0[2], wb0[3]};
                *(float4*)&ww[par][i16][16 + 4 * g4] = float4{wb1[0], wb1[1], wb1[2], wb1[3]};
            }

            // ---- the band's update S^T <- gamma_last S^T + K^T diag(R(C-1, .)) W
            const float b8[8] = {rv[0][0] * wb0[0], rv[0][1] * wb0[1], rv[0][2] * wb0[2], rv[0][3] * wb0[3],
                                 rv[1][0] * wb1[0], rv[1][1] * wb1[1], rv[1][2] * wb1[2], rv[1][3] * wb1[3]};
            u32x4 bh, bm, bl;
            split8(b8, bh, bm, bl);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 acc = {gl * sr[u][0], gl * sr[u][1], gl * sr[u][2], gl * sr[u][3]};
                acc = mfma16(kt[u], bl, acc);
                acc = mfma16(kt[u], bm, acc);
                acc = mfma16(kt[u], bh, acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) sr[u][j] = acc[j];
            }
            const float x8[8] = {sr[0][0], sr[0][1], sr[0][2], sr[0][3], sr[1][0], sr[1][1], sr[1][2], sr[1][3]};
            split8(x8, sh, sm, sl);
        } else {
            // ---- helpers: the previous chunk's output operands from its stage,
            // the chunk two ahead into it, then that chunk's outputs.  They
            // start ~512 cycles after the barrier: their LDS reads and the
            // loads they issue would otherwise land in the owners' round of LDS
            // reads, which bounds the chunk.
            lds_barrier();
            __builtin_amdgcn_s_sleep(8);
            OutOps prev;
            if (ch > 0) prev = out_ops(ob);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // its reads of that stage are done
            if (ch + 2 < nch) {
                issue_rest(ch + 2, ob);
                TG_WAIT_VMCNT(C::NLOAD);  // the next chunk's v and record have landed
            } else {
                TG_WAIT_VMCNT(0);
            }
            if (ch > 0) outputs(ch - 1, prev);
        }
    };
    TG_LDS uint8_t* s0 = (TG_LDS uint8_t*)stg0;
    TG_LDS uint8_t* s1 = (TG_LDS uint8_t*)stg1;
    TG_LDS uint8_t* s2 = (TG_LDS uint8_t*)stg2;
    if (nch > 0) {
        if (owner) {
            issue_band(0, s0);
            if (nch > 1) issue_band(1, s1);
        } else {
            issue_rest(0, s0);
            if (nch > 1) {
                issue_rest(1, s1);
                TG_WAIT_VMCNT(C::NLOAD);
            } else {
                TG_WAIT_VMCNT(0);
            }
        }
    }
    for (int64_t ch = 0; ch < nch; ch += 3) {
        chunk(ch, s0, s2);
        if (ch + 1 < nch) chunk(ch + 1, s1, s0);
        if (ch + 2 < nch) chunk(ch + 2, s2, s1);
    }
    if (nch > 0) {
        lds_barrier();  // the last chunk's Q S0^T partials and W
        if (!owner) {
            const int64_t cl = nch - 1;
            outputs(cl, out_ops(cl % 3 == 0 ? s0 : (cl % 3 == 1 ? s1 : s2)));
        }
    }
    if (owner && state_out) {
        const int c0 = 32 * w;
#pragma unroll
        for (int u = 0; u < 2; ++u)
            *(float4*)&state_out[((int64_t)h * DV + r0 + i16) * DK + c0 + 16 * u + 4 * g4] =
                float4{sr[u][0], sr[u][1], sr[u][2], sr[u][3]};
    }
}

template <int DK, int DV>
int launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha, const float* beta,
           const float* state_in, int64_t n, int hk, int hv, float* out, float* state_out, uint8_t* rec,
           hipStream_t s) {
    const int64_t nch = (n + kCC - 1) / kCC;
    if (nch > 0)
        hipLaunchKernelGGL(gdn_prep<DK>, dim3((unsigned)(hv * nch)), dim3(256), 0, s, q, k, alpha, beta, n, hk, hv,
                           nch, rec);
    hipLaunchKernelGGL((gdn_seq<DK, DV>), dim3((unsigned)(hv * (DV / kRS))), dim3(Seq<DK, DV>::NT), 0, s, q, k, v, state_in, n,
                       hk, hv, nch, rec, out, state_out);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace

namespace tgi {

size_t gdn_chunk_ws_bytes(int64_t n, int hv) {
    const int64_t nch = (n + kCC - 1) / kCC;
    return (size_t)(nch > 0 ? nch : 1) * (size_t)hv * kRecBytes;
}

int launch_gated_delta_rule_chunked(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha,
                                    const float* beta, const float* state_in, int64_t n, int hk, int hv, int dk,
                                    int dv, float* out, float* state_out, void* ws, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    uint8_t* rec = static_cast<uint8_t*>(ws);
    if (dk == 128 && dv == 128) return launch<128, 128>(q, k, v, alpha, beta, state_in, n, hk, hv, out, state_out, rec, s);
    if (dk == 128 && dv == 64) return launch<128, 64>(q, k, v, alpha, beta, state_in, n, hk, hv, out, state_out, rec, s);
    if (dk == 64 && dv == 128) return launch<64, 128>(q, k, v, alpha, beta, state_in, n, hk, hv, out, state_out, rec, s);
    if (dk == 64 && dv == 64) return launch<64, 64>(q, k, v, alpha, beta, state_in, n, hk, hv, out, state_out, rec, s);
    return TG_EUNSUPPORTED;
}

}  // namespace tgi
