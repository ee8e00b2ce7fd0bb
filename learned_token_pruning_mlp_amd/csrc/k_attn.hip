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
//  * The accumulator of S^T starts at sqrt(D) * g_h * s_j, so the matrix core
//    adds the key bias; each probability is then one FMA and one exp2:
//    p = 2^(a_t * S - m) with a_t = lambda_t * log2(e) / sqrt(D).
//  * The S^T accumulator layout is the B-operand layout of O^T = V^T . P^T
//    (keys along k), so P goes from registers to the matrix core with one
//    hardware bf16 conversion per pair; the row sums are taken from the same
//    bf16 pairs (v_dot2_f32_bf16, two keys per instruction), so numerator
//    and denominator use one P.
//  * A row whose temperature lambda_t is negative (possible when few early
//    tokens were kept) is computed as |lambda_t| * (-S): its query and its
//    key-bias scale change sign, which is exact, so every row has a positive
//    exp2 scale and one code path serves all rows.
//  * Per 32-key block a wave issues all its K-operand and score reads, then
//    the eight S^T products, then (first block of a super-tile) the next
//    super-tile's loads, then the transposing V reads, so LDS and memory-queue
//    latency overlap the matrix cores; it raises its issue priority while it
//    issues the P.V products, so that the SIMD's other wave, in its softmax,
//    does not hold them back.
//  * Work split: a workgroup owns one GQA kv head, HPW of its q heads and a
//    pair of 32-row query blocks (b, last - b), so every workgroup carries the
//    same causal work.  The keys of a query block are streamed as super-tiles
//    of NS x 32 keys; wave (head, split) takes the split-th 32 keys of each
//    super-tile for its head, keeping its own running max and sum, and the
//    NS partial results of a head are merged through LDS at the end of the
//    block.  HPW heads share every K/V super-tile in LDS.  With 2 heads x 4
//    splits a 2048-key prompt still gives two waves per SIMD.
//  * K and V super-tiles go from memory straight into LDS with 16-byte
//    direct loads, double-buffered (the next super-tile is in flight while
//    this one is multiplied).  Rows are stored with their 16-byte pieces
//    XOR-permuted by a function of the row that keeps the K-operand reads
//    and the transposing V reads (ds_read_b64_tr_b16, which hands each lane
//    four keys of one head_dim column) free of LDS bank conflicts.
//  * Work items are laid out so all workgroups of one kv head run on the same
//    XCD (workgroups go round-robin over the 8 XCDs), keeping that head's K/V
//    in one L2.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::f32x16;
using tgd::u32x2;
using tgd::u32x4;
template <int N>
using IC = std::integral_constant<int, N>;

#define TG_LDS __attribute__((address_space(3)))
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;

constexpr int kXcds = 8;
// Fourth word of a raw buffer resource on gfx9-family parts: 32-bit data
// format, no swizzle; with a zero stride, offsets at or past num_records read
// as zero.
constexpr int kBufferWord3 = 0x00020000;
constexpr float kLog2e = 1.44269504088896340736f;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define TG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

template <int D, int HPW, int RB, int NS, int KB>
struct AttnCfg {
    static constexpr int WAVES = HPW * RB * NS;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int QROWS = 32 * RB;             // query rows per block
    static constexpr int WKEYS = 32 * KB;             // keys per wave per super-tile
    static constexpr int SKEYS = WKEYS * NS;          // keys per super-tile
    static constexpr int PIECES = D / 8;              // 16-byte pieces per K/V row
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int TILE_BYTES = SKEYS * ROW_BYTES;  // K (or V) bytes per super-tile
    static constexpr int BLOCKS = TILE_BYTES / 1024;      // 1 KB direct-load blocks
    static constexpr int LOADS = BLOCKS / WAVES;          // per wave, for K and again for V
    static constexpr int DB = D / 32;                 // 32-row blocks of head_dim in O^T
    static constexpr int QS = D / 16;                 // k-steps of the QK^T product
    static_assert(BLOCKS % WAVES == 0 && LOADS >= 1, "tile shape");
    static_assert(SKEYS <= 64 * WAVES, "one score per lane");
    // merge scratch: one slot per wave holding half of its O^T accumulators
    // (8 floats per lane per 32 head_dim rows), taken from the K buffer of the
    // finished stage, then its V buffer; a slot never straddles the two
    static constexpr int SLOT_BYTES = DB * 2048;
    static_assert(NS == 1 || (WAVES * SLOT_BYTES <= 2 * TILE_BYTES && TILE_BYTES % SLOT_BYTES == 0),
                  "merge scratch");
    static_assert(NS == 1 || NS == 2 || NS == 4, "merge rounds");
};

// Direct load of `size` bytes per lane from base + voff + soff into LDS at
// lds + size * lane, through a raw buffer resource covering `bytes` bytes:
// offsets at or past the end read as zero.
template <int SIZE>
__device__ __forceinline__ void buffer_to_lds(const void* base, int bytes, TG_LDS uint8_t* lds, uint32_t voff,
                                              uint32_t soff) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferWord3);
    static_assert(SIZE == 16 || SIZE == 4, "direct-load size");
    if constexpr (SIZE == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TG_LDS void*)lds, 16, voff, soff, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TG_LDS void*)lds, 4, voff, soff, 0, 0);
}

// Permutation of the 16-byte pieces inside a K/V row (XOR mask by row).
// gfx950 LDS has 64 banks; a 16-byte read serves 16 consecutive lanes per
// cycle and needs their (address/16) mod 16 distinct, the transposing 8-byte
// read serves 32 lanes per cycle and needs (address/8) mod 32 distinct.
// 256-byte rows: swap the two-bit halves of row mod 16 (a bijection over any
// 16 consecutive rows for the K-operand reads; rows 4k..4k+3 differ in the
// upper two bits for the transposing V reads).  128-byte rows (two rows per
// bank sweep): rotate (row/2) mod 8 right by one bit.
template <int PIECES>
__device__ __forceinline__ int swz(int r) {
    if (PIECES == 16) {
        const int x = r & 15;
        return ((x << 2) | (x >> 2)) & 15;
    }
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
}

// Workgroup barrier that waits only for this wave's LDS accesses: memory
// loads in flight (the next query block's rows, the next super-tile) stay in
// flight across it.  The memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// acc + lo + hi of a packed bf16 pair, in fp32.
__device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    constexpr uint32_t kOnes = 0x3f803f80u;  // (1.0, 1.0) in bf16
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), __builtin_bit_cast(bf16x2_t, kOnes),
                                           acc, false);
}

// Normalise and write units LO .. LO+N-1 of a lane's O^T accumulators (unit
// u = 4 values: head_dim rows 32 (u/4) + 8 (u%4) + 4 g .. +3 of query row t).
// Compile-time unit indices keep the accumulators in fixed registers.
template <int D, int LO, int N, bool OUT_F32>
__device__ __forceinline__ void store_units(const f32x16 (&o)[D / 32], float l, int t, int nk, int hq, int h, int g,
                                            void* __restrict__ out) {
    if (t >= nk) return;
    const float inv = 1.0f / l;
#pragma unroll
    for (int u = LO; u < LO + N; ++u) {
        const int i = 4 * (u % 4);
        const int dd = (u / 4) * 32 + 8 * (u % 4) + 4 * g;
        const int64_t off = ((int64_t)t * hq + h) * D + dd;
        const float y0 = o[u / 4][i] * inv, y1 = o[u / 4][i + 1] * inv;
        const float y2 = o[u / 4][i + 2] * inv, y3 = o[u / 4][i + 3] * inv;
        if (OUT_F32) {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + off) = float4{y0, y1, y2, y3};
        } else {
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + off) =
                u32x2{tgd::cvt_pk_bf16(y0, y1), tgd::cvt_pk_bf16(y2, y3)};
        }
    }
}

template <int D, int HPW, int RB, int NS, int KB, bool OUT_F32>
__global__ __launch_bounds__(64 * HPW * RB * NS, 1) void gated_attn(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ kk,
                                                              const uint16_t* __restrict__ v,
                                                              const float* __restrict__ key_score,
                                                              const float* __restrict__ gains,
                                                              float temp_coef, const int32_t* __restrict__ pos,
                                                              int nk, int hq, int hkv, int npairs, int per_xcd,
                                                              int n_items, void* __restrict__ out,
                                                              float* __restrict__ lse, int lse_ld) {
    using C = AttnCfg<D, HPW, RB, NS, KB>;
    // one set of LDS objects per pipeline stage, so the compiler can see that
    // reads of one stage never alias the loads in flight into the other
    __shared__ __attribute__((aligned(1024))) uint8_t sK0[C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sV0[C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sK1[C::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sV1[C::TILE_BYTES];
    __shared__ __attribute__((aligned(256))) float sS0[C::SKEYS];
    __shared__ __attribute__((aligned(256))) float sS1[C::SKEYS];
    __shared__ float mbuf[HPW * RB][NS][32];
    __shared__ float lbuf[HPW * RB][NS][32];

    // ---- work item: (kv head, head group, query-block pair), XCD-aware
    const int lin = blockIdx.x;
    const int item = (lin % kXcds) * per_xcd + lin / kXcds;
    if (item >= n_items) return;
    const int G = hq / hkv;
    const int n_hg = G / HPW;
    const int per_head = n_hg * npairs;
    const int kvh = item / per_head;
    const int rem = item % per_head;
    const int hg = rem / npairs;
    const int pr = rem % npairs;
    const int nqb = (nk + C::QROWS - 1) / C::QROWS;
    const int qbA = pr, qbB = nqb - 1 - pr;
    const auto nst = [&](int qb) { return (min(nk, C::QROWS * qb + C::QROWS) - 1) / C::SKEYS + 1; };
    const int nA = nst(qbA);
    const int ntot = nA + (qbB != qbA ? nst(qbB) : 0);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
    const int l32 = lane & 31, g = lane >> 5;
    const int hl = wave % HPW, rb = (wave / HPW) % RB, sp = wave / (HPW * RB);
    const int hr = hl + HPW * rb;  // this wave's (head, row block) slot among the merge partners
    const int h = kvh * G + hg * HPW + hl;
    const float sg = sqrtf((float)D) * gains[h];
    const int quad = lane >> 4, jj = lane & 15;
    const int tr_row = jj >> 2, tr_col = 4 * (jj & 3);

    // ---- direct loads of one super-tile (keys j0 .. j0+SKEYS-1), through
    // buffer resources: each lane's 32-bit offset within a tile is fixed for
    // the kernel and the tile start is a scalar offset.  Rows past the last
    // key fall outside the resource and read as zeros (they are always
    // causally masked).
    const int row_bytes_g = hkv * D * 2;  // bytes between consecutive keys of K and V
    const int kv_bytes = nk * row_bytes_g;
    uint32_t goff[C::LOADS];
#pragma unroll
    for (int r = 0; r < C::LOADS; ++r) {
        constexpr int rows_per_inst = 64 / C::PIECES;
        const int blk = r * C::WAVES + wave;
        const int row = blk * rows_per_inst + lane / C::PIECES;
        const int piece = (lane % C::PIECES) ^ swz<C::PIECES>(row);
        goff[r] = row * row_bytes_g + kvh * D * 2 + piece * 16;
    }
    auto issue = [&](int it, uint8_t* __restrict__ sK, uint8_t* __restrict__ sV, float* __restrict__ sS) {
        const int st = it < nA ? it : it - nA;
        const int j0 = st * C::SKEYS;
        const int tile_off = j0 * row_bytes_g;
#pragma unroll
        for (int r = 0; r < C::LOADS; ++r) {
            const int blk = r * C::WAVES + wave;
            buffer_to_lds<16>(kk, kv_bytes, (TG_LDS uint8_t*)sK + blk * 1024, goff[r], tile_off);
            buffer_to_lds<16>(v, kv_bytes, (TG_LDS uint8_t*)sV + blk * 1024, goff[r], tile_off);
        }
        if (wave * 64 < C::SKEYS)  // scores: one per lane, first SKEYS/64 waves
            buffer_to_lds<4>(key_score, nk * 4, (TG_LDS uint8_t*)sS + wave * 256, (wave * 64 + lane) * 4, j0 * 4);
    };

    // ---- per query-block state of this wave (head h, rows q0 .. q0+31)
    u32x4 qreg[C::QS];
    int qpos = 0;
    f32x16 o[C::DB];
    float m_run = -INFINITY, l_run = 0.0f, a_t = 0.0f, sgl = 0.0f;
    int q0 = 0, t = 0, wave_last = 0;

    // Query rows and original position of this lane's row of block qb.
    auto fetch_q = [&](int qb) {
        const int tq = C::QROWS * qb + 32 * rb + l32;
        const bool ok = tq < nk;
        const uint16_t* qp = q + ((int64_t)tq * hq + h) * D;
#pragma unroll
        for (int s = 0; s < C::QS; ++s)
            qreg[s] = ok ? *reinterpret_cast<const u32x4*>(qp + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
        qpos = ok ? pos[tq] : 0;
    };
    // fetched: fetch_q(qb) was issued already (the second block's rows go
    // out before the first block's merge, so their latency hides behind it)
    auto begin_block = [&](int qb, bool fetched) {
        q0 = C::QROWS * qb + 32 * rb;
        t = q0 + l32;
        wave_last = min(nk - 1, q0 + 31);
        const bool ok = t < nk;
        if (!fetched) fetch_q(qb);
        float lam = 1.0f;
        if (ok) lam = 1.0f + temp_coef * logf((float)(t + 1) / ((float)qpos + 1.0f));
        // A row with lambda < 0 takes z = |lambda| * (-S): its query and its
        // key-bias scale change sign (exact), so every row has a positive exp2
        // scale; lambda = 0 (all logits 0) takes a tiny positive one.
        const bool neg = lam < 0.0f;
        a_t = fmaxf(fabsf(lam) * kLog2e * (1.0f / sqrtf((float)D)), 1e-30f);
        sgl = neg ? -sg : sg;
        if (neg) {
#pragma unroll
            for (int s = 0; s < C::QS; ++s) qreg[s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        }
        m_run = -INFINITY;
        l_run = 0.0f;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
    };

    // ---- merge the NS split waves of each head and write the block's rows.
    // Recursive halving over the splits: in each round a wave and its partner
    // (split indices differing in one bit) swap halves of the head_dim units
    // they still hold; each keeps one half and adds the partner's copy of it,
    // both rescaled to the pair's common max.  After log2(NS) rounds a wave
    // holds the merged sums of 1/NS of head_dim and writes those output
    // columns.  A wave writes each round's outgoing half into the LDS slot it
    // read in the round before (whose only reader was itself), so one barrier
    // per round suffices.  A unit is 4 accumulator values per lane (16 bytes,
    // 1 KB per wave).
    auto finish_block = [&](uint8_t* scK, uint8_t* scV) __attribute__((always_inline)) {
        constexpr int U = 4 * C::DB;
        float l = tgd::half_sum(l_run);  // per query (the half-waves held different keys)
        if constexpr (NS == 1) {
            store_units<D, 0, U, OUT_F32>(o, l, t, nk, hq, h, g, out);
            if (lse && g == 0 && t < nk) lse[(int64_t)h * lse_ld + t] = m_run + __log2f(l);
        } else {
            const auto slot_ptr = [&](int slot) {
                const int off = (hr * NS + slot) * C::SLOT_BYTES;
                return reinterpret_cast<float*>(off < C::TILE_BYTES ? scK + off : scV + (off - C::TILE_BYTES));
            };
            lds_barrier();  // every wave is done with this stage's K/V
            // One round with split stride S while holding units LO .. LO+2*half-1;
            // x = XOR of the strides of the earlier rounds.  The branch on this
            // wave's split bit is wave-uniform; every wave meets one barrier.
            const auto round = [&](auto self, auto LO, auto S, int x) __attribute__((always_inline)) -> void {
                constexpr int lo = decltype(LO)::value, s = decltype(S)::value;
                constexpr int half = U * s / NS;
                const int ws = sp ^ x, rs = sp ^ s ^ x;
                const auto step = [&](auto KEEP) __attribute__((always_inline)) {
                    constexpr int keep = decltype(KEEP)::value;
                    constexpr int give = keep == lo ? lo + half : lo;
                    float* dst = slot_ptr(ws);
#pragma unroll
                    for (int u = give; u < give + half; ++u) {
                        const f32x16& a = o[u / 4];
                        const int i = 4 * (u % 4);
                        *reinterpret_cast<float4*>(dst + 4 * ((u - give) * 64 + lane)) =
                            float4{a[i], a[i + 1], a[i + 2], a[i + 3]};
                    }
                    if (g == 0) {
                        mbuf[hr][ws][l32] = m_run;
                        lbuf[hr][ws][l32] = l;
                    }
                    lds_barrier();
                    const float mp = mbuf[hr][rs][l32], lp = lbuf[hr][rs][l32];
                    const float mn = fmaxf(m_run, mp);
                    const float fs = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mn);
                    const float fp = mp == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mp - mn);
                    const float* src = slot_ptr(rs);
#pragma unroll
                    for (int u = keep; u < keep + half; ++u) {
                        const float4 y = *reinterpret_cast<const float4*>(src + 4 * ((u - keep) * 64 + lane));
                        f32x16& a = o[u / 4];
                        const int i = 4 * (u % 4);
                        a[i] = fmaf(a[i], fs, y.x * fp);
                        a[i + 1] = fmaf(a[i + 1], fs, y.y * fp);
                        a[i + 2] = fmaf(a[i + 2], fs, y.z * fp);
                        a[i + 3] = fmaf(a[i + 3], fs, y.w * fp);
                    }
                    l = fmaf(l, fs, lp * fp);
                    m_run = mn;
                    if constexpr (s > 1)
                        self(self, KEEP, IC<s / 2>{}, x ^ s);
                    else {
                        store_units<D, keep, half, OUT_F32>(o, l, t, nk, hq, h, g, out);
                        if (lse && sp == 0 && g == 0 && t < nk) lse[(int64_t)h * lse_ld + t] = m_run + __log2f(l);
                    }
                };
                if (sp & s)
                    step(IC<lo + half>{});
                else
                    step(IC<lo>{});
            };
            round(round, IC<0>{}, IC<NS / 2>{}, 0);
        }
    };

    // ---- LDS byte offsets of this wave's operand reads, fixed for the whole
    // kernel.  The swizzle depends on the row modulo 16 only, so the offsets
    // of key block kb and of the second 16-key half of a block are these plus
    // constants.
    //  K (A operand of S^T): key row rb0 + l32, piece 2s + g.
    //  V (A operand of O^T, transposing read): lane a+4e of a 16-lane group
    //  addresses key row kbase + e and head_dim columns dbase + 4a .. + 3.
    const int rb0 = C::WKEYS * sp;
    uint32_t koff[C::QS];
#pragma unroll
    for (int s = 0; s < C::QS; ++s) {
        const int row = rb0 + l32;
        koff[s] = row * C::ROW_BYTES + 16 * ((2 * s + g) ^ swz<C::PIECES>(row));
    }
    uint32_t voff[C::DB][2];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int row = rb0 + 4 * (quad >> 1) + 8 * half + tr_row;
            const int dcol = db * 32 + 16 * (quad & 1) + tr_col;
            voff[db][half] = row * C::ROW_BYTES + 16 * ((dcol >> 3) ^ swz<C::PIECES>(row)) + 8 * ((dcol >> 2) & 1);
        }
    }
    const uint32_t soff = 4 * (rb0 + 4 * g);

    // Running maxima are only raised when a row's block max exceeds them by
    // more than 2^kTau in the exp2 domain; in between, probabilities up to
    // 2^kTau are accumulated (exact in fp32, bf16 keeps its relative
    // precision).  This skips nearly every rescale of the accumulators.
    constexpr float kTau = 8.0f;

    // ---- one 32-key block of this wave's slice: S^T, online softmax, P.V,
    // in two parts: the front issues the K-operand and score reads and the
    // S^T products, the back reads V and does the softmax and P.V.
    // Every row has a_t > 0, so the logits in the exp2 domain are a_t * S,
    // the block max is a_t * max(S) (rounding is monotonic) and
    // p = 2^(a_t * S - m) is one FMA and one exp2.
    auto block_front = [&](int kb, const uint8_t* __restrict__ tK,
                           const float* __restrict__ tS) __attribute__((always_inline)) -> f32x16 {
        const uint8_t* bK = tK + kb * 32 * C::ROW_BYTES;
        const float* bS = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(tS) + soff) + 32 * kb;
        // all K-operand and score reads of the block go out together
        u32x4 ka[C::QS];
#pragma unroll
        for (int s = 0; s < C::QS; ++s) ka[s] = *reinterpret_cast<const u32x4*>(bK + koff[s]);
        float4 sv[4];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) sv[i4] = *reinterpret_cast<const float4*>(bS + 8 * i4);
        // S^T for 32 keys x 32 queries, started at the key bias.
        f32x16 sacc;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            sacc[4 * i4 + 0] = sgl * sv[i4].x;
            sacc[4 * i4 + 1] = sgl * sv[i4].y;
            sacc[4 * i4 + 2] = sgl * sv[i4].z;
            sacc[4 * i4 + 3] = sgl * sv[i4].w;
        }
        // Scheduling boundary: the operand reads and the bias products above
        // are issued first, then the products below.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < C::QS; ++s) sacc = tgd::mfma32(ka[s], qreg[s], sacc);
        return sacc;
    };
    auto block_back = [&](int k0, int kb, const uint8_t* __restrict__ tV, f32x16 sacc) __attribute__((always_inline)) {
        const uint8_t* bV = tV + kb * 32 * C::ROW_BYTES;
        // V operands: the transposing read hands lane jj of each 16-lane group
        // four consecutive keys of one head_dim column; issued before the
        // softmax so they land while it runs.
        u32x4 va[2][C::DB];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (TG_LDS bf16x4_t*)((TG_LDS uint8_t*)bV + voff[db][half] + 16 * s * C::ROW_BYTES));
                    const u32x2 w = __builtin_bit_cast(u32x2, x);
                    va[s][db][2 * half] = w[0];
                    va[s][db][2 * half + 1] = w[1];
                }
            }
        }
        if (k0 + 31 > q0) {  // diagonal block (wave-uniform): hide keys after the query
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (k0 + 8 * (i >> 2) + 4 * g + (i & 3) > t) sacc[i] = -INFINITY;
        }
        float smax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) smax = fmaxf(smax, sacc[i]);
        const float mt = tgd::half_max(a_t * smax);
        // Raise the running max only past the slack.  A row with no visible key
        // yet keeps m = -inf (and exponent offset 0: all its p are 0).
        const bool bump = mt > m_run + kTau;
        const bool had = m_run != -INFINITY;
        const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
        if (bump) m_run = mt;
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
        float ls = 0.0f;
        u32x4 pb[2];  // P^T as bf16, by k-step
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[i], a_t, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[i + 1], a_t, -m_use));
            const uint32_t pk = tgd::cvt_pk_bf16(p0, p1);
            pb[i >> 3][(i & 7) >> 1] = pk;
            ls = add_pair(pk, ls);  // the row sum uses the same bf16 P as P.V
        }
        l_run = l_run * alpha + ls;
        if (__builtin_amdgcn_ballot_w64(bump && had)) {
#pragma unroll
            for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
        }
        // O^T += V^T . P^T, issued at raised priority
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) o[db] = tgd::mfma32(va[s][db], pb[s], o[db]);
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- this wave's slice of one super-tile: keys j0 + WKEYS*sp .. +WKEYS-1,
    // taken as KB blocks of 32 one after another.
    // `mid` issues the next super-tile's loads.  It goes out right behind the
    // first block's queued S^T products, so that a wave held up by a full
    // memory queue waits while its matrix core is busy rather than before the
    // block starts.  It has exactly one call site (a second copy of the load
    // code costs registers), reached also by a wave whose slice lies entirely
    // in its future.
    auto compute = [&](int j0, const uint8_t* __restrict__ tK, const uint8_t* __restrict__ tV,
                       const float* __restrict__ tS, auto&& mid) {
        const int k00 = j0 + rb0;
        const bool live = k00 <= wave_last;  // wave-uniform
        f32x16 sacc;
        if (live) sacc = block_front(0, tK, tS);
        __builtin_amdgcn_sched_barrier(0);
        mid();
        __builtin_amdgcn_sched_barrier(0);
        if (!live) return;
        block_back(k00, 0, tV, sacc);
#pragma unroll 1
        for (int kb = 1; kb < KB; ++kb) {  // one block at a time keeps the register footprint of one
            const int k0 = j0 + rb0 + 32 * kb;
            if (k0 > wave_last) break;  // the rest of the slice is in this wave's future
            block_back(k0, kb, tV, block_front(kb, tK, tS));
        }
    };

    // One iteration: wait for its loads; the barrier then also means every
    // wave has finished the previous iteration, which read (and merged in)
    // the other stage, so the next iteration's loads can go there; multiply.
    // Current and next stage are distinct restrict pointers of one scope, so
    // the reads of this stage never wait on the loads in flight into the other.
    auto iterate = [&](int it, uint8_t* __restrict__ cK, uint8_t* __restrict__ cV, float* __restrict__ cS,
                       uint8_t* __restrict__ nK, uint8_t* __restrict__ nV, float* __restrict__ nS) {
        const bool inA = it < nA;
        const int st = inA ? it : it - nA;
        if (st == 0) begin_block(inA ? qbA : qbB, !inA);
        TG_WAIT_VMCNT(0);
        __builtin_amdgcn_s_barrier();
        const bool more = it + 1 < ntot;
        compute(st * C::SKEYS, cK, cV, cS, [&]() __attribute__((always_inline)) {
            if (more) issue(it + 1, nK, nV, nS);
        });
        const int last = inA ? nA - 1 : ntot - nA - 1;
        if (st == last) {
            if (inA && ntot > nA) fetch_q(qbB);  // this block's rows are no longer read
            finish_block(cK, cV);  // K and V of this stage serve as merge scratch
        }
    };

    issue(0, sK0, sV0, sS0);
    for (int it = 0; it < ntot; it += 2) {
        iterate(it, sK0, sV0, sS0, sK1, sV1, sS1);
        if (it + 1 < ntot) iterate(it + 1, sK1, sV1, sS1, sK0, sV0, sS0);
    }
}

// The stream of a launch and, optionally, two events that record the
// kernel's own start and end (an extended launch; null: a plain launch).
struct Launch {
    hipStream_t s;
    hipEvent_t start, stop;
};

template <typename... A, typename... P>
void launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, const Launch& L, A... args) {
    if (L.start || L.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, L.s, L.start, L.stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, L.s, args...);
}

template <int D, int HPW, int RB, int NS, int KB>
int launch_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* ks, const float* gains,
                float c, const int32_t* pos, int64_t nk, int hq, int hkv, void* out, int out_dtype,
                float* lse, int lse_ld, const Launch& L) {
    using C = AttnCfg<D, HPW, RB, NS, KB>;
    const int nqb = (int)((nk + C::QROWS - 1) / C::QROWS);
    const int npairs = (nqb + 1) / 2;
    const int n_items = hkv * (hq / hkv / HPW) * npairs;
    const int per_xcd = (n_items + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(per_xcd * kXcds));
    if (out_dtype == 1)
        launch_kernel(gated_attn<D, HPW, RB, NS, KB, true>, grid, dim3(C::THREADS), L, q, k, v, ks, gains, c, pos,
                      (int)nk, hq, hkv, npairs, per_xcd, n_items, out, lse, lse_ld);
    else
        launch_kernel(gated_attn<D, HPW, RB, NS, KB, false>, grid, dim3(C::THREADS), L, q, k, v, ks, gains, c, pos,
                      (int)nk, hq, hkv, npairs, per_xcd, n_items, out, lse, lse_ld);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

// Work items of a launch with query blocks of 32 * rb rows and hpw heads per workgroup.
inline int64_t attn_items(int64_t nk, int hq, int hkv, int hpw, int rb) {
    const int64_t nqb = (nk + 32 * rb - 1) / (32 * rb);
    return (int64_t)hkv * (hq / hkv / hpw) * ((nqb + 1) / 2);
}

// Workgroups of eight waves (four when a kv head has a single q head):
// heads sharing K/V x query row blocks x key splits.  Take the tallest query
// blocks (most K/V reuse per byte read) that still give every CU a
// workgroup; key splits make up the rest of the waves.  Super-tiles hold at
// most 128 keys (64 KB of K and V per stage at head_dim 128).
template <int D, int HPW>
int launch_attn_h(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* ks, const float* gains,
                  float c, const int32_t* pos, int64_t nk, int hq, int hkv, void* out, int out_dtype,
                  float* lse, int lse_ld, const Launch& L) {
    constexpr int kCUs = 256;
    constexpr int W = HPW == 1 ? 4 : 8 / HPW;  // row blocks x splits
    if constexpr (W >= 4) {
        if (attn_items(nk, hq, hkv, HPW, 4) >= kCUs)
            return launch_attn<D, HPW, 4, W / 4, 2>(q, k, v, ks, gains, c, pos, nk, hq, hkv, out, out_dtype, lse, lse_ld, L);
    }
    if constexpr (W >= 2) {
        if (attn_items(nk, hq, hkv, HPW, 2) >= kCUs)
            return launch_attn<D, HPW, 2, W / 2, 2>(q, k, v, ks, gains, c, pos, nk, hq, hkv, out, out_dtype, lse, lse_ld, L);
    }
    return launch_attn<D, HPW, 1, W, (W >= 4 ? 1 : 2)>(q, k, v, ks, gains, c, pos, nk, hq, hkv, out, out_dtype, lse, lse_ld, L);
}

template <int D>
int launch_attn_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* ks, const float* gains,
                  float c, const int32_t* pos, int64_t nk, int hq, int hkv, void* out, int out_dtype,
                  float* lse, int lse_ld, const Launch& L) {
    const int G = hq / hkv;
    if (G % 4 == 0) return launch_attn_h<D, 4>(q, k, v, ks, gains, c, pos, nk, hq, hkv, out, out_dtype, lse, lse_ld, L);
    if (G % 2 == 0) return launch_attn_h<D, 2>(q, k, v, ks, gains, c, pos, nk, hq, hkv, out, out_dtype, lse, lse_ld, L);
    return launch_attn_h<D, 1>(q, k, v, ks, gains, c, pos, nk, hq, hkv, out, out_dtype, lse, lse_ld, L);
}

}  // namespace

namespace tgi {

int launch_gated_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const float* key_score, const float* gains, float temp_coef,
                           const int32_t* pos, int64_t n_kept, int hq, int hkv, int head_dim,
                           void* out, int out_dtype, float* lse, int lse_ld, void* stream, void* start_event,
                           void* stop_event) {
    const Launch L{(hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event};
    switch (head_dim) {
        case 64:
            return launch_attn_d<64>(q, k, v, key_score, gains, temp_coef, pos, n_kept, hq, hkv, out, out_dtype, lse, lse_ld, L);
        case 128:
            return launch_attn_d<128>(q, k, v, key_score, gains, temp_coef, pos, n_kept, hq, hkv, out, out_dtype, lse, lse_ld, L);
        default:
            return TG_EUNSUPPORTED;
    }
}

}  // namespace tgi
