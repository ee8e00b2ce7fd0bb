// k_select.hip -- forced-keep top-K over the normalised gate scores.
//
// The top-K selector keeps the best prunable tokens while question /
// instruction tokens are always kept (fluxbbs.com TokenGate article, section
// on where the gate sits; slinene.github.io digest, method key points;
// news.farwalk.ai, "How does TokenGate learned token pruning work?";
// aiwillknow.com, Figure 1(a)(b)).  K counts every kept token.
//
// Exact radix select on order-preserving 32-bit keys:
//   key(x) grows with x; -0.0 maps like +0.0; NaN maps to 0 (below -inf).
// Three digit rounds (11, 11 and 10 bits) find the key T of the (K-F)-th best
// prunable token and the number m of tokens equal to T that are taken (the m
// lowest-index ones).  The emit pass then writes the kept indices in
// ascending order: token i goes to slot (#forced-or-above-T before i) +
// min(#ties before i, m).  Everything is integer arithmetic, so the result is
// bit-exact and deterministic.
//
// Up to 16384 tokens one workgroup of 1024 threads does the whole selection
// (one launch, no workspace traffic); longer prompts, up to 524288 tokens,
// take the many-workgroup form further below (three launches over chunks of
// the prompt).  In the one-workgroup form each thread keeps the keys of 16
// consecutive tokens in registers after one read of the scores, so
// every later phase works on registers; the histogram copies are cleared
// while that read is in flight, the first histogram goes into eight LDS
// copies chosen by lane (float keys crowd into a few dozen top-11-bit bins,
// so lanes of one wave would otherwise collide on the same words), and the
// later rounds filter the keys by the prefix chosen so far.  Bin searches
// run in one wave with DPP scans; the emit pass takes one block scan of
// packed counts and visits only the kept tokens.  Prompts too long for the
// many-workgroup form take one workgroup that re-reads the scores
// (L2-resident) in each sweep and gathers the first round's bucket into LDS
// when it fits.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kForcedMark = 0xffffffffu;  // no score maps here (max key is +inf's)

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (f != f) return 0u;           // NaN ranks below everything
    if (u == 0x80000000u) u = 0u;    // -0.0 equals +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan over the 64 lanes of a wave with DPP lane moves (no LDS
// round trips): shifts by 1, 2, 4 and 8 inside each row of 16 lanes (lanes
// with no source add 0), then the last lane of row 0 is added to row 1 and of
// row 2 to row 3 (row_bcast:15), then the last lane of row 1 to rows 2 and 3
// (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Exclusive scan over the whole workgroup with one barrier: wave scans, wave
// totals through LDS (wsum: kWaves slots, alternated by the caller between
// consecutive scans so a slow reader of the last one is never overwritten),
// and every thread adds the totals of the waves below its own.  Returns the
// exclusive prefix; *total gets the workgroup sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(x);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t below = 0, all = 0;
#pragma unroll
    for (int w4 = 0; w4 < kWaves; w4 += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(&wsum[w4]);
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            all += vv[q];
            if (w4 + q < wave) below += vv[q];
        }
    }
    *total = all;
    return below + incl - x;
}

// Keys of tokens i .. i+3 (i a multiple of 4), straight from the scores.
__device__ __forceinline__ uint4 keys4_global(const float* __restrict__ score, const uint8_t* __restrict__ forced,
                                              uint32_t i, uint32_t n) {
    float v[4];
    uint32_t f = 0;
    if (i + 4 <= n) {
        const float4 s4 = *reinterpret_cast<const float4*>(score + i);
        v[0] = s4.x, v[1] = s4.y, v[2] = s4.z, v[3] = s4.w;
        if (forced) f = *reinterpret_cast<const uint32_t*>(forced + i);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[q] = (i + q < n) ? score[i + q] : 0.0f;
            if (forced && i + q < n && forced[i + q]) f |= 1u << (8 * q);
        }
    }
    uint4 k;
    k.x = (f & 0x000000ffu) ? kForcedMark : order_key(v[0]);
    k.y = (f & 0x0000ff00u) ? kForcedMark : order_key(v[1]);
    k.z = (f & 0x00ff0000u) ? kForcedMark : order_key(v[2]);
    k.w = (f & 0xff000000u) ? kForcedMark : order_key(v[3]);
    return k;
}

// Prompts of up to kThreads * KPT tokens: thread t holds the keys of tokens
// t*KPT .. t*KPT+KPT-1 in registers for the whole selection (one read of the
// scores), so no phase touches LDS for keys.  Same rounds and emit as the
// long-prompt kernel below.
// With SEQNORM the scores read are the scorer's raw ones: the first 256
// threads form 1 / rho from its partial sums in the fixed order every
// sequence-norm kernel uses, each thread scales its scores, writes them to
// s_norm (which may be `score` itself: a thread reads its tokens before it
// writes them) and selects on them, so the result equals the sequence norm
// followed by the plain select, bit for bit, in one launch.
template <int KPT, bool SEQNORM>
__global__ __launch_bounds__(kThreads) void select_topk_regs(const float* score,
                                                             const uint8_t* __restrict__ forced,
                                                             int64_t n64, int64_t n_forced, int64_t k64,
                                                             int32_t* __restrict__ kept,
                                                             int32_t* __restrict__ dev_status,
                                                             const float* __restrict__ block_ss, int64_t nblocks,
                                                             float eps_seq, float* s_norm) {
    static_assert(KPT % 4 == 0 && KPT <= 32, "keys per thread");
    constexpr int kBins = 2048;
    // first-round histogram in eight copies (lane % 8 picks one), so lanes of
    // a wave that hit the same bin mostly update different words (float keys
    // crowd into a few dozen top-11-bit bins); copy 0 then holds the sum, and
    // copies 1 and 2 (cleared while the copies are summed) serve the second
    // and third rounds
    constexpr int kCopies = 8;
    __shared__ __attribute__((aligned(16))) uint32_t histc[kCopies][kBins];
    __shared__ __attribute__((aligned(16))) uint32_t wsum[2][kWaves];
    __shared__ uint32_t ctl[4];

    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t n = (uint32_t)n64, k = (uint32_t)k64;
    const uint32_t base = (uint32_t)tid * KPT;
    const int nvalid = base >= n ? 0 : (int)min((uint32_t)KPT, n - base);  // this thread's tokens

    // Scores and forced flags of this thread's tokens are loaded first; the
    // histogram copies are cleared while the loads are in flight.  A thread
    // whose tokens are all in range issues its loads back to back with no
    // branch between them (one round trip); only the thread with the ragged
    // tail takes the per-token path.
    float4 sc[KPT / 4];
    uint32_t fm[KPT / 4];
    if (base + KPT <= n) {
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) sc[v] = *reinterpret_cast<const float4*>(score + base + 4 * v);
        if (forced) {
#pragma unroll
            for (int v = 0; v < KPT / 4; ++v) fm[v] = *reinterpret_cast<const uint32_t*>(forced + base + 4 * v);
        } else {
#pragma unroll
            for (int v = 0; v < KPT / 4; ++v) fm[v] = 0u;
        }
    } else {
#pragma unroll
      for (int v = 0; v < KPT / 4; ++v) {
        const uint32_t i = base + 4 * v;
        if (i + 4 <= n) {
            sc[v] = *reinterpret_cast<const float4*>(score + i);
            fm[v] = forced ? *reinterpret_cast<const uint32_t*>(forced + i) : 0u;
        } else {
            float t4[4];
            uint32_t f = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                t4[q] = (i + q < n) ? score[i + q] : 0.0f;
                if (forced && i + q < n && forced[i + q]) f |= 1u << (8 * q);
            }
            sc[v] = float4{t4[0], t4[1], t4[2], t4[3]};
            fm[v] = f;
        }
      }
    }

    auto pick_bin = [&](const uint32_t* hist, uint32_t remaining, int nbins) {
        if (threadIdx.x < 64) {
            const int per = nbins / 64;
            const int hi = nbins - lane * per;
            uint32_t sum = 0;
            for (int i = 0; i < per; i += 4) {
                const uint4 h4 = *reinterpret_cast<const uint4*>(&hist[hi - per + i]);
                sum += h4.x + h4.y + h4.z + h4.w;
            }
            const uint32_t incl = wave_incl_scan(sum);
            const int L = __builtin_ctzll(__builtin_amdgcn_ballot_w64(incl >= remaining));
            const uint32_t before = __builtin_amdgcn_readlane(incl - sum, L);
            const int hiL = nbins - L * per;
            const uint32_t c = lane < per ? hist[hiL - 1 - lane] : 0u;
            const uint32_t ci = wave_incl_scan(c) + before;
            const int b = __builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < per && ci >= remaining));
            if (lane == b) {
                ctl[0] = hiL - 1 - b;
                ctl[1] = remaining - (ci - c);
            }
        }
        __syncthreads();
    };

    if constexpr (SEQNORM) {
        __shared__ double red[tgd::kSeqSumThreads / 64];
        if (tid < tgd::kSeqSumThreads) tgd::seq_ss_partial(block_ss, nblocks, red);
        __syncthreads();
        const float inv = tgd::seq_inv_rho(red, n64, eps_seq);
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) {
            sc[v].x *= inv, sc[v].y *= inv, sc[v].z *= inv, sc[v].w *= inv;
            const uint32_t i = base + 4 * v;
            if (i + 4 <= n) {
                *reinterpret_cast<float4*>(s_norm + i) = sc[v];
            } else {
                const float t4[4] = {sc[v].x, sc[v].y, sc[v].z, sc[v].w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (i + q < n) s_norm[i + q] = t4[q];
            }
        }
    }

    // Radix pass 1: forced count and the histogram of the top 11 bits.
    for (int b = tid * 4; b < kCopies * kBins; b += kThreads * 4)
        *reinterpret_cast<uint4*>(&histc[0][0] + b) = uint4{0u, 0u, 0u, 0u};
    uint32_t key[KPT];
#pragma unroll
    for (int v = 0; v < KPT / 4; ++v) {
        const float x[4] = {sc[v].x, sc[v].y, sc[v].z, sc[v].w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            key[4 * v + q] = (fm[v] >> (8 * q)) & 0xffu ? kForcedMark : order_key(x[q]);
    }
    __syncthreads();
    uint32_t fcw = 0;  // forced tokens seen by this wave (wave-uniform)
    uint32_t* myhist = histc[lane % kCopies];
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const bool ok = e < nvalid;
        const bool f = ok && key[e] == kForcedMark;
        fcw += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(f));
        if (ok && !f) atomicAdd(&myhist[key[e] >> 21], 1u);
    }
    if (lane == 0) wsum[0][threadIdx.x >> 6] = fcw;
    __syncthreads();
    uint64_t F = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) F += wsum[0][w];
    // (each thread also clears the words of copies 1 and 2 it read: the
    // second and third rounds count into them)
    for (int b = tid * 4; b < kBins; b += kThreads * 4) {
        uint4 h = *reinterpret_cast<const uint4*>(&histc[0][b]);
#pragma unroll
        for (int c = 1; c < kCopies; ++c) {
            const uint4 x = *reinterpret_cast<const uint4*>(&histc[c][b]);
            h.x += x.x, h.y += x.y, h.z += x.z, h.w += x.w;
        }
        *reinterpret_cast<uint4*>(&histc[0][b]) = h;
        *reinterpret_cast<uint4*>(&histc[1][b]) = uint4{0u, 0u, 0u, 0u};
        *reinterpret_cast<uint4*>(&histc[2][b]) = uint4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    int64_t R = (int64_t)k - (int64_t)F;  // prunable tokens to choose
    if (tid == 0 && dev_status) {
        int32_t st = 0;
        if ((int64_t)F != n_forced) st |= TG_STATUS_FORCED_MISMATCH;
        if (R < 0) st |= TG_STATUS_FORCED_OVER_K;
        *dev_status = st;
    }
    if (R < 0) R = 0;

    uint32_t T = 0xffffffffu, m = 0;  // R == 0: no prunable token is taken
    if (R > 0) {
        pick_bin(histc[0], (uint32_t)R, kBins);
        uint32_t prefix = ctl[0] << 21, pmask = 0x7ffu << 21, remaining = ctl[1];
        __syncthreads();
        // Rounds 2 and 3: next 11 bits, then the last 10, over the keys that
        // share the prefix chosen so far.
#pragma unroll
        for (int round = 0; round < 2; ++round) {
            const int shift = round == 0 ? 10 : 0;
            const uint32_t dmask = round == 0 ? 0x7ffu : 0x3ffu;
            uint32_t* hr = histc[1 + round];  // cleared during the merge
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const uint32_t key_e = key[e];
                if (e < nvalid && key_e != kForcedMark && (key_e & pmask) == prefix)
                    atomicAdd(&hr[(key_e >> shift) & dmask], 1u);
            }
            __syncthreads();
            pick_bin(hr, remaining, (int)dmask + 1);
            prefix |= ctl[0] << shift;
            pmask |= dmask << shift;
            remaining = ctl[1];
            __syncthreads();
        }
        T = prefix;
        m = remaining;
    }

    // Emit, in index order: slot = (#kind1 before) + min(#ties before, m).
    uint32_t ka = 0, kb = 0;  // bit e: token base+e is forced or above T / equal to T
#pragma unroll
    for (int e = 0; e < KPT; ++e) {  // (no branches: compares and shifts only)
        const uint32_t ok = e < nvalid ? 1u : 0u;
        const uint32_t a = ok & ((key[e] == kForcedMark) | (key[e] > T));
        const uint32_t b = ok & (a ^ 1u) & (key[e] == T);
        ka |= a << e;
        kb |= b << e;
    }
    // both counts in one word: each is at most KPT per thread and n <= 32768
    const uint32_t ca = __builtin_popcount(ka), cb = __builtin_popcount(kb);
    uint32_t tot;
    const uint32_t ex = block_excl_scan((ca << 16) | cb, wsum[1], &tot);
    const uint32_t A = ex >> 16, B = ex & 0xffffu;
    // Only kept tokens are visited: those of kind 1 and the first m - B ties
    // of this thread (ties before it took B of the m).
    uint32_t keep = ka;
    if (B < m) {
        uint32_t ties = kb;
        if (m - B < cb) {
            uint32_t rest = kb;
            for (uint32_t r = 0; r < m - B; ++r) rest &= rest - 1;
            ties &= ~rest;
        }
        keep |= ties;
    }
    while (keep) {
        const int e = __builtin_ctz(keep);
        keep &= keep - 1;
        const uint32_t below = (1u << e) - 1u;
        const uint32_t a_before = A + __builtin_popcount(ka & below);
        const uint32_t b_before = B + __builtin_popcount(kb & below);
        const uint32_t slot = a_before + (b_before < m ? b_before : m);
        if (slot < k) kept[slot] = (int32_t)(base + e);
    }
}

// Longer prompts: the keys are re-read from the scores (L2-resident) in each
// sweep.
__global__ __launch_bounds__(kThreads) void select_topk_block(const float* __restrict__ score,
                                                              const uint8_t* __restrict__ forced,
                                                              int64_t n64, int64_t n_forced, int64_t k64,
                                                              int32_t* __restrict__ kept,
                                                              int32_t* __restrict__ dev_status) {
    constexpr int kBins = 2048;
    constexpr int kCap = 4096;  // gathered candidates
    // first-round histogram in three copies (lane % 3 picks one), so lanes of
    // a wave that hit the same bin mostly update different words; copy 0 then
    // holds the sum and serves the later rounds, and the gathered candidates
    // take the place of copies 1 and 2
    constexpr int kCopies = 3;
    static_assert((kCopies - 1) * kBins >= kCap, "candidate room");
    __shared__ __attribute__((aligned(16))) uint32_t hist4[kCopies][kBins];
    uint32_t* hist = hist4[0];
    uint32_t* cand = hist4[1];
    __shared__ __attribute__((aligned(16))) uint32_t wsum[2][kWaves];
    __shared__ uint32_t ctl[4];

    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t n = (uint32_t)n64, k = (uint32_t)k64;
    constexpr uint32_t kStep = kThreads * 16;  // tokens per sweep step: 4 groups of 4 per thread

    // Keys of 4 consecutive tokens starting at i (a multiple of 4; entries
    // past n are garbage and skipped by the callers).
    auto keys4 = [&](uint32_t i) -> uint4 { return keys4_global(score, forced, i, n); };
    // Sweep every token; f(i, key) for each i < n.
    auto sweep = [&](auto&& f) {
        for (uint32_t c0 = 0; c0 < n; c0 += kStep) {
            uint4 kv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) kv[e] = keys4(c0 + (e * kThreads + tid) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t i = c0 + (e * kThreads + tid) * 4;
                const uint32_t kk[4] = {kv[e].x, kv[e].y, kv[e].z, kv[e].w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (i + q < n) f(i + q, kk[q]);
            }
        }
    };
    // Find the bin holding the remaining-th largest key of the histogram
    // (bins scanned from the top); sets ctl[0] = bin, ctl[1] = rank inside it.
    // One wave does it with two wave scans (no workgroup barrier inside):
    // lane l sums the l-th chunk of nbins/64 bins counted from the top; the
    // lane whose running count reaches `remaining` owns the bin, which its
    // chunk's bins then locate with a second scan.
    auto pick_bin = [&](uint32_t remaining, int nbins) {
        if (threadIdx.x < 64) {
            const int per = nbins / 64;
            const int hi = nbins - lane * per;
            uint32_t sum = 0;
            for (int i = 0; i < per; i += 4) {
                const uint4 h4 = *reinterpret_cast<const uint4*>(&hist[hi - per + i]);
                sum += h4.x + h4.y + h4.z + h4.w;
            }
            const uint32_t incl = wave_incl_scan(sum);
            const int L = __builtin_ctzll(__builtin_amdgcn_ballot_w64(incl >= remaining));
            const uint32_t before = __builtin_amdgcn_readlane(incl - sum, L);
            const int hiL = nbins - L * per;
            const uint32_t c = lane < per ? hist[hiL - 1 - lane] : 0u;
            const uint32_t ci = wave_incl_scan(c) + before;
            const int b = __builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < per && ci >= remaining));
            if (lane == b) {
                ctl[0] = hiL - 1 - b;
                ctl[1] = remaining - (ci - c);
            }
        }
        __syncthreads();
    };
    auto clear_hist = [&]() {
        for (int b = tid; b < kBins; b += kThreads) hist[b] = 0;
    };

    // Sweep 1: keys to LDS, forced count, histogram of the top 11 bits.
    for (int b = tid * 4; b < kCopies * kBins; b += kThreads * 4)
        *reinterpret_cast<uint4*>(&hist4[0][0] + b) = uint4{0u, 0u, 0u, 0u};
    __syncthreads();
    uint32_t fcw = 0;  // forced tokens seen by this wave (wave-uniform)
    uint32_t* myhist = hist4[lane % kCopies];
    for (uint32_t c0 = 0; c0 < n; c0 += kStep) {
        uint4 kv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[e] = keys4_global(score, forced, c0 + (e * kThreads + tid) * 4, n);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t i = c0 + (e * kThreads + tid) * 4;
            const uint32_t kk[4] = {kv[e].x, kv[e].y, kv[e].z, kv[e].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool ok = i + q < n;
                const bool f = ok && kk[q] == kForcedMark;
                fcw += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(f));
                if (ok && !f) atomicAdd(&myhist[kk[q] >> 21], 1u);
            }
        }
    }
    if (lane == 0) wsum[0][threadIdx.x >> 6] = fcw;
    __syncthreads();
    uint64_t F = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) F += wsum[0][w];
    // merge the histogram copies into copy 0
    for (int b = tid * 4; b < kBins; b += kThreads * 4) {
        uint4 h = *reinterpret_cast<const uint4*>(&hist4[0][b]);
#pragma unroll
        for (int c = 1; c < kCopies; ++c) {
            const uint4 x = *reinterpret_cast<const uint4*>(&hist4[c][b]);
            h.x += x.x, h.y += x.y, h.z += x.z, h.w += x.w;
        }
        *reinterpret_cast<uint4*>(&hist4[0][b]) = h;
    }
    __syncthreads();
    int64_t R = (int64_t)k - (int64_t)F;  // prunable tokens to choose
    if (tid == 0 && dev_status) {
        int32_t st = 0;
        if ((int64_t)F != n_forced) st |= TG_STATUS_FORCED_MISMATCH;
        if (R < 0) st |= TG_STATUS_FORCED_OVER_K;
        *dev_status = st;
    }
    if (R < 0) R = 0;

    uint32_t T = 0xffffffffu, m = 0;  // R == 0: no prunable token is taken
    if (R > 0) {
        // Radix pass 1: top 11 bits.
        pick_bin((uint32_t)R, kBins);
        uint32_t prefix = ctl[0] << 21, pmask = 0x7ffu << 21, remaining = ctl[1];
        const uint32_t bucket = hist[ctl[0]];
        __syncthreads();

        // Gather the bucket's keys when they fit (the later rounds then read
        // only them); buckets too large to gather (e.g. all scores equal) take
        // a prefix-filtered sweep of all keys instead.
        const bool gathered = bucket <= (uint32_t)kCap;
        if (gathered) {
            // each wave reserves room for its matches with one LDS atomic per
            // four keys a lane; a lane's slots follow from ballots of the
            // matches (all lanes below it, then its own lower keys)
            if (tid == 0) ctl[2] = 0;
            __syncthreads();
            for (uint32_t c0 = 0; c0 < n; c0 += kStep) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t i = c0 + (e * kThreads + tid) * 4;
                    const uint4 kv = keys4(i);
                    const uint32_t kq[4] = {kv.x, kv.y, kv.z, kv.w};
                    bool hit[4];
                    uint64_t bq[4];
                    uint32_t wtot = 0, pre = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        hit[q] = i + q < n && kq[q] != kForcedMark && (kq[q] & pmask) == prefix;
                        bq[q] = __builtin_amdgcn_ballot_w64(hit[q]);
                        wtot += (uint32_t)__builtin_popcountll(bq[q]);
                        pre += lanes_below(bq[q]);
                    }
                    if (wtot == 0) continue;  // wave-uniform
                    uint32_t base = 0;
                    if (lane == 0) base = atomicAdd(&ctl[2], wtot);
                    base = __builtin_amdgcn_readlane(base, 0) + pre;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (hit[q]) cand[base++] = kq[q];
                }
            }
            __syncthreads();
        }
        // Rounds 2 and 3: next 11 bits, then the last 10.
#pragma unroll
        for (int round = 0; round < 2; ++round) {
            const int shift = round == 0 ? 10 : 0;
            const uint32_t dmask = round == 0 ? 0x7ffu : 0x3ffu;
            clear_hist();
            __syncthreads();
            if (gathered) {
                for (uint32_t c = tid; c < bucket; c += kThreads) {
                    const uint32_t key = cand[c];
                    if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
                }
            } else {
                sweep([&](uint32_t, uint32_t key) {
                    if (key != kForcedMark && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
                });
            }
            __syncthreads();
            pick_bin(remaining, (int)dmask + 1);
            prefix |= ctl[0] << shift;
            pmask |= dmask << shift;
            remaining = ctl[1];
            __syncthreads();
        }
        T = prefix;
        m = remaining;
    }

    // Emit, in index order: slot = (#kind1 before) + min(#ties before, m).
    // Sixteen consecutive tokens per thread, so up to 16384 tokens take one
    // pass (one workgroup scan).
    uint64_t carryA = 0, carryB = 0;
    int pass = 0;
    for (uint32_t c0 = 0; c0 < n; c0 += kThreads * 16, ++pass) {
        const uint32_t base = c0 + (uint32_t)tid * 16;
        uint32_t ka = 0, kb = 0;  // bit e: token base+e is forced or above T / equal to T
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const uint4 kv = keys4(base + 4 * v4);
            const uint32_t kq[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = 4 * v4 + q;
                if (base + e < n) {
                    const uint32_t key = kq[q];
                    if (key == kForcedMark || key > T) ka |= 1u << e;
                    else if (key == T) kb |= 1u << e;
                }
            }
        }
        // both counts in one word: each is at most 16 per thread and 16384
        // per pass
        const uint32_t ca = __builtin_popcount(ka), cb = __builtin_popcount(kb);
        uint32_t tot;
        const uint32_t ex = block_excl_scan((ca << 16) | cb, wsum[pass & 1], &tot);
        const uint64_t A = carryA + (ex >> 16), B = carryB + (ex & 0xffffu);
        // Only kept tokens are visited: those of kind 1 and the first m - B
        // ties of this thread (ties before it took B of the m).  Token e's
        // slot is (#kind 1 before it) + min(#ties before it, m).
        uint32_t keep = ka;
        if (B < m) {
            uint32_t ties = kb;
            if (m - B < (uint64_t)cb) {
                // only the first m - B of them fit: clear the rest
                uint32_t rest = kb;
                for (uint32_t r = 0; r < (uint32_t)(m - B); ++r) rest &= rest - 1;
                ties &= ~rest;
            }
            keep |= ties;
        }
        while (keep) {
            const int e = __builtin_ctz(keep);
            keep &= keep - 1;
            const uint32_t below = (1u << e) - 1u;
            const uint64_t a_before = A + __builtin_popcount(ka & below);
            const uint64_t b_before = B + __builtin_popcount(kb & below);
            const uint64_t slot = a_before + (b_before < m ? b_before : m);
            if (slot < k) kept[slot] = (int32_t)(base + e);
        }
        carryA += tot >> 16;
        carryB += tot & 0xffffu;
    }
}

// ---------------------------------------------------------------------------
// Many-workgroup select for long prompts.  The prompt is cut into chunks of
// 256 * KPT consecutive tokens, one workgroup of 256 threads each (a thread
// holds KPT consecutive keys in registers), and the selection takes three
// launches over the same grid:
//   selm_hist    each chunk's histogram of the keys' top 11 bits (u16) and
//                its forced count;
//   selm_gather  every workgroup adds up all chunks' counts of 64 groups of
//                32 bins, picks the group, adds up all chunks' counts of that
//                group's bins and picks the first round's bin b1 (the same
//                sums and picks in every workgroup); it counts its chunk's
//                prunable keys above b1 and stores its keys in b1 (the
//                candidates) after those of the chunks before it, in index
//                order;
//   selm_emit    every workgroup reads all candidates (into LDS when they
//                fit) and runs rounds 2 and 3 over them (identically), which
//                fixes T and m, adds up the counts of the chunks before its
//                own and writes its chunk's kept indices.
// Integer arithmetic and no global atomics: bit-exact and deterministic, and
// no workspace word needs clearing (every one is written before it is read).

constexpr int kMT = tgi::kSelectThreads;
constexpr int kMWaves = kMT / 64;

// Exclusive scan over a 256-thread workgroup (one barrier); wsum has kMWaves
// slots, alternated by the caller between consecutive scans.
__device__ __forceinline__ uint32_t block_excl_scan_m(uint32_t x, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(x);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t below = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kMWaves; ++w) {
        const uint32_t v = wsum[w];
        all += v;
        if (w < wave) below += v;
    }
    *total = all;
    return below + incl - x;
}

// Keys of this thread's KPT consecutive tokens base .. base + KPT - 1
// (kForcedMark for forced tokens; entries at or past n are unused).
// A thread whose tokens are all in range issues its loads back to back with no
// branch between them (one round trip); the ragged tail takes keys4_global.
template <int KPT>
__device__ __forceinline__ void chunk_keys(const float* __restrict__ score, const uint8_t* __restrict__ forced,
                                           uint32_t base, uint32_t n, uint32_t (&key)[KPT]) {
    if (base + KPT <= n) {
        float4 s4[KPT / 4];
        uint32_t f[KPT / 4];
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) s4[v] = *reinterpret_cast<const float4*>(score + base + 4 * v);
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) f[v] = forced ? *reinterpret_cast<const uint32_t*>(forced + base + 4 * v) : 0u;
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) {
            key[4 * v] = (f[v] & 0x000000ffu) ? kForcedMark : order_key(s4[v].x);
            key[4 * v + 1] = (f[v] & 0x0000ff00u) ? kForcedMark : order_key(s4[v].y);
            key[4 * v + 2] = (f[v] & 0x00ff0000u) ? kForcedMark : order_key(s4[v].z);
            key[4 * v + 3] = (f[v] & 0xff000000u) ? kForcedMark : order_key(s4[v].w);
        }
    } else {
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) {
            const uint4 k4 = keys4_global(score, forced, base + 4 * v, n);
            key[4 * v] = k4.x, key[4 * v + 1] = k4.y, key[4 * v + 2] = k4.z, key[4 * v + 3] = k4.w;
        }
    }
}

// Scores and forced-flag words of this thread's KPT consecutive tokens, for
// the fused sequence norm (the keys are formed after the scaling); entries
// at or past n read as 0.  Same load pattern as chunk_keys.
template <int KPT>
__device__ __forceinline__ void chunk_vals(const float* score, const uint8_t* __restrict__ forced, uint32_t base,
                                           uint32_t n, float4 (&sc)[KPT / 4], uint32_t (&fm)[KPT / 4]) {
    if (base + KPT <= n) {
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) sc[v] = *reinterpret_cast<const float4*>(score + base + 4 * v);
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) fm[v] = forced ? *reinterpret_cast<const uint32_t*>(forced + base + 4 * v) : 0u;
    } else {
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) {
            float t4[4];
            uint32_t f = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t i = base + 4 * v + q;
                t4[q] = i < n ? score[i] : 0.0f;
                if (forced && i < n && forced[i]) f |= 1u << (8 * q);
            }
            sc[v] = float4{t4[0], t4[1], t4[2], t4[3]};
            fm[v] = f;
        }
    }
}

// The bin of `hist` (nbins, counted from the top) holding the remaining-th
// largest key; one wave, two wave scans.  Sets ctl[0] = bin, ctl[1] = rank
// inside it; ends with a barrier.
__device__ __forceinline__ void pick_bin_m(const uint32_t* hist, uint32_t remaining, int nbins, uint32_t* ctl) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int per = nbins / 64;
        const int hi = nbins - lane * per;
        uint32_t sum = 0;
        for (int i = 0; i < per; i += 4) {
            const uint4 h4 = *reinterpret_cast<const uint4*>(&hist[hi - per + i]);
            sum += h4.x + h4.y + h4.z + h4.w;
        }
        const uint32_t incl = wave_incl_scan(sum);
        const int L = __builtin_ctzll(__builtin_amdgcn_ballot_w64(incl >= remaining));
        const uint32_t before = __builtin_amdgcn_readlane(incl - sum, L);
        const int hiL = nbins - L * per;
        const uint32_t c = lane < per ? hist[hiL - 1 - lane] : 0u;
        const uint32_t ci = wave_incl_scan(c) + before;
        const int b = __builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < per && ci >= remaining));
        if (lane == b) {
            ctl[0] = hiL - 1 - b;
            ctl[1] = remaining - (ci - c);
        }
    }
    __syncthreads();
}

// Sum over the 64 lanes of a wave, valid in lane 63 (the last lane of an
// inclusive DPP scan: no LDS round trips).
__device__ __forceinline__ uint32_t wave_sum_last(uint32_t x) { return wave_incl_scan(x); }

// hist[bin] += 1 for every active lane; when all active lanes of the wave
// share one bin (ties, or scores that crowd into one bin) a single lane adds
// their count.
__device__ __forceinline__ void hist_add_wave(uint32_t* hist, uint32_t bin, bool active) {
    const uint64_t act = __builtin_amdgcn_ballot_w64(active);
    if (act == 0) return;  // wave-uniform
    const int first = __builtin_ctzll(act);
    const uint32_t b0 = __builtin_amdgcn_readlane(bin, first);
    if (__builtin_amdgcn_ballot_w64(active && bin == b0) == act) {
        if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[b0], (uint32_t)__builtin_popcountll(act));
    } else if (active) {
        atomicAdd(&hist[bin], 1u);
    }
}

// With SEQNORM the scores read are the scorer's raw ones: every workgroup
// forms 1 / rho from all the partial sums in the fixed order of every
// sequence-norm kernel (so all get the same value), scales its chunk's scores,
// writes them to s_norm (which may be `score` itself: a thread reads its
// tokens before it writes them, and no other workgroup reads them in this
// launch) and histograms their keys.  The two later launches read s_norm, so
// the result equals the sequence norm followed by the plain select, bit for
// bit, with one launch fewer.
template <int KPT, bool SEQNORM>
__global__ __launch_bounds__(kMT) void selm_hist(const float* score, const uint8_t* __restrict__ forced,
                                                 uint32_t n, tgi::SelectWs w, const float* __restrict__ block_ss,
                                                 int64_t nblocks, float eps_seq, float* s_norm) {
    constexpr int kCopies = 4;  // lane % 4 picks a copy: fewer lanes of a wave on one word
    __shared__ __attribute__((aligned(16))) uint32_t h[kCopies][2048];
    __shared__ uint32_t fw[kMWaves];
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t c = blockIdx.x;
    const uint32_t base = c * (uint32_t)(kMT * KPT) + (uint32_t)tid * KPT;
    uint32_t key[KPT];
    if constexpr (SEQNORM) {
        static_assert(kMT == tgd::kSeqSumThreads, "every thread adds partials");
        __shared__ double red[tgd::kSeqSumThreads / 64];
        float4 sc[KPT / 4];
        uint32_t fm[KPT / 4];
        chunk_vals<KPT>(score, forced, base, n, sc, fm);
#pragma unroll
        for (int i = 0; i < kCopies * 2048 / (4 * kMT); ++i)
            *reinterpret_cast<uint4*>(&h[0][0] + 4 * (i * kMT + tid)) = uint4{0u, 0u, 0u, 0u};
        tgd::seq_ss_partial(block_ss, nblocks, red);
        __syncthreads();
        const float inv = tgd::seq_inv_rho(red, (int64_t)n, eps_seq);
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) sc[v].x *= inv, sc[v].y *= inv, sc[v].z *= inv, sc[v].w *= inv;
        if (base + KPT <= n) {
#pragma unroll
            for (int v = 0; v < KPT / 4; ++v) *reinterpret_cast<float4*>(s_norm + base + 4 * v) = sc[v];
        } else {
#pragma unroll
            for (int v = 0; v < KPT / 4; ++v) {
                const float t4[4] = {sc[v].x, sc[v].y, sc[v].z, sc[v].w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (base + 4 * v + q < n) s_norm[base + 4 * v + q] = t4[q];
            }
        }
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) {
            const float x[4] = {sc[v].x, sc[v].y, sc[v].z, sc[v].w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                key[4 * v + q] = (fm[v] >> (8 * q)) & 0xffu ? kForcedMark : order_key(x[q]);
        }
    } else {
        chunk_keys<KPT>(score, forced, base, n, key);  // loads in flight while the copies are cleared
#pragma unroll
        for (int i = 0; i < kCopies * 2048 / (4 * kMT); ++i)
            *reinterpret_cast<uint4*>(&h[0][0] + 4 * (i * kMT + tid)) = uint4{0u, 0u, 0u, 0u};
        __syncthreads();
    }
    const int nvalid = base >= n ? 0 : (int)min((uint32_t)KPT, n - base);
    uint32_t fcount = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const bool ok = e < nvalid;
        const bool f = ok && key[e] == kForcedMark;
        fcount += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(f));
        if (ok && !f) atomicAdd(&h[lane % kCopies][key[e] >> 21], 1u);
    }
    if (lane == 0) fw[tid >> 6] = fcount;
    __syncthreads();
    // thread t merges bins 8t .. 8t+7 and stores them as u16 (a chunk holds
    // at most 8192 keys); the four threads of a group of 32 bins add their
    // sums into that group's coarse count
    uint32_t sum[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sum[j] = 0;
#pragma unroll
    for (int cp = 0; cp < kCopies; ++cp) {
        const uint4 a = *reinterpret_cast<const uint4*>(&h[cp][8 * tid]);
        const uint4 b = *reinterpret_cast<const uint4*>(&h[cp][8 * tid + 4]);
        sum[0] += a.x, sum[1] += a.y, sum[2] += a.z, sum[3] += a.w;
        sum[4] += b.x, sum[5] += b.y, sum[6] += b.z, sum[7] += b.w;
    }
    *reinterpret_cast<uint4*>(w.hist + (size_t)c * 2048 + 8 * tid) =
        uint4{sum[0] | (sum[1] << 16), sum[2] | (sum[3] << 16), sum[4] | (sum[5] << 16), sum[6] | (sum[7] << 16)};
    uint32_t g = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) g += sum[j];
    g += __shfl_xor(g, 1, 64);
    g += __shfl_xor(g, 2, 64);
    if ((tid & 3) == 0) w.coarse[(size_t)c * 64 + (tid >> 2)] = (uint16_t)g;
    if (tid == 0) {
        uint32_t f = 0;
#pragma unroll
        for (int i = 0; i < kMWaves; ++i) f += fw[i];
        w.forced[c] = f;
    }
}

// The bin holding the remaining-th largest count of a histogram of 64 bins
// (one per lane of wave 0, lane l holding bin 63 - l, i.e. from the top):
// returns (bin, rank inside it) to every lane of the wave.
__device__ __forceinline__ void pick64(uint32_t cnt_from_top, uint32_t remaining, uint32_t* bin, uint32_t* rank) {
    const uint32_t incl = wave_incl_scan(cnt_from_top);
    const int L = __builtin_ctzll(__builtin_amdgcn_ballot_w64(incl >= remaining));
    *bin = 63u - (uint32_t)L;
    *rank = remaining - __builtin_amdgcn_readlane(incl - cnt_from_top, L);
}

template <int KPT>
__global__ __launch_bounds__(kMT) void selm_gather(const float* __restrict__ score,
                                                   const uint8_t* __restrict__ forced, uint32_t n, uint32_t chunks,
                                                   uint32_t k, int64_t n_forced, int32_t* __restrict__ dev_status,
                                                   tgi::SelectWs w) {
    __shared__ uint32_t coarse[64], fine[32], ctl[8], fsum;
    __shared__ uint32_t fall[tgi::kSelectMaxChunks][32];  // every chunk's counts in the chosen group of 32 bins
    __shared__ uint32_t wsum[2][kMWaves];
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t c = blockIdx.x;
    const uint32_t base = c * (uint32_t)(kMT * KPT) + (uint32_t)tid * KPT;
    uint32_t key[KPT];
    chunk_keys<KPT>(score, forced, base, n, key);
    // Every chunk's coarse counts added up without atomics: lane l of each
    // wave reads chunk l's counts of 16 groups (two 16-byte loads), and each
    // group's sum over the 64 lanes is a wave reduction; wave v covers
    // groups 16v .. 16v+15.  Wave 0 also adds up the forced counts.
    const int wave = tid >> 6;
    {
        const bool ok = (uint32_t)lane < chunks;
        const uint16_t* row = w.coarse + (size_t)lane * 64 + 16 * wave;
        const uint4 v0 = ok ? *reinterpret_cast<const uint4*>(row) : uint4{0u, 0u, 0u, 0u};
        const uint4 v1 = ok ? *reinterpret_cast<const uint4*>(row + 8) : uint4{0u, 0u, 0u, 0u};
        const uint32_t f = (wave == 0 && ok) ? w.forced[lane] : 0u;
        const uint32_t vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t t = wave_sum_last((vv[j >> 1] >> (16 * (j & 1))) & 0xffffu);
            if (lane == 63) coarse[16 * wave + j] = t;
        }
        const uint32_t ft = wave_sum_last(f);
        if (wave == 0 && lane == 63) fsum = ft;
    }
    __syncthreads();
    const uint32_t F = fsum;
    int64_t R = (int64_t)k - (int64_t)F;  // prunable tokens to choose
    if (c == 0 && tid == 0 && dev_status) {
        int32_t st = 0;
        if ((int64_t)F != n_forced) st |= TG_STATUS_FORCED_MISMATCH;
        if (R < 0) st |= TG_STATUS_FORCED_OVER_K;
        *dev_status = st;
    }
    if (R < 0) R = 0;
    uint32_t b1 = 0, r1 = 0, start = 0, total = 0;
    if (R > 0) {
        // the group of 32 bins, then the bin inside it: only that group's
        // counts of every chunk are read (and kept, per chunk)
        if (tid < 64) {
            uint32_t grp, rank;
            pick64(coarse[63 - lane], (uint32_t)R, &grp, &rank);
            if (lane == 0) ctl[0] = grp, ctl[1] = rank;
        }
        __syncthreads();
        const uint32_t grp = ctl[0], rank = ctl[1];
        {
            // lane l: chunk l's bins 8v .. 8v+7 of the group (wave v)
            const bool ok = (uint32_t)lane < chunks;
            const uint4 v = ok ? *reinterpret_cast<const uint4*>(w.hist + (size_t)lane * 2048 + 32 * grp + 8 * wave)
                               : uint4{0u, 0u, 0u, 0u};
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t x = (vv[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                fall[lane][8 * wave + j] = x;
                const uint32_t t = wave_sum_last(x);
                if (lane == 63) fine[8 * wave + j] = t;
            }
        }
        __syncthreads();
        if (tid < 64) {
            uint32_t bin, rk;  // lanes 0..31 hold bins 31..0 of the group; the rest hold 0
            pick64(lane < 32 ? fine[31 - lane] : 0u, rank, &bin, &rk);
            const uint32_t jb = bin - 32;  // bin inside the group
            // the chunks' counts in that bin: where this chunk's candidates start
            const uint32_t cnt = (uint32_t)lane < chunks ? fall[lane][jb] : 0u;
            const uint32_t incl = wave_incl_scan(cnt);
            const uint32_t st_c = __builtin_amdgcn_readlane(incl - cnt, (int)c);
            if (lane == 63) ctl[2] = 32 * grp + jb, ctl[3] = rk, ctl[4] = st_c, ctl[5] = incl;
        }
        __syncthreads();
        b1 = ctl[2], r1 = ctl[3], start = ctl[4], total = ctl[5];
    }
    // this chunk: prunable keys above bin b1, and its keys in b1 (stored in
    // index order after a scan of the per-thread counts)
    const int nvalid = base >= n ? 0 : (int)min((uint32_t)KPT, n - base);
    uint32_t na = 0, nb = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const bool p = R > 0 && e < nvalid && key[e] != kForcedMark;
        na += (p && (key[e] >> 21) > b1) ? 1u : 0u;
        nb += (p && (key[e] >> 21) == b1) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan_m((na << 16) | nb, wsum[0], &tot);
    uint32_t* out = w.cand + start + (ex & 0xffffu);
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        if (R > 0 && e < nvalid && key[e] != kForcedMark && (key[e] >> 21) == b1) *out++ = key[e];
    }
    if (tid == 0) {
        w.above[c] = tot >> 16;
        w.cstart[c] = start;
        if (c == 0) {
            w.ctl[0] = b1;
            w.ctl[1] = r1;
            w.ctl[2] = F;
            w.ctl[3] = (uint32_t)R;
            w.ctl[4] = total;
        }
    }
}

template <int KPT>
__global__ __launch_bounds__(kMT) void selm_emit(const float* __restrict__ score, const uint8_t* __restrict__ forced,
                                                 uint32_t n, uint32_t chunks, uint32_t k,
                                                 int32_t* __restrict__ kept, tgi::SelectWs w) {
    constexpr uint32_t CH = kMT * KPT;
    constexpr uint32_t kCache = 16384;  // candidates held in LDS when they fit
    __shared__ __attribute__((aligned(16))) uint32_t hist[2048];
    __shared__ __attribute__((aligned(16))) uint32_t cache[kCache];
    __shared__ uint32_t ctl[4];
    __shared__ uint32_t wsum[2][kMWaves];
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t c = blockIdx.x;
    const uint32_t base = c * CH + (uint32_t)tid * KPT;
    uint32_t key[KPT];
    chunk_keys<KPT>(score, forced, base, n, key);
    // The first kSpec candidate words are read before their count is known
    // (the array holds at least n words; words past the count are never used).
    constexpr uint32_t kSpec = 4 * 4 * kMT;
    uint4 spec[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t i = 4 * (u * kMT + (uint32_t)tid);
        spec[u] = i + 4 <= n ? *reinterpret_cast<const uint4*>(w.cand + i) : uint4{0u, 0u, 0u, 0u};
    }
    const uint32_t b1 = w.ctl[0], r1 = w.ctl[1], R = w.ctl[3], C = w.ctl[4];
    const uint32_t c_end = w.cstart[c];  // candidates of the chunks before this one: [0, c_end)
    const bool cached = C <= kCache;
    if (R > 0 && cached) {
        // all candidates into LDS: the speculative words, then the rest 16
        // bytes a thread per trip (the array is 256-byte aligned; the last
        // piece is read word by word)
#pragma unroll
        for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(&cache[4 * (u * kMT + tid)]) = spec[u];
        const uint32_t full = C / 4;
        for (uint32_t i = kSpec / 4 + tid; i < full; i += kMT)
            *reinterpret_cast<uint4*>(&cache[4 * i]) = *reinterpret_cast<const uint4*>(w.cand + 4 * i);
        if ((uint32_t)tid < C - 4 * full) cache[4 * full + tid] = w.cand[4 * full + tid];
    }
    // the forced and above-b1 counts of the chunks before this one (wave 0)
    uint32_t fa_before = 0;
    if (tid < 64) {
        const uint32_t fa = (uint32_t)lane < c ? w.forced[lane] + w.above[lane] : 0u;
        fa_before = __builtin_amdgcn_readlane(wave_incl_scan(fa), 63);
    }

    uint32_t T = 0xffffffffu, m = 0;  // R == 0: no prunable token is taken
    if (R > 0) {
        // Rounds 2 and 3 (next 11 bits, last 10) over all candidates.
        uint32_t prefix = b1 << 21, pmask = 0x7ffu << 21, remaining = r1;
#pragma unroll
        for (int round = 0; round < 2; ++round) {
            const int shift = round == 0 ? 10 : 0;
            const uint32_t dmask = round == 0 ? 0x7ffu : 0x3ffu;
            for (int b = tid; b < 2048; b += kMT) hist[b] = 0;
            __syncthreads();  // (also: the candidates are in LDS)
            if (cached) {
                // four keys a thread per trip (one 16-byte LDS read)
                for (uint32_t f0 = 0; f0 < C; f0 += 4 * kMT) {  // whole-workgroup trips
                    const uint32_t f = f0 + 4 * (uint32_t)tid;
                    const uint4 k4 = f < C ? *reinterpret_cast<const uint4*>(&cache[f]) : uint4{0u, 0u, 0u, 0u};
                    const uint32_t kq[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        hist_add_wave(hist, (kq[q] >> shift) & dmask, f + q < C && (kq[q] & pmask) == prefix);
                }
            } else {
                for (uint32_t f0 = 0; f0 < C; f0 += kMT) {  // whole-workgroup trips
                    const uint32_t f = f0 + (uint32_t)tid;
                    const uint32_t key_f = f < C ? w.cand[f] : 0u;
                    hist_add_wave(hist, (key_f >> shift) & dmask, f < C && (key_f & pmask) == prefix);
                }
            }
            __syncthreads();
            pick_bin_m(hist, remaining, (int)dmask + 1, ctl);
            prefix |= ctl[0] << shift;
            pmask |= dmask << shift;
            remaining = ctl[1];
            __syncthreads();
        }
        T = prefix;
        m = remaining;
    }

    // Kept tokens and ties in the chunks before this one: forced and above
    // b1 from the counts, above and equal to T from their candidates.
    uint32_t a_pre = tid == 0 ? fa_before : 0u, b_pre = 0;  // (wave 0 holds fa_before in every lane)
    if (cached) {
        for (uint32_t f = 4 * (uint32_t)tid; f < c_end; f += 4 * kMT) {
            const uint4 k4 = *reinterpret_cast<const uint4*>(&cache[f]);
            const uint32_t kq[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a_pre += (f + q < c_end && kq[q] > T) ? 1u : 0u;
                b_pre += (f + q < c_end && kq[q] == T) ? 1u : 0u;
            }
        }
    } else {
        for (uint32_t f = tid; f < c_end; f += kMT) {
            const uint32_t key_f = w.cand[f];
            a_pre += key_f > T ? 1u : 0u;
            b_pre += key_f == T ? 1u : 0u;
        }
    }
    // workgroup totals (two scans: each total may exceed 16 bits)
    uint32_t A0, B0;
    block_excl_scan_m(a_pre, wsum[0], &A0);
    block_excl_scan_m(b_pre, wsum[1], &B0);

    // Emit this chunk in index order: slot = (#kind 1 before) + min(#ties before, m).
    const int nvalid = base >= n ? 0 : (int)min((uint32_t)KPT, n - base);
    uint32_t ka = 0, kb = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const uint32_t ok = e < nvalid ? 1u : 0u;
        const uint32_t a = ok & ((key[e] == kForcedMark) | (key[e] > T));
        const uint32_t b = ok & (a ^ 1u) & (key[e] == T);
        ka |= a << e;
        kb |= b << e;
    }
    const uint32_t ca = __builtin_popcount(ka), cb = __builtin_popcount(kb);
    uint32_t tot;
    // both counts in one word: each is at most KPT per thread and CH <= 8192 per chunk
    const uint32_t ex = block_excl_scan_m((ca << 16) | cb, wsum[0], &tot);
    const uint64_t A = (uint64_t)A0 + (ex >> 16), B = (uint64_t)B0 + (ex & 0xffffu);
    uint32_t keep = ka;
    if (B < m) {
        uint32_t ties = kb;
        if (m - B < (uint64_t)cb) {
            uint32_t rest = kb;
            for (uint32_t r = 0; r < (uint32_t)(m - B); ++r) rest &= rest - 1;
            ties &= ~rest;
        }
        keep |= ties;
    }
    while (keep) {
        const int e = __builtin_ctz(keep);
        keep &= keep - 1;
        const uint32_t below = (1u << e) - 1u;
        const uint64_t a_before = A + __builtin_popcount(ka & below);
        const uint64_t b_before = B + __builtin_popcount(kb & below);
        const uint64_t slot = a_before + (b_before < m ? b_before : m);
        if (slot < k) kept[slot] = (int32_t)(base + e);
    }
}

// With block_ss set, `score` holds the raw scores and the first launch forms
// the normalised ones into s_norm, which the other two read.
template <int KPT>
int launch_select_multi(const float* score, const uint8_t* forced, int64_t n, int64_t n_forced, int64_t k,
                        int32_t* kept_idx, int32_t* dev_status, const tgi::SelectWs& w, hipStream_t s,
                        const float* block_ss = nullptr, float eps_seq = 0.0f, float* s_norm = nullptr) {
    const uint32_t chunks = (uint32_t)tgi::select_chunks(n);
    if (block_ss) {
        hipLaunchKernelGGL((selm_hist<KPT, true>), dim3(chunks), dim3(kMT), 0, s, score, forced, (uint32_t)n, w,
                           block_ss, tgi::gate_partials(n), eps_seq, s_norm);
        score = s_norm;
    } else {
        hipLaunchKernelGGL((selm_hist<KPT, false>), dim3(chunks), dim3(kMT), 0, s, score, forced, (uint32_t)n, w,
                           nullptr, (int64_t)0, 0.0f, nullptr);
    }
    hipLaunchKernelGGL(selm_gather<KPT>, dim3(chunks), dim3(kMT), 0, s, score, forced, (uint32_t)n, chunks,
                       (uint32_t)k, n_forced, dev_status, w);
    hipLaunchKernelGGL(selm_emit<KPT>, dim3(chunks), dim3(kMT), 0, s, score, forced, (uint32_t)n, chunks,
                       (uint32_t)k, kept_idx, w);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace

namespace tgi {

int launch_select_topk(const float* score, const uint8_t* forced, int64_t n, int64_t n_forced,
                       int64_t k, int32_t* kept_idx, int32_t* dev_status, void* ws, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const int kpt = select_kpt(n);
    if (kpt > 0) {
        const SelectWs w = select_ws(static_cast<char*>(ws) + gate_bytes(n), n);
        switch (kpt) {
            case 8: return launch_select_multi<8>(score, forced, n, n_forced, k, kept_idx, dev_status, w, s);
            case 16: return launch_select_multi<16>(score, forced, n, n_forced, k, kept_idx, dev_status, w, s);
            default: return launch_select_multi<32>(score, forced, n, n_forced, k, kept_idx, dev_status, w, s);
        }
    }
    if (n <= kThreads * 16)
        hipLaunchKernelGGL((select_topk_regs<16, false>), dim3(1), dim3(kThreads), 0, s, score, forced, n, n_forced,
                           k, kept_idx, dev_status, nullptr, 0, 0.0f, nullptr);
    else
        hipLaunchKernelGGL(select_topk_block, dim3(1), dim3(kThreads), 0, s, score, forced, n, n_forced, k,
                           kept_idx, dev_status);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

int launch_seqnorm_select(const float* s_raw, const float* block_ss, int64_t n, float eps_seq,
                          float* score_norm, const uint8_t* forced, int64_t n_forced, int64_t k,
                          int32_t* kept_idx, int32_t* dev_status, void* ws, void* stream) {
    static_assert(kSelectOneWgMax == kThreads * 16, "one workgroup of 16 keys a thread");
    static_assert(kSelectMultiMin == kSelectOneWgMax + 1, "the two forms meet");
    const int kpt = select_kpt(n);
    if (kpt > 0) {
        hipStream_t s = (hipStream_t)stream;
        const SelectWs w = select_ws(static_cast<char*>(ws) + gate_bytes(n), n);
        switch (kpt) {
            case 8:
                return launch_select_multi<8>(s_raw, forced, n, n_forced, k, kept_idx, dev_status, w, s, block_ss,
                                              eps_seq, score_norm);
            case 16:
                return launch_select_multi<16>(s_raw, forced, n, n_forced, k, kept_idx, dev_status, w, s, block_ss,
                                               eps_seq, score_norm);
            default:
                return launch_select_multi<32>(s_raw, forced, n, n_forced, k, kept_idx, dev_status, w, s, block_ss,
                                               eps_seq, score_norm);
        }
    }
    if (n > kSelectOneWgMax) return TG_EUNSUPPORTED;
    hipLaunchKernelGGL((select_topk_regs<16, true>), dim3(1), dim3(kThreads), 0, (hipStream_t)stream, s_raw, forced,
                       n, n_forced, k, kept_idx, dev_status, block_ss, gate_partials(n), eps_seq, score_norm);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace tgi
