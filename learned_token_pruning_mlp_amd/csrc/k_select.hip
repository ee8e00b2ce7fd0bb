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
// One workgroup of 1024 threads does the whole selection (one launch, no
// workspace traffic).  Up to 32768 tokens each thread keeps the keys of 16
// (or 32) consecutive tokens in registers after one read of the scores, so
// every later phase works on registers; the histogram copies are cleared
// while that read is in flight, the first histogram goes into eight LDS
// copies chosen by lane (float keys crowd into a few dozen top-11-bit bins,
// so lanes of one wave would otherwise collide on the same words), and the
// later rounds filter the keys by the prefix chosen so far.  Bin searches run in one wave with DPP scans; the emit pass takes one
// block scan of packed counts and visits only the kept tokens.  Longer
// prompts re-read the scores (L2-resident) in each sweep and gather the
// first round's bucket into LDS when it fits.
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
template <int KPT>
__global__ __launch_bounds__(kThreads) void select_topk_regs(const float* __restrict__ score,
                                                             const uint8_t* __restrict__ forced,
                                                             int64_t n64, int64_t n_forced, int64_t k64,
                                                             int32_t* __restrict__ kept,
                                                             int32_t* __restrict__ dev_status) {
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
    // histogram copies are cleared while the loads are in flight.
    float4 sc[KPT / 4];
    uint32_t fm[KPT / 4];
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

}  // namespace

namespace tgi {

int launch_select_topk(const float* score, const uint8_t* forced, int64_t n, int64_t n_forced,
                       int64_t k, int32_t* kept_idx, int32_t* dev_status, void* ws, void* stream) {
    (void)ws;
    hipStream_t s = (hipStream_t)stream;
    if (n <= kThreads * 16)
        hipLaunchKernelGGL(select_topk_regs<16>, dim3(1), dim3(kThreads), 0, s, score, forced, n, n_forced, k,
                           kept_idx, dev_status);
    else if (n <= kThreads * 32)
        hipLaunchKernelGGL(select_topk_regs<32>, dim3(1), dim3(kThreads), 0, s, score, forced, n, n_forced, k,
                           kept_idx, dev_status);
    else
        hipLaunchKernelGGL(select_topk_block, dim3(1), dim3(kThreads), 0, s, score, forced, n, n_forced, k,
                           kept_idx, dev_status);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace tgi
