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
// Four 8-bit digit rounds find the key T of the (K-F)-th best prunable token
// and the number m of tokens equal to T that are taken (the m lowest-index
// ones).  The emit pass then writes the kept indices in ascending order:
// token i goes to slot (#forced-or-above-T before i) + min(#ties before i, m).
// Everything is integer arithmetic, so the result is bit-exact and
// deterministic.
//
// One workgroup of 1024 threads does the whole selection (one launch, no
// workspace traffic).  Up to 32768 tokens the keys stay in LDS (128 KB of the
// CU's 160 KB) after one read of the scores; longer prompts re-read the
// scores (L2-resident) in each round.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 32768;
constexpr uint32_t kForcedMark = 0xffffffffu;  // no score maps here (max key is +inf's)

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (f != f) return 0u;           // NaN ranks below everything
    if (u == 0x80000000u) u = 0u;    // -0.0 equals +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan over the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        T y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// Exclusive scan over the whole workgroup; returns the block total in *total.
__device__ __forceinline__ uint64_t block_excl_scan(uint64_t x, uint64_t* wsum, uint64_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t incl = wave_incl_scan(x, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        uint64_t w = lane < kWaves ? wsum[lane] : 0;
        uint64_t wi = wave_incl_scan(w, lane);
        if (lane < kWaves) wsum[lane] = wi - w;  // exclusive offsets
        if (lane == kWaves - 1) wsum[kWaves] = wi;
    }
    __syncthreads();
    uint64_t r = incl - x + wsum[wave];
    *total = wsum[kWaves];
    __syncthreads();
    return r;
}

// Adds one count per active lane to hist[bin].  Keys of real data often share
// a few digit values (a Gaussian score has most of its mass in two or three
// top-byte bins), and 64 lanes adding to one LDS word serialise.  So the
// bins of the first two active lanes are counted with a ballot and added once
// each; the remaining lanes, now mostly spread out, use plain LDS atomics.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool act, int lane) {
#pragma unroll
    for (int peel = 0; peel < 2; ++peel) {
        const uint64_t am = __builtin_amdgcn_ballot_w64(act);
        if (am == 0) return;
        const int leader = __builtin_ctzll(am);
        const uint32_t lb = __builtin_amdgcn_readlane(bin, leader);
        const bool same = act && bin == lb;
        const uint64_t sm = __builtin_amdgcn_ballot_w64(same);
        if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__builtin_popcountll(sm));
        act = act && !same;
    }
    if (act) atomicAdd(&hist[bin], 1u);
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

template <bool kKeysInLds>
__global__ __launch_bounds__(kThreads) void select_topk_block(const float* __restrict__ score,
                                                              const uint8_t* __restrict__ forced,
                                                              int64_t n64, int64_t n_forced, int64_t k64,
                                                              int32_t* __restrict__ kept,
                                                              int32_t* __restrict__ dev_status) {
    __shared__ __attribute__((aligned(16))) uint32_t keys[kKeysInLds ? kLdsKeys : 4];
    __shared__ uint32_t whist[kWaves][256];
    __shared__ uint64_t wsum[kWaves + 1];
    __shared__ uint32_t ctl[4];
    __shared__ uint32_t wtot[4];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint32_t n = (uint32_t)n64, k = (uint32_t)k64;
    constexpr uint32_t kStep = kThreads * 16;  // tokens per sweep step: 4 groups of 4 per thread

    // Keys of 4 consecutive tokens starting at i (a multiple of 4; entries
    // past n read as kForcedMark-free zeros and are skipped by the callers).
    auto keys4 = [&](uint32_t i) -> uint4 {
        if (kKeysInLds) return *reinterpret_cast<const uint4*>(&keys[i]);
        return keys4_global(score, forced, i, n);
    };

    // Round 0: count the forced tokens (and park the keys in LDS).
    uint64_t fc = 0;
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
                if (i + q < n) {
                    fc += kk[q] == kForcedMark ? 1u : 0u;
                    if (kKeysInLds) keys[i + q] = kk[q];
                }
            }
        }
    }
    uint64_t F;
    block_excl_scan(fc, wsum, &F);  // its barriers also publish the LDS keys
    int64_t R = (int64_t)k - (int64_t)F;  // prunable tokens to choose
    if (tid == 0 && dev_status) {
        int32_t st = 0;
        if ((int64_t)F != n_forced) st |= TG_STATUS_FORCED_MISMATCH;
        if (R < 0) st |= TG_STATUS_FORCED_OVER_K;
        *dev_status = st;
    }
    if (R < 0) R = 0;

    // Rounds 1-4: radix select of the R-th largest prunable key.
    uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)R;
    uint32_t T = 0xffffffffu, m = 0;  // R == 0: no prunable token is taken
    if (R > 0) {
        for (int round = 0; round < 4; ++round) {
            const int shift = 24 - 8 * round;
            for (int b = tid; b < kWaves * 256; b += kThreads) (&whist[0][0])[b] = 0;
            __syncthreads();
            for (uint32_t c0 = 0; c0 < n; c0 += kStep) {
                uint4 kv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) kv[e] = keys4(c0 + (e * kThreads + tid) * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t i = c0 + (e * kThreads + tid) * 4;
                    const uint32_t kk[4] = {kv[e].x, kv[e].y, kv[e].z, kv[e].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t key = kk[q];
                        const bool act = i + q < n && key != kForcedMark && (key & pmask) == prefix;
                        hist_add(&whist[wave][0], (key >> shift) & 255u, act, lane);
                    }
                }
            }
            __syncthreads();
            uint32_t c = 0, incl = 0, b = 0;
            if (tid < 256) {
                // bins in descending order: thread t looks at digit 255 - t
                b = 255u - tid;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) c += whist[w][b];
                incl = wave_incl_scan(c, lane);
                if (lane == 63) wtot[wave] = incl;
            }
            __syncthreads();
            if (tid < 256) {
                for (int w = 0; w < wave; ++w) incl += wtot[w];
                const uint32_t excl = incl - c;
                if (excl < remaining && remaining <= incl) {
                    ctl[0] = b;
                    ctl[1] = remaining - excl;
                }
            }
            __syncthreads();
            prefix |= ctl[0] << shift;
            pmask |= 255u << shift;
            remaining = ctl[1];
            __syncthreads();
        }
        T = prefix;
        m = remaining;
    }

    // Emit, in index order: slot = (#kind1 before) + min(#ties before, m).
    uint64_t carry = 0;
    for (uint32_t c0 = 0; c0 < n; c0 += kThreads * 8) {
        const uint32_t base = c0 + (uint32_t)tid * 8;
        const uint4 k0 = keys4(base), k1 = keys4(base + 4);
        const uint32_t kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        uint8_t kind[8];  // 0 = dropped, 1 = forced or above T, 2 = equal to T
        uint32_t ca = 0, cb = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint8_t kd = 0;
            if (base + e < n) {
                const uint32_t key = kk[e];
                if (key == kForcedMark) kd = 1;
                else if (key > T) kd = 1;
                else if (key == T) kd = 2;
            }
            kind[e] = kd;
            ca += kd == 1;
            cb += kd == 2;
        }
        uint64_t tot;
        const uint64_t ex = block_excl_scan(((uint64_t)ca << 32) | cb, wsum, &tot) + carry;
        uint32_t A = (uint32_t)(ex >> 32), B = (uint32_t)ex;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (kind[e] == 1) {
                const uint32_t slot = A + (B < m ? B : m);
                if (slot < k) kept[slot] = (int32_t)(base + e);
                ++A;
            } else if (kind[e] == 2) {
                if (B < m) {
                    const uint32_t slot = A + B;
                    if (slot < k) kept[slot] = (int32_t)(base + e);
                }
                ++B;
            }
        }
        carry += tot;
    }
}

}  // namespace

namespace tgi {

int launch_select_topk(const float* score, const uint8_t* forced, int64_t n, int64_t n_forced,
                       int64_t k, int32_t* kept_idx, int32_t* dev_status, void* ws, void* stream) {
    (void)ws;
    hipStream_t s = (hipStream_t)stream;
    if (n <= kLdsKeys)
        hipLaunchKernelGGL(select_topk_block<true>, dim3(1), dim3(kThreads), 0, s, score, forced, n,
                           n_forced, k, kept_idx, dev_status);
    else
        hipLaunchKernelGGL(select_topk_block<false>, dim3(1), dim3(kThreads), 0, s, score, forced, n,
                           n_forced, k, kept_idx, dev_status);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace tgi
