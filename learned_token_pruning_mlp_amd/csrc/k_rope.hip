// k_rope.hip -- rotary embedding at the original positions of the kept tokens.
//
// Kept tokens keep their original position encoding (aiwillknow.com,
// Figure 1(a)(b)), so the upper layers rotate q and k by pos_t, not by the
// rank t in the kept list.  Half-split pairs (j, j + D/2), frequency
// theta^(-2j/D).  Angles and rotations are evaluated in fp64 (at positions
// near 1.3e5 an fp32 angle is off by ~1e-2 rad) and each output is rounded to
// bf16 once, to nearest-even.
//
// HBM-bound in-place update.  q and k of the same rows are rotated in one
// launch: a workgroup takes one row of both tensors, first issues the
// 16-byte loads of both halves of its (head, 8-pair) pieces, then evaluates
// the row's cos/sin pairs into LDS while the loads are in flight (once per
// row for all q and k heads), then every thread rotates and stores.  The
// frequency of pair j is 2^(-(2j/D) log2 theta) in fp64 on the device (the
// per-element path takes them from the host's fp64 pow); each angle is
// reduced to [-pi, pi] exactly enough (two-constant Cody-Waite step with
// fused multiply-adds, error ~1e-15 rad) before sin/cos.  Other head_dims and unaligned
// tensors take a per-element loop, one tensor at a time.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::u32x4;

constexpr int kThreads = 128;

// Frequencies theta^(-2j/D), j < D/2, evaluated once on the host in fp64.
struct Freqs {
    double f[128];
};

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) { return (double)__uint_as_float(bits16 << 16); }

// fp64 -> bf16, nearest-even, for finite values.  The hardware rounds to fp32
// (nearest-even); a second rounding to bf16 can only go wrong when that fp32
// value sits exactly on a bf16 tie, in which case the side of the exact value
// decides.
__device__ __forceinline__ uint32_t f64_to_bf16(double y) {
    const float f = (float)y;
    uint32_t u = __float_as_uint(f);
    if ((u & 0xffffu) == 0x8000u && (double)f != y) u += (fabs(y) > fabs((double)f)) ? 1u : 0xffffffffu;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// cos/sin of p * f (one angle), reduced to [-pi, pi] first.
__device__ __forceinline__ void angle(int32_t p, double f, double* c, double* s) {
    constexpr double kTwoPiHi = 6.283185307179586;        // 2 pi rounded to double
    constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2 pi - kTwoPiHi
    constexpr double kInvTwoPi = 0.15915494309189535;
    const double phi = (double)p * f;
    const double k = rint(phi * kInvTwoPi);
    const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, phi));
    sincos(r, s, c);
}

// cos/sin of pos * f_j for j < half into LDS.
__device__ __forceinline__ void angles(int32_t p, int half, const Freqs& fr, double* cs, double* sn) {
    for (int j = threadIdx.x; j < half; j += kThreads) angle(p, fr.f[j], &cs[j], &sn[j]);
}

__device__ __forceinline__ void rotate8(u32x4 a, u32x4 b, const double* c8, const double* s8, u32x4& ya, u32x4& yb) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t oa = 0, ob = 0;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const double c = c8[2 * w + p], s = s8[2 * w + p];
            const double av = bf16_to_f64((a[w] >> (16 * p)) & 0xffffu);
            const double bv = bf16_to_f64((b[w] >> (16 * p)) & 0xffffu);
            oa |= f64_to_bf16(fma(av, c, -(bv * s))) << (16 * p);
            ob |= f64_to_bf16(fma(bv, c, av * s)) << (16 * p);
        }
        ya[w] = oa;
        yb[w] = ob;
    }
}

// head_dim 64, 128 or 256 and both tensors 16-byte aligned: eight pairs per
// 16-byte piece.  One workgroup takes one row of two tensors that share the
// positions (q with h0 heads and k with h1 heads; h1 = 0 for one tensor), so
// the fp64 angles of a row are evaluated once for all its heads.  Order of
// work: the angle inputs (position, frequency), then every data load of the
// row, then the angles (waiting only for their inputs while the data loads
// fly), then rotate and store.
constexpr int kThreadsV8 = 256;
constexpr int kUnitsV8 = 4;  // 16-byte pieces per thread in the first pass (at most)

template <int D>
__global__ __launch_bounds__(kThreadsV8) void rope_row_v8(uint16_t* __restrict__ x0, int h0,
                                                          uint16_t* __restrict__ x1, int h1,
                                                          const int32_t* __restrict__ pos, double log2_theta) {
    constexpr int HALF = D / 2, GROUPS = HALF / 8;
    static_assert((GROUPS & (GROUPS - 1)) == 0, "power-of-two groups");
    __shared__ double cs[HALF], sn[HALF];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int units = (h0 + h1) * GROUPS;
    const int passes = min(kUnitsV8, (units + kThreadsV8 - 1) / kThreadsV8);  // workgroup-uniform
    // unit e: head hh = e / GROUPS (the first h0 in x0, the rest in x1),
    // pairs 8 * (e % GROUPS) .. +7
    auto unit_ptr = [&](int e) -> uint16_t* {
        const int hh = e / GROUPS, j0 = 8 * (e % GROUPS);
        return hh < h0 ? x0 + (row * h0 + hh) * D + j0 : x1 + (row * h1 + (hh - h0)) * D + j0;
    };
    // angle inputs: the position (a scalar load) and this thread's frequency
    // theta^(-2j/D) = 2^(-(2j/D) log2 theta), evaluated in fp64 (no vector
    // load, so the angles never wait for the data loads)
    const int32_t p = pos[row];
    const double f = exp2(-(double)(2 * (tid < HALF ? tid : 0)) / (double)D * log2_theta);
    u32x4 a[kUnitsV8], b[kUnitsV8];
#pragma unroll
    for (int u = 0; u < kUnitsV8; ++u) {
        if (u >= passes) break;
        // threads past the last unit re-read unit 0 (always present) and do
        // not store: no branch around the loads, so they stay in flight together
        const int e = u * kThreadsV8 + tid;
        const uint16_t* xp = unit_ptr(e < units ? e : 0);
        a[u] = *reinterpret_cast<const u32x4*>(xp);
        b[u] = *reinterpret_cast<const u32x4*>(xp + HALF);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (tid < HALF) angle(p, f, &cs[tid], &sn[tid]);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kUnitsV8; ++u) {
        if (u >= passes) break;
        const int e = u * kThreadsV8 + tid;
        if (e < units) {
            uint16_t* xp = unit_ptr(e);
            const int j0 = 8 * (e % GROUPS);
            u32x4 ya, yb;
            rotate8(a[u], b[u], &cs[j0], &sn[j0], ya, yb);
            *reinterpret_cast<u32x4*>(xp) = ya;
            *reinterpret_cast<u32x4*>(xp + HALF) = yb;
        }
    }
    // rows with more heads than one pass holds
    for (int e = kUnitsV8 * kThreadsV8 + tid; e < units; e += kThreadsV8) {
        uint16_t* xp = unit_ptr(e);
        const int j0 = 8 * (e % GROUPS);
        const u32x4 av = *reinterpret_cast<const u32x4*>(xp);
        const u32x4 bv = *reinterpret_cast<const u32x4*>(xp + HALF);
        u32x4 ya, yb;
        rotate8(av, bv, &cs[j0], &sn[j0], ya, yb);
        *reinterpret_cast<u32x4*>(xp) = ya;
        *reinterpret_cast<u32x4*>(xp + HALF) = yb;
    }
}

// Any even D <= 256, 2-byte alignment: one pair per thread.
__global__ __launch_bounds__(kThreads) void rope_row_v1(uint16_t* __restrict__ x, const int32_t* __restrict__ pos,
                                                        int heads, int D, Freqs fr) {
    __shared__ double cs[128], sn[128];
    const int64_t row = blockIdx.x;
    const int half = D / 2;
    angles(pos[row], half, fr, cs, sn);
    __syncthreads();
    uint16_t* xr = x + row * heads * D;
    for (int e = threadIdx.x; e < heads * half; e += kThreads) {
        const int hh = e / half, j = e % half;
        uint16_t* xp = xr + hh * D;
        const double av = bf16_to_f64(xp[j]);
        const double bv = bf16_to_f64(xp[j + half]);
        xp[j] = (uint16_t)f64_to_bf16(fma(av, cs[j], -(bv * sn[j])));
        xp[j + half] = (uint16_t)f64_to_bf16(fma(bv, cs[j], av * sn[j]));
    }
}

}  // namespace

namespace tgi {

static Freqs make_freqs(int head_dim, double theta) {
    Freqs fr;
    const int half = head_dim / 2;
    for (int j = 0; j < 128; ++j) fr.f[j] = j < half ? pow(theta, -2.0 * (double)j / (double)head_dim) : 0.0;
    return fr;
}

int launch_rope_qk(uint16_t* q, uint16_t* k, const int32_t* pos, int64_t rows, int hq, int hk, int head_dim,
                   double theta, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const Freqs fr = make_freqs(head_dim, theta);
    const bool vec = (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
                     (reinterpret_cast<uintptr_t>(q) & 15) == 0 && (hk == 0 || (reinterpret_cast<uintptr_t>(k) & 15) == 0);
    if (vec) {
        const dim3 grid((unsigned)rows);
        if (head_dim == 64)
            hipLaunchKernelGGL(rope_row_v8<64>, grid, dim3(kThreadsV8), 0, s, q, hq, k, hk, pos, log2(theta));
        else if (head_dim == 128)
            hipLaunchKernelGGL(rope_row_v8<128>, grid, dim3(kThreadsV8), 0, s, q, hq, k, hk, pos, log2(theta));
        else
            hipLaunchKernelGGL(rope_row_v8<256>, grid, dim3(kThreadsV8), 0, s, q, hq, k, hk, pos, log2(theta));
    } else {
        hipLaunchKernelGGL(rope_row_v1, dim3((unsigned)rows), dim3(kThreads), 0, s, q, pos, hq, head_dim, fr);
        if (hk > 0)
            hipLaunchKernelGGL(rope_row_v1, dim3((unsigned)rows), dim3(kThreads), 0, s, k, pos, hk, head_dim, fr);
    }
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

int launch_rope(uint16_t* x, const int32_t* pos, int64_t rows, int heads, int head_dim, double theta,
                void* stream) {
    return launch_rope_qk(x, nullptr, pos, rows, heads, 0, head_dim, theta, stream);
}

}  // namespace tgi
