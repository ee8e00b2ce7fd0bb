// k_rope.hip -- rotary embedding at the original positions of the kept tokens.
//
// Kept tokens keep their original position encoding (aiwillknow.com,
// Figure 1(a)(b)), so the upper layers rotate q and k by pos_t, not by the
// rank t in the kept list.  Half-split pairs (j, j + D/2), frequency
// theta^(-2j/D).  Angles and rotations are evaluated in fp64 (at positions
// near 1.3e5 an fp32 angle is off by ~1e-2 rad) and each output is rounded to
// bf16 once, to nearest-even.
//
// HBM-bound in-place update, one workgroup per row.  Each thread first issues
// the 16-byte loads of both halves of its (head, 8-pair) pieces, then the
// row's cos/sin pairs are evaluated into LDS while the loads are in flight,
// then every thread rotates and stores.  The frequencies are evaluated once
// per call on the host (fp64 pow) and passed by value; each angle is reduced
// to [-pi, pi] exactly enough (two-constant Cody-Waite step with fused
// multiply-adds, error ~1e-15 rad) before sin/cos.  Shapes whose halves are
// not 16-byte multiples take a per-element loop.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::u32x4;

constexpr int kThreads = 128;
constexpr int kUnits = 4;  // 16-byte pieces per thread and pass

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

// cos/sin of pos * f_j for j < half into LDS.
__device__ __forceinline__ void angles(double p, int half, const Freqs& fr, double* cs, double* sn) {
    constexpr double kTwoPiHi = 6.283185307179586;        // 2 pi rounded to double
    constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2 pi - kTwoPiHi
    constexpr double kInvTwoPi = 0.15915494309189535;
    for (int j = threadIdx.x; j < half; j += kThreads) {
        const double phi = p * fr.f[j];
        const double k = rint(phi * kInvTwoPi);
        const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, phi));
        double s, c;
        sincos(r, &s, &c);
        cs[j] = c;
        sn[j] = s;
    }
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

// D/2 a multiple of 8 and x 16-byte aligned: eight pairs per 16-byte piece.
__global__ __launch_bounds__(kThreads) void rope_row_v8(uint16_t* __restrict__ x, const int32_t* __restrict__ pos,
                                                        int heads, int D, Freqs fr) {
    __shared__ double cs[128], sn[128];
    const int64_t row = blockIdx.x;
    const int half = D / 2, groups = half / 8;
    const int units = heads * groups;
    uint16_t* xr = x + row * heads * D;
    const double p = (double)pos[row];
    for (int base = 0; base < units; base += kThreads * kUnits) {
        u32x4 a[kUnits], b[kUnits];
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int e = base + u * kThreads + threadIdx.x;
            if (e < units) {
                const uint16_t* xp = xr + (e / groups) * D + 8 * (e % groups);
                a[u] = *reinterpret_cast<const u32x4*>(xp);
                b[u] = *reinterpret_cast<const u32x4*>(xp + half);
            }
        }
        if (base == 0) {
            angles(p, half, fr, cs, sn);
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int e = base + u * kThreads + threadIdx.x;
            if (e < units) {
                uint16_t* xp = xr + (e / groups) * D + 8 * (e % groups);
                const int j0 = 8 * (e % groups);
                u32x4 ya, yb;
                rotate8(a[u], b[u], cs + j0, sn + j0, ya, yb);
                *reinterpret_cast<u32x4*>(xp) = ya;
                *reinterpret_cast<u32x4*>(xp + half) = yb;
            }
        }
    }
}

// Any even D <= 256, 2-byte alignment: one pair per thread.
__global__ __launch_bounds__(kThreads) void rope_row_v1(uint16_t* __restrict__ x, const int32_t* __restrict__ pos,
                                                        int heads, int D, Freqs fr) {
    __shared__ double cs[128], sn[128];
    const int64_t row = blockIdx.x;
    const int half = D / 2;
    angles((double)pos[row], half, fr, cs, sn);
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

int launch_rope(uint16_t* x, const int32_t* pos, int64_t rows, int heads, int head_dim, double theta,
                void* stream) {
    Freqs fr;
    const int half = head_dim / 2;
    for (int j = 0; j < 128; ++j) fr.f[j] = j < half ? pow(theta, -2.0 * (double)j / (double)head_dim) : 0.0;
    const dim3 grid((unsigned)rows);
    const bool vec = half % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    if (vec)
        hipLaunchKernelGGL(rope_row_v8, grid, dim3(kThreads), 0, (hipStream_t)stream, x, pos, heads, head_dim, fr);
    else
        hipLaunchKernelGGL(rope_row_v1, grid, dim3(kThreads), 0, (hipStream_t)stream, x, pos, heads, head_dim, fr);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace tgi
