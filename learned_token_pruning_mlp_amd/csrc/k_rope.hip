// k_rope.hip -- rotary embedding at the original positions of the kept tokens.
//
// Kept tokens keep their original position encoding (aiwillknow.com,
// Figure 1(a)(b)), so the upper layers rotate q and k by pos_t, not by the
// rank t in the kept list.  Half-split pairs (j, j + D/2), frequency
// theta^(-2j/D).  Angles and rotations are evaluated in fp64 (at positions
// near 1.3e5 an fp32 angle is off by ~1e-2 rad) and each output is rounded to
// bf16 once: round-to-odd to fp32, then nearest-even to bf16, which equals a
// direct nearest-even rounding of the fp64 value.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    float f = __double2float_rz(x);
    uint32_t u = __float_as_uint(f);
    if ((double)f != x && x == x) u |= 1u;  // sticky bit: round-to-odd
    return (uint16_t)tgd::f32_to_bf16(__uint_as_float(u));
}

__global__ __launch_bounds__(kThreads) void rope_rows(uint16_t* __restrict__ x, const int32_t* __restrict__ pos,
                                                      int heads, int D, double log_theta) {
    __shared__ double cs[128], sn[128];
    const int64_t row = blockIdx.x;
    const int half = D / 2;
    const double p = (double)pos[row];
    for (int j = threadIdx.x; j < half; j += kThreads) {
        const double f = exp(-(2.0 * (double)j / (double)D) * log_theta);
        double s, c;
        sincos(p * f, &s, &c);
        cs[j] = c;
        sn[j] = s;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < heads * half; e += kThreads) {
        const int hh = e / half, j = e % half;
        uint16_t* xr = x + (row * heads + hh) * D;
        const double a = (double)tgd::bf16lo(xr[j]);
        const double b = (double)tgd::bf16lo(xr[j + half]);
        const double ya = a * cs[j] - b * sn[j];
        const double yb = b * cs[j] + a * sn[j];
        xr[j] = f64_to_bf16(ya);
        xr[j + half] = f64_to_bf16(yb);
    }
}

}  // namespace

namespace tgi {

int launch_rope(uint16_t* x, const int32_t* pos, int64_t rows, int heads, int head_dim, double theta,
                void* stream) {
    hipLaunchKernelGGL(rope_rows, dim3((unsigned)rows), dim3(kThreads), 0, (hipStream_t)stream, x, pos, heads,
                       head_dim, log(theta));
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace tgi
