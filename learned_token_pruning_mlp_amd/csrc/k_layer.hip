// k_layer.hip -- the per-token pieces of an upper decoder layer on the kept rows.
//
// Above the gate only the kept tokens go through the backbone's layers
// (fluxbbs.com TokenGate article, section on where the gate sits;
// aiwillknow.com, Figure 1(a)(b)).  The backbone here is Qwen3-shaped: a
// pre-norm block with RMSNorm, q/k RMSNorm per head, RoPE, attention, an
// output projection with a residual add, RMSNorm, and a SwiGLU MLP with a
// residual add.  The projections are plain GEMMs (rocBLAS, tg_blas.cpp);
// these kernels are the two row-wise pieces between them:
//
//   rmsnorm_rows: y_r = x_r / sqrt(mean_k x_rk^2 + eps) * w, in fp32, rounded
//                 once to bf16.  Row lengths that are multiples of 8 (16-byte
//                 pieces); one group of dim/8 lanes (at most 64) per row, so a
//                 256-thread workgroup takes one row of 2048 and 32 heads of
//                 64.
//   swiglu_rows:  out_r = silu(g_r) * u_r with g, u the two halves of one row
//                 of the fused gate/up projection, in fp32, rounded once.
//
// Both are HBM-bound streaming kernels with 16-byte loads and stores.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::u32x4;

constexpr int kThreads = 256;

__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// LANES lanes per row (a power of two, <= 64): each lane holds PER pieces of
// 8 values; the row sum goes through a butterfly inside the lane group.
// y may equal x (the per-head norms of q and k run in place), so neither is
// declared restrict: every lane reads its pieces before any lane of the row
// writes, and a row is read and written by one lane group only.
template <int LANES, int PER>
__global__ __launch_bounds__(kThreads) void rmsnorm_rows(const uint16_t* x,
                                                         const uint16_t* __restrict__ w, uint16_t* y,
                                                         int64_t rows, int dim, float eps) {
    constexpr int RPB = kThreads / LANES;  // rows per workgroup
    const int tid = threadIdx.x;
    const int sub = tid % LANES;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / LANES;
    const bool ok = row < rows;
    const int pieces = dim / 8;
    // A lane whose pieces are all in range loads them (and its weights) with
    // no branch between the accesses, so they go out together; the guarded
    // path (short rows, rows past the end) waits per access.
    const bool all = ok && (PER - 1) * LANES + sub < pieces;
    u32x4 v[PER], wv[PER];
    if (all) {
#pragma unroll
        for (int p = 0; p < PER; ++p) v[p] = *reinterpret_cast<const u32x4*>(x + row * dim + 8 * (p * LANES + sub));
#pragma unroll
        for (int p = 0; p < PER; ++p) wv[p] = *reinterpret_cast<const u32x4*>(w + 8 * (p * LANES + sub));
    } else {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = p * LANES + sub;
            const bool in = ok && c < pieces;
            v[p] = in ? *reinterpret_cast<const u32x4*>(x + row * dim + 8 * c) : u32x4{0u, 0u, 0u, 0u};
            wv[p] = in ? *reinterpret_cast<const u32x4*>(w + 8 * c) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = lo16(v[p][e]), b = hi16(v[p][e]);
            ss = fmaf(a, a, ss);
            ss = fmaf(b, b, ss);
        }
    }
#pragma unroll
    for (int o = LANES / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float r = 1.0f / sqrtf(ss / (float)dim + eps);
    if (!ok) return;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int c = p * LANES + sub;
        if (c >= pieces) continue;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = tgd::cvt_pk_bf16(lo16(v[p][e]) * r * lo16(wv[p][e]), hi16(v[p][e]) * r * hi16(wv[p][e]));
        *reinterpret_cast<u32x4*>(y + row * dim + 8 * c) = o;
    }
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// One thread per 16-byte piece of the output (8 values).
__global__ __launch_bounds__(kThreads) void swiglu_rows(const uint16_t* __restrict__ gu, uint16_t* __restrict__ out,
                                                        int64_t rows, int inter) {
    const int pieces = inter / 8;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= rows * pieces) return;
    const int64_t row = i / pieces;
    const int c = (int)(i % pieces);
    const u32x4 g = *reinterpret_cast<const u32x4*>(gu + row * 2 * inter + 8 * c);
    const u32x4 u = *reinterpret_cast<const u32x4*>(gu + row * 2 * inter + inter + 8 * c);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = tgd::cvt_pk_bf16(silu(lo16(g[e])) * lo16(u[e]), silu(hi16(g[e])) * hi16(u[e]));
    *reinterpret_cast<u32x4*>(out + row * inter + 8 * c) = o;
}

template <int LANES, int PER>
void launch_rms(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t rows, int dim, float eps, hipStream_t s) {
    constexpr int RPB = kThreads / LANES;
    hipLaunchKernelGGL((rmsnorm_rows<LANES, PER>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kThreads), 0, s, x,
                       w, y, rows, dim, eps);
}

}  // namespace

namespace tgi {

int launch_rmsnorm(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t rows, int dim, float eps,
                   void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const int pieces = dim / 8;
    if (pieces <= 8)
        launch_rms<8, 1>(x, w, y, rows, dim, eps, s);
    else if (pieces <= 16)
        launch_rms<16, 1>(x, w, y, rows, dim, eps, s);
    else if (pieces <= 32)
        launch_rms<32, 1>(x, w, y, rows, dim, eps, s);
    else if (pieces <= 64)
        launch_rms<64, 1>(x, w, y, rows, dim, eps, s);
    else if (pieces <= 128)
        launch_rms<64, 2>(x, w, y, rows, dim, eps, s);
    else if (pieces <= 256)
        launch_rms<64, 4>(x, w, y, rows, dim, eps, s);
    else if (pieces <= 512)
        launch_rms<64, 8>(x, w, y, rows, dim, eps, s);
    else
        return TG_EUNSUPPORTED;
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

int launch_swiglu(const uint16_t* gu, uint16_t* out, int64_t rows, int inter, void* stream) {
    const int64_t total = rows * (inter / 8);
    hipLaunchKernelGGL(swiglu_rows, dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       (hipStream_t)stream, gu, out, rows, inter);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace tgi
