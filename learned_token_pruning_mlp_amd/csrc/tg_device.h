// tg_device.h -- small device helpers shared by the HIP kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 bit patterns (low / high half of a packed word) widened to fp32, exactly.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair with the hardware converter (v_cvt_pk_bf16_f32,
// round to nearest even); lo lands in bits 0..15.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// 32x32x16 bf16 matrix-core product: C += A * B.
// A: lane l holds row (l % 32), 8 k-values of k-group (l / 32).
// B: lane l holds column (l % 32), the same 8 k-values of k-group (l / 32).
// C: lane l holds column (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4) for i = 0..15.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Values of lanes l and l ^ 32 combined, in every lane (gfx950 cross-half
// swap: one VALU op, no LDS).
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Sequence RMSNorm of the gate scores: 1 / rho, rho = sqrt(sum s^2 / n + eps),
// from the scorer's per-workgroup partial sums of squared raw scores, in one
// fixed order, so that every kernel that forms it gets the same value:
// threads 0 .. 255 of a workgroup each add every 256-th partial in fp64
// (seq_ss_partial), the four waves reduce by an xor butterfly whose lane-0
// value is kept, and the four wave sums are added in wave order
// (seq_inv_rho, after a barrier).  The scores are then s * (1 / rho).
// A thread's partials are loaded four at a time from clamped indices, with no
// branch between the loads (one round trip per four, not one per partial);
// the ones past the end count as +0.0, which leaves the sum of non-negative
// terms unchanged, so the order of the additions is the one stated above.
constexpr int kSeqSumThreads = 256;
__device__ __forceinline__ void seq_ss_partial(const float* block_ss, int64_t nblocks, double* red) {
    const int tid = threadIdx.x;  // < kSeqSumThreads
    double acc = 0.0;
    for (int64_t b0 = tid; b0 < nblocks; b0 += 4 * kSeqSumThreads) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t b = b0 + (int64_t)j * kSeqSumThreads;
            x[j] = block_ss[b < nblocks ? b : nblocks - 1];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc += b0 + (int64_t)j * kSeqSumThreads < nblocks ? (double)x[j] : 0.0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if ((tid & 63) == 0) red[tid >> 6] = acc;
}
__device__ __forceinline__ float seq_inv_rho(const double* red, int64_t n, float eps) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kSeqSumThreads / 64; ++w) tot += red[w];
    return (float)(1.0 / sqrt(tot / (double)n + (double)eps));
}

}  // namespace tgd
