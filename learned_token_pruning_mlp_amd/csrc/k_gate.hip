// k_gate.hip -- gate scoring network and sequence RMSNorm of the scores.
//
// At the gate layer a small MLP reads each token's normalised post-attention
// residual and returns one scalar; the scores are then RMSNorm-normalised
// along the sequence (fluxbbs.com TokenGate article, section on where the
// gate sits; slinene.github.io digest, method key points; aiwillknow.com,
// Figure 1(a)(b)).
//
// Kernel 1 (gate_mlp): one workgroup takes 64 residual rows.  The residual
// row norm is applied after the product, as a per-row scale (the product is
// linear in the row), so the matrix cores see the exact bf16 residual:
//     a_ij = r_i * (h_i . w1_j) + b1_j,  r_i = 1/sqrt(mean_k h_ik^2 + eps)
// The product runs on 32x32x16 bf16 MFMA with fp32 accumulation as
// C^T = W1 . H^T: each lane then owns one token column and 16 hidden rows per
// block, so GELU, the w2 dot product and the reduction over hidden units stay
// in registers except for one exchange between the two half-waves and one
// between waves.  Residual and W1 tiles of 64 d-columns go from memory
// straight into a three-stage LDS ring with 16-byte direct loads (two tiles
// in flight while the third is multiplied; W1 is re-read from L2 by every
// workgroup, the residual once from HBM).  Rows are stored with their eight
// 16-byte pieces XOR-permuted so the operand reads spread over the banks.
// The row sums of squares come from the same operand reads.  Each workgroup
// also writes the sum of its scores' squares (fixed order).
//
// Kernel 2 (gate_seqnorm): every workgroup reduces those per-block partial
// sums in the same fixed order (fp64), forms rho = sqrt(mean s^2 + eps) and
// scales its slice of the scores.  No float atomics: results are
// deterministic run to run.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::f32x16;
using tgd::u32x4;

constexpr int kThreads = 256;
constexpr int kBT = tgi::kGateRowsPerBlock;  // 64 rows per workgroup
constexpr int kKC = 64;                      // d-columns per LDS tile

template <int HD>
struct Cfg {
    static constexpr int WAVES_H = HD >= 128 ? 4 : 2;  // waves along hidden units
    static constexpr int WAVES_T = 4 / WAVES_H;         // waves along tokens
    static constexpr int WH = HD / WAVES_H;             // hidden units per wave
    static constexpr int WT = kBT / WAVES_T;            // tokens per wave
    static constexpr int MB = WH / 32;                  // 32-row blocks of hidden units
    static constexpr int NB = WT / 32;                  // 32-column blocks of tokens
    static_assert(MB >= 1 && NB >= 1, "tile shape");
};

// GELU(a) = a * Phi(a) = a/2 * (1 + erf(a / sqrt 2)).  erf by the rational
// approximation of Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (|error| <= 1.5e-7 for x >= 0; odd extension):
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x).
// Over the 256 hidden units of a score this moves the normalised score by
// about 1e-5 at most.
__device__ __forceinline__ float gelu_erf(float a) {
    constexpr float p = 0.3275911f;
    constexpr float a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f, a4 = -1.453152027f,
                    a5 = 1.061405429f;
    const float x = fabsf(a) * 0.70710678118654752440f;
    const float t = __builtin_amdgcn_rcpf(fmaf(p, x, 1.0f));
    const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
    const float e = __builtin_amdgcn_exp2f(-x * x * 1.44269504088896340736f);
    const float erf_abs = fmaf(-poly, e, 1.0f);
    const float erf_v = a < 0.0f ? -erf_abs : erf_abs;
    return 0.5f * a * (1.0f + erf_v);
}

// Permutation of the eight 16-byte pieces of a 128-byte LDS row (XOR mask
// by row).  gfx950 LDS has 64 banks and a 16-byte read serves 16 consecutive
// lanes per cycle, which need distinct (address/16) mod 16: two 128-byte rows
// span the banks once, so rotating (row/2) mod 8 right by one bit gives the
// 16 rows read together 16 distinct bank groups.
__device__ __forceinline__ int swz8(int r) {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
}

#define TG_LDS __attribute__((address_space(3)))

// N 16-byte LDS reads issued together and waited for before the block ends
// (the registers an inline-assembly load writes must be complete when the
// block ends).
template <int N>
__device__ __forceinline__ void lds_read_wait(u32x4 (&v)[N], const uint32_t (&a)[N]);
template <>
__device__ __forceinline__ void lds_read_wait<4>(u32x4 (&v)[4], const uint32_t (&a)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
}
template <>
__device__ __forceinline__ void lds_read_wait<6>(u32x4 (&v)[6], const uint32_t (&a)[6]) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b128 %2, %8\n\t"
        "ds_read_b128 %3, %9\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
        : "memory");
}
template <>
__device__ __forceinline__ void lds_read_wait<8>(u32x4 (&v)[8], const uint32_t (&a)[8]) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
          "=&v"(v[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define TG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

template <int HD>
__global__ __launch_bounds__(kThreads) void gate_mlp(const uint16_t* __restrict__ resid,
                                                     const uint16_t* __restrict__ w1,
                                                     const uint16_t* __restrict__ b1,
                                                     const uint16_t* __restrict__ w2, float b2,
                                                     int64_t n, int d, float eps_row,
                                                     float* __restrict__ s_out,
                                                     float* __restrict__ block_ss) {
    using C = Cfg<HD>;
    constexpr int H_BYTES = kBT * kKC * 2;            // residual tile: 64 rows x 128 bytes
    constexpr int W_BYTES = HD * kKC * 2;             // W1 tile: HD rows x 128 bytes
    constexpr int STAGE = H_BYTES + W_BYTES;
    constexpr int H_LOADS = H_BYTES / 1024 / 4;       // 1 KB direct-load instructions per wave
    constexpr int W_LOADS = W_BYTES / 1024 / 4;
    constexpr int VM_PER_TILE = H_LOADS + W_LOADS;
    // three pipeline stages, separate objects (see the tile loop)
    __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[STAGE];
    __shared__ float sB1[HD], sW2[HD];
    __shared__ float sSq[C::WAVES_H][kBT];
    __shared__ float sPart[C::WAVES_H][kBT];
    __shared__ float sR[kBT];
    __shared__ float sS[kBT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wh = wave % C::WAVES_H, wt = wave / C::WAVES_H;
    const int l32 = lane & 31, g = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.x * kBT;
    const int nchunks = d / kKC;

    for (int j = tid; j < HD; j += kThreads) {
        sB1[j] = b1 ? tgd::bf16lo(b1[j]) : 0.0f;
        sW2[j] = tgd::bf16lo(w2[j]);
    }

    // Direct HBM -> LDS loads of one 64-column tile: each wave instruction
    // fills one 1 KB block = 8 rows of 128 bytes; lane l writes slot l%8 of
    // row l/8 with the piece (l%8) ^ swz8(row).  Residual rows past n repeat
    // row n-1 (their scores are never written).
    // Instructions [i0, i1) of the VM_PER_TILE direct loads of a tile: the
    // residual blocks first, then the W1 blocks.
    auto issue_part = [&](int c, uint8_t* stg, int i0, int i1) {
        const int slot = lane & 7;
#pragma unroll
        for (int r = 0; r < VM_PER_TILE; ++r) {
            if (r < i0 || r >= i1) continue;
            if (r < H_LOADS) {
                const int blk = r * 4 + wave, row = blk * 8 + (lane >> 3);
                const int64_t gr = min(row0 + row, n - 1);
                const uint16_t* src = resid + gr * d + c * kKC + 8 * (slot ^ swz8(row));
                __builtin_amdgcn_global_load_lds(src, (TG_LDS void*)((TG_LDS uint8_t*)stg + blk * 1024), 16, 0, 0);
            } else {
                const int blk = (r - H_LOADS) * 4 + wave, row = blk * 8 + (lane >> 3);
                const uint16_t* src = w1 + (int64_t)row * d + c * kKC + 8 * (slot ^ swz8(row));
                __builtin_amdgcn_global_load_lds(src, (TG_LDS void*)((TG_LDS uint8_t*)stg + H_BYTES + blk * 1024),
                                                 16, 0, 0);
            }
        }
    };
    auto issue = [&](int c, uint8_t* stg) { issue_part(c, stg, 0, VM_PER_TILE); };

    f32x16 acc[C::MB][C::NB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = f32x16{};
    float ssq[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) ssq[nb] = 0.0f;

    // Per-lane LDS byte offsets (within a stage) of the operand rows, without
    // the piece: B (residual) rows first, then A (W1) rows.
    uint32_t roff[C::NB + C::MB];
    int rswz[C::NB + C::MB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
        const int row = wt * C::WT + nb * 32 + l32;
        roff[nb] = row * 128;
        rswz[nb] = swz8(row);
    }
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
        const int row = wh * C::WH + mb * 32 + l32;
        roff[C::NB + mb] = H_BYTES + row * 128;
        rswz[C::NB + mb] = swz8(row);
    }

    // One tile: wait for its loads (the next tile's stay in flight), start the
    // loads two tiles ahead into the stage every wave finished reading at the
    // previous step, multiply.  k-step s of half-wave g reads piece 2s+g of a
    // row.  The operand reads are issued from inline assembly that waits for
    // them before it ends: the compiler cannot tell these LDS reads from the
    // loads in flight into the other stages and would otherwise wait for all
    // of them; the explicit vector-memory waits above order them instead.
    auto step = [&](int c, const uint8_t* cur, uint8_t* ahead) {
        if (c + 1 < nchunks) {
            TG_WAIT_VMCNT(VM_PER_TILE);
        } else {
            TG_WAIT_VMCNT(0);
        }
        __builtin_amdgcn_s_barrier();
        const bool more = c + 2 < nchunks;
        const uint32_t base = (uint32_t)(uintptr_t)(const TG_LDS uint8_t*)cur;
        constexpr int NOP = C::NB + C::MB;  // operand reads per k-step
        constexpr int NPAIR = kKC / 32;     // k-step pairs per tile
#pragma unroll
        for (int s2 = 0; s2 < kKC / 16; s2 += 2) {
            // the loads two tiles ahead go out in slices between the pairs, so
            // the load path is not swamped before any multiply starts
            if (more) {
                constexpr int per = (VM_PER_TILE + NPAIR - 1) / NPAIR;
                issue_part(c + 2, ahead, (s2 / 2) * per, (s2 / 2 + 1) * per);
            }
            // both k-steps' operands in one block: the reads of this pair are in
            // flight while the matrix cores still work on the previous pair
            u32x4 op[2 * NOP];
            uint32_t addr[2 * NOP];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int i = 0; i < NOP; ++i)
                    addr[u * NOP + i] = base + roff[i] + 16 * ((2 * (s2 + u) + g) ^ rswz[i]);
            lds_read_wait<2 * NOP>(op, addr);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int s = s2 + u;
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb)
                        acc[mb][nb] = tgd::mfma32(op[u * NOP + C::NB + mb], op[u * NOP + nb], acc[mb][nb]);
                // row sums of squares: the waves sharing a token block split the k-steps
                if (s % C::WAVES_H == wh) {
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float lo = tgd::bf16lo(op[u * NOP + nb][q]), hi = tgd::bf16hi(op[u * NOP + nb][q]);
                            ssq[nb] = fmaf(lo, lo, ssq[nb]);
                            ssq[nb] = fmaf(hi, hi, ssq[nb]);
                        }
                    }
                }
            }
        }
    };
    issue(0, st0);
    if (nchunks > 1) issue(1, st1);
    for (int c = 0; c < nchunks; c += 3) {
        step(c, st0, st2);
        if (c + 1 < nchunks) step(c + 1, st1, st0);
        if (c + 2 < nchunks) step(c + 2, st2, st1);
    }

    // Row norms: combine the two half-waves, then the waves of a token block.
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
        float v = ssq[nb] + __shfl_xor(ssq[nb], 32, 64);
        if (g == 0) sSq[wh][wt * C::WT + nb * 32 + l32] = v;
    }
    __syncthreads();
    if (tid < kBT) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < C::WAVES_H; ++w) t += sSq[w][tid];
        sR[tid] = 1.0f / sqrtf(t / (float)d + eps_row);
    }
    __syncthreads();

    // GELU and the w2 dot product over this wave's hidden units.
    float part[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
        const float r = sR[wt * C::WT + nb * 32 + l32];
        float p = 0.0f;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int j = wh * C::WH + mb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                const float a = fmaf(r, acc[mb][nb][i], sB1[j]);
                p = fmaf(sW2[j], gelu_erf(a), p);
            }
        }
        p += __shfl_xor(p, 32, 64);
        part[nb] = p;
    }
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
        if (g == 0) sPart[wh][wt * C::WT + nb * 32 + l32] = part[nb];
    __syncthreads();

    if (tid < kBT) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < C::WAVES_H; ++w) s += sPart[w][tid];
        s += b2;
        const int64_t row = row0 + tid;
        const bool ok = row < n;
        if (ok) s_out[row] = s;
        sS[tid] = ok ? s * s : 0.0f;
    }
    __syncthreads();
    if (wave == 0) {
        float v = sS[lane];  // kBT == 64: one value per lane, fixed-order tree
        v = tgd::wave_sum(v);
        if (lane == 0) block_ss[blockIdx.x] = v;
    }
}

constexpr int kNormThreads = 256;
constexpr int kNormPerThread = 4;

__global__ __launch_bounds__(kNormThreads) void gate_seqnorm(const float* __restrict__ s_raw,
                                                             const float* __restrict__ block_ss,
                                                             int64_t nblocks, int64_t n, float eps_seq,
                                                             float* __restrict__ s_norm) {
    __shared__ double red[kNormThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    double acc = 0.0;
    for (int64_t b = tid; b < nblocks; b += kNormThreads) acc += (double)block_ss[b];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kNormThreads / 64; ++w) tot += red[w];
    const float rho = (float)sqrt(tot / (double)n + (double)eps_seq);
    const int64_t base = (int64_t)blockIdx.x * kNormThreads * kNormPerThread;
#pragma unroll
    for (int e = 0; e < kNormPerThread; ++e) {
        int64_t i = base + (int64_t)e * kNormThreads + tid;
        if (i < n) s_norm[i] = s_raw[i] / rho;
    }
}

template <int HD>
int launch_gate_hd(const uint16_t* resid, const uint16_t* w1, const uint16_t* b1, const uint16_t* w2,
                   float b2, int64_t n, int d, float eps_row, float* s_out, float* block_ss,
                   hipStream_t s) {
    const int64_t nb = tgi::gate_blocks(n);
    hipLaunchKernelGGL(gate_mlp<HD>, dim3((unsigned)nb), dim3(kThreads), 0, s, resid, w1, b1, w2, b2, n,
                       d, eps_row, s_out, block_ss);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace

namespace tgi {

int launch_gate_score(const uint16_t* resid, const uint16_t* w1, const uint16_t* b1,
                      const uint16_t* w2, float b2, int64_t n, int d, int hd, float eps_row,
                      float eps_seq, float* score_norm, float* score_raw, void* ws, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    float* block_ss = reinterpret_cast<float*>(ws);
    float* s_out = score_raw ? score_raw : score_norm;
    int rc;
    switch (hd) {
        case 64: rc = launch_gate_hd<64>(resid, w1, b1, w2, b2, n, d, eps_row, s_out, block_ss, s); break;
        case 128: rc = launch_gate_hd<128>(resid, w1, b1, w2, b2, n, d, eps_row, s_out, block_ss, s); break;
        case 256: rc = launch_gate_hd<256>(resid, w1, b1, w2, b2, n, d, eps_row, s_out, block_ss, s); break;
        default: return TG_EUNSUPPORTED;
    }
    if (rc != TG_OK) return rc;
    const int64_t per = (int64_t)kNormThreads * kNormPerThread;
    hipLaunchKernelGGL(gate_seqnorm, dim3((unsigned)((n + per - 1) / per)), dim3(kNormThreads), 0, s, s_out,
                       block_ss, gate_blocks(n), n, eps_seq, score_norm);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace tgi
