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
// between waves.  Operand tiles of 64 d-columns are double-buffered in LDS;
// the next tile's global loads are in flight while the current tile is
// multiplied.  The row sums of squares come from the same LDS tiles.  Each
// workgroup also writes the sum of its scores' squares (fixed order).
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
constexpr int kLd = kKC + 8;                 // padded LDS row (bf16 elements), 144 bytes

template <int HD>
struct Cfg {
    static constexpr int WAVES_H = HD >= 128 ? 4 : 2;  // waves along hidden units
    static constexpr int WAVES_T = 4 / WAVES_H;         // waves along tokens
    static constexpr int WH = HD / WAVES_H;             // hidden units per wave
    static constexpr int WT = kBT / WAVES_T;            // tokens per wave
    static constexpr int MB = WH / 32;                  // 32-row blocks of hidden units
    static constexpr int NB = WT / 32;                  // 32-column blocks of tokens
    static constexpr int H_PIECES = kBT * kKC / 8 / kThreads;  // 16-byte loads per thread
    static constexpr int W_PIECES = HD * kKC / 8 / kThreads;
    static_assert(MB >= 1 && NB >= 1, "tile shape");
};

__device__ __forceinline__ float gelu_erf(float a) {
    return 0.5f * a * (1.0f + erff(a * 0.70710678118654752440f));
}

template <int HD>
__global__ __launch_bounds__(kThreads) void gate_mlp(const uint16_t* __restrict__ resid,
                                                     const uint16_t* __restrict__ w1,
                                                     const uint16_t* __restrict__ b1,
                                                     const uint16_t* __restrict__ w2, float b2,
                                                     int64_t n, int d, float eps_row,
                                                     float* __restrict__ s_out,
                                                     float* __restrict__ block_ss) {
    using C = Cfg<HD>;
    __shared__ __attribute__((aligned(16))) uint16_t sH[2][kBT * kLd];
    __shared__ __attribute__((aligned(16))) uint16_t sW[2][HD * kLd];
    __shared__ float sB1[HD], sW2[HD];
    __shared__ float sSq[C::WAVES_H][kBT];
    __shared__ float sPart[C::WAVES_H][kBT];
    __shared__ float sR[kBT];
    __shared__ float sS[kBT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wh = wave % C::WAVES_H, wt = wave / C::WAVES_H;
    const int l32 = lane & 31, g = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.x * kBT;

    for (int j = tid; j < HD; j += kThreads) {
        sB1[j] = b1 ? tgd::bf16lo(b1[j]) : 0.0f;
        sW2[j] = tgd::bf16lo(w2[j]);
    }

    u32x4 hreg[C::H_PIECES], wreg[C::W_PIECES];
    auto load_tile = [&](int c) {
        const int col0 = c * kKC;
#pragma unroll
        for (int r = 0; r < C::H_PIECES; ++r) {
            int p = tid + kThreads * r, row = p >> 3, col = (p & 7) * 8;
            int64_t gr = row0 + row;
            hreg[r] = gr < n ? *reinterpret_cast<const u32x4*>(resid + gr * d + col0 + col) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < C::W_PIECES; ++r) {
            int p = tid + kThreads * r, row = p >> 3, col = (p & 7) * 8;
            wreg[r] = *reinterpret_cast<const u32x4*>(w1 + (int64_t)row * d + col0 + col);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int r = 0; r < C::H_PIECES; ++r) {
            int p = tid + kThreads * r, row = p >> 3, col = (p & 7) * 8;
            *reinterpret_cast<u32x4*>(&sH[buf][row * kLd + col]) = hreg[r];
        }
#pragma unroll
        for (int r = 0; r < C::W_PIECES; ++r) {
            int p = tid + kThreads * r, row = p >> 3, col = (p & 7) * 8;
            *reinterpret_cast<u32x4*>(&sW[buf][row * kLd + col]) = wreg[r];
        }
    };

    f32x16 acc[C::MB][C::NB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = f32x16{};
    float ssq[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) ssq[nb] = 0.0f;

    const int nchunks = d / kKC;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        if (c + 1 < nchunks) load_tile(c + 1);
        const uint16_t* tH = sH[buf];
        const uint16_t* tW = sW[buf];
#pragma unroll
        for (int s = 0; s < kKC / 16; ++s) {
            const int kof = s * 16 + g * 8;
            u32x4 a[C::MB], b[C::NB];
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
                a[mb] = *reinterpret_cast<const u32x4*>(&tW[(wh * C::WH + mb * 32 + l32) * kLd + kof]);
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
                b[nb] = *reinterpret_cast<const u32x4*>(&tH[(wt * C::WT + nb * 32 + l32) * kLd + kof]);
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = tgd::mfma32(a[mb], b[nb], acc[mb][nb]);
            // row sums of squares: the waves sharing a token block split the k-steps
            if (s % C::WAVES_H == wh) {
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float lo = tgd::bf16lo(b[nb][q]), hi = tgd::bf16hi(b[nb][q]);
                        ssq[nb] = fmaf(lo, lo, ssq[nb]);
                        ssq[nb] = fmaf(hi, hi, ssq[nb]);
                    }
                }
            }
        }
        if (c + 1 < nchunks) store_tile(buf ^ 1);
        __syncthreads();
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
