// k_gate_bwd.hip -- backward of the gate's scoring network.
//
// The gate is trained end to end through the attention bias of the kept
// tokens (fluxbbs.com TokenGate article, sections on where the gate sits and
// on token-gated attention; slinene.github.io digest, method key points;
// aiwillknow.com, Figure 1(a)(b)).  The forward is
//   r_i = (mean_k h_ik^2 + eps_row)^(-1/2),  z_ij = h_i . W1_j,
//   a_ij = r_i z_ij + b1_j,  u_ij = a_ij Phi(a_ij),  s_i = sum_j w2_j u_ij + b2,
//   rho = (mean_i s_i^2 + eps_seq)^(1/2),  shat_i = s_i / rho,
// and given dshat (the kept tokens' score gradients, zero elsewhere):
//   ds_i = dshat_i / rho - s_i (sum_m dshat_m s_m) / (n rho^3)
//   dw2_j = sum_i ds_i u_ij,  db2 = sum_i ds_i,
//   da_ij = ds_i w2_j (Phi(a_ij) + a_ij phi(a_ij)),  db1_j = sum_i da_ij,
//   dz_ij = r_i da_ij,  dW1 = dz^T h,
//   dh_i = dz_i W1 - (sum_j da_ij z_ij) r_i^3 h_i / d.
//
// Kernels: gbw_clear + gbw_scalars scatter dshat and form 1/rho and the
// sequence-norm coefficient (fixed-order fp64 sums); Z = h W1^T is a rocBLAS
// GEMM (fp32 out); gbw_rows takes 16 rows per wave (a lane holds hd/64
// hidden units and d/512 pieces of the row), writes dz (bf16, the operand of
// the two gradient GEMMs), the row-norm term of dh (fp32) and per-wave
// partials of dw2, db1 and db2; rocBLAS then adds dz W1 into dh (beta = 1)
// and forms dW1 = dz^T h as a batch of token chunks (gbw_sum_parts adds the
// chunk partials in order); gbw_reduce sums the other partials in a fixed
// order.
// No float atomics anywhere (the rocBLAS handle has atomics disabled).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::u32x4;

constexpr int kRowsPerWave = tgi::kGateBwdRowsPerWave;
constexpr int kWaves = 4;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kInvSqrt2 = 0.70710678118654752440f;
constexpr float kInvSqrt2Pi = 0.39894228040143267794f;

// erf by the rational approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7 for x >= 0),
// extended to x < 0 by oddness; exp(-x^2) is taken as exp2(-x^2 log2 e).
__device__ __forceinline__ float erf_as(float x) {
    const float ax = fabsf(x);
    const float t = 1.0f / (1.0f + 0.3275911f * ax);
    const float poly =
        t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float e = 1.0f - poly * __builtin_amdgcn_exp2f(-ax * ax * kLog2e);
    return x < 0.0f ? -e : e;
}

__global__ __launch_bounds__(256) void gbw_clear(float* __restrict__ dsh, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dsh[i] = 0.0f;
}

// One workgroup: scatters dshat, sums s^2 over all tokens and dshat s over
// the kept ones (fp64, fixed order); sc = {1/rho, (sum dshat s) / (n rho^3)}.
// Kept indices outside [0, n) are skipped.
__global__ __launch_bounds__(1024) void gbw_scalars(const float* __restrict__ s, int64_t n,
                                                    const float* __restrict__ dsk, const int32_t* __restrict__ idx,
                                                    int64_t k, float eps_seq, float* __restrict__ dsh,
                                                    float* __restrict__ sc) {
    __shared__ double red[2][16];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    double ss = 0.0, cd = 0.0;
    for (int64_t i = tid; i < n; i += 1024) ss += (double)s[i] * (double)s[i];
    for (int64_t t = tid; t < k; t += 1024) {
        const int32_t i = idx[t];
        if (i < 0 || (int64_t)i >= n) continue;
        dsh[i] = dsk[t];
        cd += (double)dsk[t] * (double)s[i];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        ss += __shfl_xor(ss, o, 64);
        cd += __shfl_xor(cd, o, 64);
    }
    if (lane == 0) {
        red[0][w] = ss;
        red[1][w] = cd;
    }
    __syncthreads();
    if (tid == 0) {
        double a = 0.0, b = 0.0;
        for (int i = 0; i < 16; ++i) {
            a += red[0][i];
            b += red[1][i];
        }
        const double rho = sqrt(a / (double)n + (double)eps_seq);
        sc[0] = (float)(1.0 / rho);
        sc[1] = (float)(b / ((double)n * rho * rho * rho));
    }
}

// kRowsPerWave rows per wave.  Lane L holds hidden units L*UPL .. +UPL-1 and
// the 16-byte pieces L, L+64, ... of the residual row.
template <int HD, int PPL>
__global__ __launch_bounds__(64 * kWaves) void gbw_rows(
    const uint16_t* __restrict__ h, const float* __restrict__ Z, const uint16_t* __restrict__ b1,
    const uint16_t* __restrict__ w2, const float* __restrict__ s, const float* __restrict__ dsh,
    const float* __restrict__ sc, int64_t n, int d, float eps_row, uint16_t* __restrict__ dz,
    float* __restrict__ dh, float* __restrict__ dw2p, float* __restrict__ db1p, float* __restrict__ db2p) {
    constexpr int UPL = HD / 64;  // (PPL: 16-byte pieces of a row per lane, 64-lane passes; d <= 512 * PPL)
    const int lane = threadIdx.x & 63;
    const int64_t wg = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t row0 = wg * kRowsPerWave;
    if (row0 >= n) return;
    const int pieces = d / 8;
    const float inv_rho = sc[0], coef = sc[1];
    float b1v[UPL], w2v[UPL], aw2[UPL], ab1[UPL];
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const int j = lane * UPL + u;
        b1v[u] = b1 ? tgd::bf16lo(b1[j]) : 0.0f;
        w2v[u] = tgd::bf16lo(w2[j]);
        aw2[u] = ab1[u] = 0.0f;
    }
    float ab2 = 0.0f;
    const int64_t rows = n - row0 < kRowsPerWave ? n - row0 : kRowsPerWave;
    // A row's operands: its residual pieces, Z row, dshat and raw score.  The
    // next row's are loaded (its index clamped to the wave's last row, so the
    // loads are unconditional) before this row's outputs are stored; loads
    // and stores complete in issue order, so waiting for them never waits for
    // the previous row's stores.  When the pieces fill PPL 64-lane passes
    // exactly, the piece loads are unconditional too.
    struct RowIn {
        u32x4 hv[PPL];
        float zv[UPL];
        float dsh, s;
    };
    // the row loop, with FULL = (the pieces fill the PPL passes exactly) fixed
    auto run = [&](auto FULL) {
    constexpr bool full = decltype(FULL)::value;
    auto load_row = [&](int64_t i, RowIn& in) {
        if constexpr (full) {
#pragma unroll
            for (int q = 0; q < PPL; ++q) in.hv[q] = *reinterpret_cast<const u32x4*>(h + i * d + 8 * (lane + 64 * q));
        } else {
#pragma unroll
            for (int q = 0; q < PPL; ++q) {
                const int p = lane + 64 * q;
                in.hv[q] = p < pieces ? *reinterpret_cast<const u32x4*>(h + i * d + 8 * p) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < UPL; ++u) in.zv[u] = Z[i * HD + lane * UPL + u];
        in.dsh = dsh[i];
        in.s = s[i];
    };
    auto row_step = [&](int rr, const RowIn& cur, RowIn& nxt) {
        const int64_t i = row0 + rr;
        load_row(row0 + (rr + 1 < rows ? rr + 1 : rr), nxt);
        float ss = 0.0f;
#pragma unroll
        for (int q = 0; q < PPL; ++q) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = tgd::bf16lo(cur.hv[q][e]), hi = tgd::bf16hi(cur.hv[q][e]);
                ss = fmaf(lo, lo, ss);
                ss = fmaf(hi, hi, ss);
            }
        }
        ss = tgd::wave_sum(ss);
        const float r = 1.0f / sqrtf(ss / (float)d + eps_row);
        const float dsi = cur.dsh * inv_rho - cur.s * coef;
        float dr = 0.0f;
        float dzv[UPL];
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const float a = fmaf(r, cur.zv[u], b1v[u]);
            const float Phi = 0.5f * (1.0f + erf_as(a * kInvSqrt2));
            const float phi = kInvSqrt2Pi * __builtin_amdgcn_exp2f(-0.5f * a * a * kLog2e);
            const float da = dsi * w2v[u] * fmaf(a, phi, Phi);
            aw2[u] = fmaf(dsi, a * Phi, aw2[u]);
            ab1[u] += da;
            dr = fmaf(da, cur.zv[u], dr);
            dzv[u] = r * da;
        }
        if constexpr (UPL == 4) {
            *reinterpret_cast<uint2*>(dz + i * HD + lane * 4) =
                uint2{tgd::pack_bf16x2(dzv[0], dzv[1]), tgd::pack_bf16x2(dzv[2], dzv[3])};
        } else if constexpr (UPL == 2) {
            *reinterpret_cast<uint32_t*>(dz + i * HD + lane * 2) = tgd::pack_bf16x2(dzv[0], dzv[1]);
        } else {
            dz[i * HD + lane] = (uint16_t)(tgd::pack_bf16x2(dzv[0], 0.0f) & 0xffffu);
        }
        dr = tgd::wave_sum(dr);
        const float e = -dr * r * r * r / (float)d;
#pragma unroll
        for (int q = 0; q < PPL; ++q) {
            const int p = lane + 64 * q;
            if (full || p < pieces) {
                float4* o = reinterpret_cast<float4*>(dh + i * d + 8 * p);
                o[0] = float4{e * tgd::bf16lo(cur.hv[q][0]), e * tgd::bf16hi(cur.hv[q][0]),
                              e * tgd::bf16lo(cur.hv[q][1]), e * tgd::bf16hi(cur.hv[q][1])};
                o[1] = float4{e * tgd::bf16lo(cur.hv[q][2]), e * tgd::bf16hi(cur.hv[q][2]),
                              e * tgd::bf16lo(cur.hv[q][3]), e * tgd::bf16hi(cur.hv[q][3])};
            }
        }
        ab2 += dsi;
    };
    RowIn ra, rb;
    load_row(row0, ra);
    for (int rr = 0; rr < (int)rows; rr += 2) {
        row_step(rr, ra, rb);
        if (rr + 1 < (int)rows) row_step(rr + 1, rb, ra);
    }
    };
    if (pieces == PPL * 64)
        run(std::true_type{});
    else
        run(std::false_type{});
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        dw2p[wg * HD + lane * UPL + u] = aw2[u];
        db1p[wg * HD + lane * UPL + u] = ab1[u];
    }
    if (lane == 0) db2p[wg] = ab2;
}

// Workgroup b < hd: dw2[b]; hd <= b < 2 hd: db1[b - hd]; b == 2 hd: db2.
// Each sums its nw per-wave partials in a fixed order (fp64).
__global__ __launch_bounds__(256) void gbw_reduce(const float* __restrict__ dw2p, const float* __restrict__ db1p,
                                                  const float* __restrict__ db2p, int nw, int hd,
                                                  float* __restrict__ dw2, float* __restrict__ db1,
                                                  float* __restrict__ db2) {
    __shared__ double red[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int b = blockIdx.x;
    double acc = 0.0;
    if (b < hd) {
        for (int i = tid; i < nw; i += 256) acc += (double)dw2p[(int64_t)i * hd + b];
    } else if (b < 2 * hd) {
        for (int i = tid; i < nw; i += 256) acc += (double)db1p[(int64_t)i * hd + (b - hd)];
    } else {
        for (int i = tid; i < nw; i += 256) acc += (double)db2p[i];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) red[w] = acc;
    __syncthreads();
    if (tid == 0) {
        const float v = (float)(red[0] + red[1] + red[2] + red[3]);
        if (b < hd)
            dw2[b] = v;
        else if (b < 2 * hd)
            db1[b - hd] = v;
        else
            *db2 = v;
    }
}

// dW1 = sum of the per-chunk partials, in chunk order.
__global__ __launch_bounds__(256) void gbw_sum_parts(const float4* __restrict__ parts, int nparts, int64_t n4,
                                                     float4* __restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n4) return;
    float4 a = parts[e];
    for (int p = 1; p < nparts; ++p) {
        const float4 b = parts[(int64_t)p * n4 + e];
        a.x += b.x, a.y += b.y, a.z += b.z, a.w += b.w;
    }
    out[e] = a;
}

template <int HD>
int launch_rows(const uint16_t* resid, const uint16_t* b1, const uint16_t* w2, const float* s_raw, int64_t n, int d,
                float eps_row, const tgi::GateBwdWs& ws, float* dresid, hipStream_t st) {
    const int64_t nw = tgi::gate_bwd_waves(n);
    const dim3 grid((unsigned)((nw + kWaves - 1) / kWaves)), block(64 * kWaves);
    // 16-byte pieces of a row per lane: d <= 512 * PPL (the C ABI takes d <= 4096)
    const int pieces = d / 8, ppl = (pieces + 63) / 64;
    if (ppl <= 1)
        hipLaunchKernelGGL((gbw_rows<HD, 1>), grid, block, 0, st, resid, ws.z, b1, w2, s_raw, ws.dsh, ws.sc, n, d,
                           eps_row, ws.dz, dresid, ws.dw2p, ws.db1p, ws.db2p);
    else if (ppl <= 2)
        hipLaunchKernelGGL((gbw_rows<HD, 2>), grid, block, 0, st, resid, ws.z, b1, w2, s_raw, ws.dsh, ws.sc, n, d,
                           eps_row, ws.dz, dresid, ws.dw2p, ws.db1p, ws.db2p);
    else if (ppl <= 4)
        hipLaunchKernelGGL((gbw_rows<HD, 4>), grid, block, 0, st, resid, ws.z, b1, w2, s_raw, ws.dsh, ws.sc, n, d,
                           eps_row, ws.dz, dresid, ws.dw2p, ws.db1p, ws.db2p);
    else
        hipLaunchKernelGGL((gbw_rows<HD, 8>), grid, block, 0, st, resid, ws.z, b1, w2, s_raw, ws.dsh, ws.sc, n, d,
                           eps_row, ws.dz, dresid, ws.dw2p, ws.db1p, ws.db2p);
    return TG_OK;
}

}  // namespace

namespace tgi {

int launch_gate_score_bwd(void* blas, const uint16_t* resid, const uint16_t* w1, const uint16_t* b1,
                          const uint16_t* w2, int64_t n, int d, int hd, float eps_row, float eps_seq,
                          const float* score_raw, const float* dscore_kept, const int32_t* kept_idx, int64_t k,
                          float* dresid, float* dw1, float* db1, float* dw2, float* db2, void* workspace,
                          void* stream) {
    const GateBwdWs ws = gate_bwd_ws(workspace, n, hd, d);
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(gbw_clear, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ws.dsh, n);
    hipLaunchKernelGGL(gbw_scalars, dim3(1), dim3(1024), 0, st, score_raw, n, dscore_kept, kept_idx, k, eps_seq,
                       ws.dsh, ws.sc);
    if (hipGetLastError() != hipSuccess) return TG_EDEVICE;
    // Z [n, hd] = h W1^T (column-major Z^T = W1 . h^T: A = W1 as [d x hd] transposed, B = h as [d x n])
    int rc = gemm_bf16_f32(blas, true, false, hd, (int)n, d, w1, d, resid, d, 0.0f, ws.z, hd, stream);
    if (rc != TG_OK) return rc;
    switch (hd) {
        case 64: rc = launch_rows<64>(resid, b1, w2, score_raw, n, d, eps_row, ws, dresid, st); break;
        case 128: rc = launch_rows<128>(resid, b1, w2, score_raw, n, d, eps_row, ws, dresid, st); break;
        case 256: rc = launch_rows<256>(resid, b1, w2, score_raw, n, d, eps_row, ws, dresid, st); break;
        default: return TG_EUNSUPPORTED;
    }
    if (hipGetLastError() != hipSuccess) return TG_EDEVICE;
    // dh [n, d] += dz W1 (column-major dh^T += W1^T . dz^T: A = W1 as [d x hd], B = dz as [hd x n])
    rc = gemm_bf16_f32(blas, false, false, d, (int)n, hd, w1, d, ws.dz, hd, 1.0f, dresid, d, stream);
    if (rc != TG_OK) return rc;
    // dW1 [hd, d] = dz^T h (column-major dW1^T = h^T . dz: A = h as [d x rows], B = dz as [hd x rows]
    // transposed), split over the tokens: one long-K product would leave most of the chip idle
    const int splits = gate_bwd_splits(n);
    const int64_t chunk = n / splits, rem = n - chunk * splits;
    if (splits == 1 && rem == 0) {
        rc = gemm_bf16_f32(blas, false, true, d, hd, (int)n, resid, d, ws.dz, hd, 0.0f, dw1, d, stream);
        if (rc != TG_OK) return rc;
    } else {
        const int64_t hdd = (int64_t)hd * d;
        rc = gemm_bf16_f32_batched(blas, false, true, d, hd, (int)chunk, resid, d, chunk * d, ws.dz, hd, chunk * hd,
                                   ws.w1p, d, hdd, splits, stream);
        if (rc != TG_OK) return rc;
        int nparts = splits;
        if (rem > 0) {
            const int64_t r0 = chunk * splits;
            rc = gemm_bf16_f32(blas, false, true, d, hd, (int)rem, resid + r0 * d, d, ws.dz + r0 * hd, hd, 0.0f,
                               ws.w1p + (int64_t)splits * hdd, d, stream);
            if (rc != TG_OK) return rc;
            nparts = splits + 1;
        }
        const int64_t n4 = hdd / 4;
        hipLaunchKernelGGL(gbw_sum_parts, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                           reinterpret_cast<const float4*>(ws.w1p), nparts, n4, reinterpret_cast<float4*>(dw1));
    }
    const int nw = (int)gate_bwd_waves(n);
    hipLaunchKernelGGL(gbw_reduce, dim3((unsigned)(2 * hd + 1)), dim3(256), 0, st, ws.dw2p, ws.db1p, ws.db2p, nw, hd,
                       dw2, db1, db2);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace tgi
