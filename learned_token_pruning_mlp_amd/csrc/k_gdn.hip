// k_gdn.hip -- the gated delta rule over the kept tokens (recurrent mixer of
// the hybrid backbone).
//
// In the hybrid backbone most layers are Gated-DeltaNet mixers; above the gate
// the recurrent mixers run on the kept tokens only, while the lower layers'
// recurrent state has read every token (fluxbbs.com TokenGate article,
// section on the hybrid architecture; aiwillknow.com, section on the two
// kinds of state in hybrid models).  The mixer's core is the gated delta rule
// (Yang, Kautz and Hatamizadeh, "Gated Delta Networks", 2024): per v head,
// with S in R^{dv x dk},
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t,
// computed row by row as
//   u = S_{t-1}[r,:] . k_t,  S_t[r,:] = alpha_t S_{t-1}[r,:] + beta_t (v_t[r] - alpha_t u) k_t,
//   o_t[r] = S_t[r,:] . q_t.
// Rows of S evolve independently given the shared k, q and gates, so a wave
// takes 8 rows of one head: lane (r, c) holds row r, columns c*dk/8 .. +dk/8
// in registers; the two row dot products reduce over the row's 8 lanes with
// three DPP steps.  Tokens are taken in order (the recurrence is sequential);
// the next token's q, k, v and gates are loaded while the current one is
// applied.  fp32 state and arithmetic; deterministic.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::u32x4;

// Sum over the 8 lanes of a half-row (lanes 8m .. 8m+7), in every one of them:
// swap within quads (1,0,3,2), then (2,3,0,1), then the mirrored lane of the
// other quad of the half-row.
__device__ __forceinline__ float sum8(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    return x;
}

template <int CPL>
struct Tok {
    u32x4 k[CPL / 8], q[CPL / 8];
    float v, a, b;
};

template <int DK, int DV>
__global__ __launch_bounds__(64) void gdn_scan(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                               const uint16_t* __restrict__ v, const float* __restrict__ alpha,
                                               const float* __restrict__ beta, const float* __restrict__ state_in,
                                               int64_t n, int hk, int hv, float* __restrict__ out,
                                               float* __restrict__ state_out) {
    constexpr int CPL = DK / 8;  // state columns per lane
    const int lane = threadIdx.x;
    const int h = blockIdx.x / (DV / 8), rb = blockIdx.x % (DV / 8);
    const int hq = h / (hv / hk);
    const int r = lane >> 3, c = lane & 7;
    const int row = rb * 8 + r;
    float S[CPL];
    const int64_t soff = ((int64_t)h * DV + row) * DK + c * CPL;
#pragma unroll
    for (int i = 0; i < CPL; ++i) S[i] = state_in ? state_in[soff + i] : 0.0f;

    auto load = [&](int64_t t, Tok<CPL>& x) {
        const int64_t qo = (t * hk + hq) * DK + c * CPL;
#pragma unroll
        for (int p = 0; p < CPL / 8; ++p) {
            x.k[p] = *reinterpret_cast<const u32x4*>(k + qo + 8 * p);
            x.q[p] = *reinterpret_cast<const u32x4*>(q + qo + 8 * p);
        }
        x.v = tgd::bf16lo(v[(t * hv + h) * DV + row]);
        x.a = alpha[t * hv + h];
        x.b = beta[t * hv + h];
    };
    Tok<CPL> cur{}, nxt{};
    if (n > 0) load(0, cur);
    for (int64_t t = 0; t < n; ++t) {
        if (t + 1 < n) load(t + 1, nxt);
        float kf[CPL], qf[CPL];
#pragma unroll
        for (int p = 0; p < CPL / 8; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[8 * p + 2 * e] = tgd::bf16lo(cur.k[p][e]);
                kf[8 * p + 2 * e + 1] = tgd::bf16hi(cur.k[p][e]);
                qf[8 * p + 2 * e] = tgd::bf16lo(cur.q[p][e]);
                qf[8 * p + 2 * e + 1] = tgd::bf16hi(cur.q[p][e]);
            }
        float u0 = 0.0f, u1 = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; i += 2) {
            u0 = fmaf(S[i], kf[i], u0);
            u1 = fmaf(S[i + 1], kf[i + 1], u1);
        }
        const float u = sum8(u0 + u1);
        const float w = cur.b * (cur.v - cur.a * u);
        float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; i += 2) {
            S[i] = fmaf(cur.a, S[i], w * kf[i]);
            S[i + 1] = fmaf(cur.a, S[i + 1], w * kf[i + 1]);
            o0 = fmaf(S[i], qf[i], o0);
            o1 = fmaf(S[i + 1], qf[i + 1], o1);
        }
        const float o = sum8(o0 + o1);
        if (c == 0) out[(t * hv + h) * DV + row] = o;
        cur = nxt;
    }
    if (state_out) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) state_out[soff + i] = S[i];
    }
}

template <int DK, int DV>
int launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha, const float* beta,
           const float* state_in, int64_t n, int hk, int hv, float* out, float* state_out, hipStream_t s) {
    hipLaunchKernelGGL((gdn_scan<DK, DV>), dim3((unsigned)(hv * (DV / 8))), dim3(64), 0, s, q, k, v, alpha, beta,
                       state_in, n, hk, hv, out, state_out);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace

namespace tgi {

int launch_gated_delta_rule(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha,
                            const float* beta, const float* state_in, int64_t n, int hk, int hv, int dk, int dv,
                            float* out, float* state_out, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (dk == 128 && dv == 128) return launch<128, 128>(q, k, v, alpha, beta, state_in, n, hk, hv, out, state_out, s);
    if (dk == 128 && dv == 64) return launch<128, 64>(q, k, v, alpha, beta, state_in, n, hk, hv, out, state_out, s);
    if (dk == 64 && dv == 128) return launch<64, 128>(q, k, v, alpha, beta, state_in, n, hk, hv, out, state_out, s);
    if (dk == 64 && dv == 64) return launch<64, 64>(q, k, v, alpha, beta, state_in, n, hk, hv, out, state_out, s);
    return TG_EUNSUPPORTED;
}

}  // namespace tgi
