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
// takes 2 rows of one head: lane (r, c) holds row r, columns c*dk/32 ..
// +dk/32 in registers; the two row dot products reduce over the row's 32
// lanes (four DPP steps and one cross-row swap).  Tokens are taken in order (the recurrence is sequential),
// in unrolled groups of eight: the group's LDS reads of q, k, v and the gates
// go out together, and one token's output reduction overlaps the next one's
// state chain.  fp32 state and arithmetic; deterministic.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

constexpr int kWaves = 4;   // waves per workgroup (consecutive row pairs of one head)
constexpr int kChunk = 32;  // tokens per LDS stage
constexpr int kGroup = 8;   // tokens per unrolled group

#define TG_LDS __attribute__((address_space(3)))
typedef unsigned int lu2 __attribute__((ext_vector_type(2)));  // LDS-side uint2

// Sum over the 32 lanes of a half-wave, in every one of them: swap within
// quads (1,0,3,2), then (2,3,0,1), then the mirrored lane of the other quad
// of each 8-lane half-row, then the mirrored lane of the other half of the
// 16-lane row, then the lane of the other row (lane ^ 16, gfx950 swap).
__device__ __forceinline__ float sum32(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct loads from memory into LDS: `SIZE` bytes per lane from base + voff
// land at lds + SIZE * lane, through a raw buffer resource covering `bytes`
// bytes, so offsets at or past the end (tokens past the last) read as zero.
constexpr int kBufferWord3 = 0x00020000;

template <int SIZE>
__device__ __forceinline__ void lds_load(const void* base, uint32_t bytes, TG_LDS uint8_t* lds, uint32_t voff) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
    if constexpr (SIZE == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TG_LDS void*)lds, 16, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TG_LDS void*)lds, 4, voff, 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define TG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// A workgroup: kWaves waves on 2 * kWaves consecutive rows of one head's
// state; lane (r, c) = (lane / 32, lane % 32) of wave w holds row
// row0 + 2 w + r, columns c * dk/32 .. +dk/32.  Tokens go through LDS in
// chunks of kChunk, two stages: the k and q rows, the workgroup's v values
// and the two gates of the next chunk load while this one is applied.
template <int DK, int DV>
struct Gdn {
    static constexpr int CPL = DK / 32;                   // state columns per lane
    static constexpr int ROWS = 2 * kWaves;               // state rows per workgroup
    static constexpr int KQ = kChunk * DK * 2;            // bytes of k (or q) rows per chunk
    static constexpr int VB = kChunk * ROWS * 2;          // bytes of v per chunk
    static constexpr int STAGE = 2 * KQ + VB + 2 * kChunk * 4;
    static_assert(KQ % (64 * kWaves * 16) == 0, "k/q chunk in whole direct loads");
    static_assert(VB == 2 * 64 * 4, "v chunk in one 4-byte load per lane of the first two waves");
};

template <int DK, int DV>
__global__ __launch_bounds__(64 * kWaves) void gdn_scan(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v,
                                                        const float* __restrict__ alpha,
                                                        const float* __restrict__ beta,
                                                        const float* state_in, int64_t n, int hk, int hv,
                                                        float* __restrict__ out,
                                                        float* state_out) {  // state_out may be state_in
    using C = Gdn<DK, DV>;
    constexpr int CPL = C::CPL;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::STAGE];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h = blockIdx.x / (DV / C::ROWS), row0 = (blockIdx.x % (DV / C::ROWS)) * C::ROWS;
    const int hq = h / (hv / hk);
    const int r = lane >> 5, c = lane & 31;
    const int row = row0 + 2 * w + r;
    float S[CPL];
    const int64_t soff = ((int64_t)h * DV + row) * DK + c * CPL;
#pragma unroll
    for (int i = 0; i < CPL; ++i) S[i] = state_in ? state_in[soff + i] : 0.0f;

    const uint32_t qk_bytes = (uint32_t)n * (uint32_t)hk * DK * 2u;
    const uint32_t v_bytes = (uint32_t)n * (uint32_t)hv * DV * 2u;
    const uint32_t g_bytes = (uint32_t)n * (uint32_t)hv * 4u;
    TG_LDS uint8_t* st0 = (TG_LDS uint8_t*)smem;
    TG_LDS uint8_t* st1 = st0 + C::STAGE;

    // chunk ch into a stage: k rows, q rows (token-major, 2 dk bytes each),
    // v (kChunk x ROWS bf16), alpha (kChunk fp32), beta (kChunk fp32)
    auto issue = [&](int64_t ch, TG_LDS uint8_t* __restrict__ sb) {
        const int64_t t0 = ch * kChunk;
#pragma unroll
        for (int it = 0; it < C::KQ / (64 * kWaves * 16); ++it) {
            const int e = it * 64 * kWaves + tid;  // 16-byte piece of the chunk
            const int tt = e / (DK / 8), p = e % (DK / 8);
            const uint32_t go = ((uint32_t)(t0 + tt) * (uint32_t)hk + (uint32_t)hq) * (DK * 2u) + 16u * p;
            lds_load<16>(k, qk_bytes, sb + it * 64 * kWaves * 16 + w * 1024, go);
            lds_load<16>(q, qk_bytes, sb + C::KQ + it * 64 * kWaves * 16 + w * 1024, go);
        }
        if (w < 2) {  // v: thread tid -> token tid / 4, 4-byte word tid % 4 of the ROWS values
            const int tt = tid / (C::ROWS / 2), wd = tid % (C::ROWS / 2);
            const uint32_t go = ((uint32_t)(t0 + tt) * (uint32_t)hv + (uint32_t)h) * (DV * 2u) + row0 * 2u + 4u * wd;
            lds_load<4>(v, v_bytes, sb + 2 * C::KQ + w * 256, go);
        }
        if (w == 0 && lane < kChunk) {
            const uint32_t go = ((uint32_t)(t0 + lane) * (uint32_t)hv + (uint32_t)h) * 4u;
            lds_load<4>(alpha, g_bytes, sb + 2 * C::KQ + C::VB, go);
            lds_load<4>(beta, g_bytes, sb + 2 * C::KQ + C::VB + kChunk * 4, go);
        }
    };
    auto step = [&](int64_t ch, const TG_LDS uint8_t* __restrict__ cb, TG_LDS uint8_t* __restrict__ nb,
                    int64_t nch) {
        // This wave's share of the chunk is in LDS.  Loads complete in issue
        // order and the one memory operation issued after them is the
        // previous chunk's output store, which may stay in flight.
        if (ch == 0) {
            TG_WAIT_VMCNT(0);
        } else {
            TG_WAIT_VMCNT(1);
        }
        // ... and every wave's; the other stage is free again.  A bare barrier
        // (with a compiler memory fence, so no LDS read moves above it): a
        // workgroup fence here would also wait for the output store.
        asm volatile("s_barrier" ::: "memory");
        if (ch + 1 < nch) issue(ch + 1, nb);
        asm volatile("" ::: "memory");  // the chunk's output store stays behind these loads
        const int64_t t0 = ch * kChunk;
        const int tn = n - t0 < kChunk ? (int)(n - t0) : kChunk;
        const TG_LDS uint16_t* kc = (const TG_LDS uint16_t*)cb;
        const TG_LDS uint16_t* qc = (const TG_LDS uint16_t*)(cb + C::KQ);
        const TG_LDS uint16_t* vc = (const TG_LDS uint16_t*)(cb + 2 * C::KQ);
        const TG_LDS float* ac = (const TG_LDS float*)(cb + 2 * C::KQ + C::VB);
        const TG_LDS float* bc = ac + kChunk;
        float ov = 0.0f;  // lane c keeps the output of token t0 + c of its row
        // one token; `live` is false only past the last token of a short chunk
        // (uniform over the workgroup), where the state is left as it is
        auto token = [&](int tt, bool live) {
            float kf[CPL], qf[CPL];
            uint32_t kw[CPL / 2], qw[CPL / 2];
            if constexpr (CPL == 4) {
                const lu2 kk = *(const TG_LDS lu2*)(kc + tt * DK + c * CPL);
                const lu2 qq = *(const TG_LDS lu2*)(qc + tt * DK + c * CPL);
                kw[0] = kk.x, kw[1] = kk.y, qw[0] = qq.x, qw[1] = qq.y;
            } else {
                kw[0] = *(const TG_LDS uint32_t*)(kc + tt * DK + c * CPL);
                qw[0] = *(const TG_LDS uint32_t*)(qc + tt * DK + c * CPL);
            }
#pragma unroll
            for (int e = 0; e < CPL / 2; ++e) {
                kf[2 * e] = tgd::bf16lo(kw[e]), kf[2 * e + 1] = tgd::bf16hi(kw[e]);
                qf[2 * e] = tgd::bf16lo(qw[e]), qf[2 * e + 1] = tgd::bf16hi(qw[e]);
            }
            const float vr = __uint_as_float((uint32_t)vc[tt * C::ROWS + 2 * w + r] << 16);
            const float a = ac[tt], b = bc[tt];
            float u = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) u = fmaf(S[i], kf[i], u);
            u = sum32(u);
            const float wv = b * (vr - a * u);
            float o = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const float si = fmaf(a, S[i], wv * kf[i]);
                S[i] = live ? si : S[i];
                o = fmaf(S[i], qf[i], o);
            }
            o = sum32(o);
            ov = c == tt ? o : ov;
        };
        // groups of kGroup tokens with a fixed trip count, so that the group's
        // LDS reads are issued ahead of the chain of state updates
        if (tn == kChunk) {
            for (int g = 0; g < kChunk; g += kGroup) {
#pragma unroll
                for (int j = 0; j < kGroup; ++j) token(g + j, true);
            }
        } else {
            for (int g = 0; g < tn; g += kGroup) {
#pragma unroll
                for (int j = 0; j < kGroup; ++j) token(g + j, g + j < tn);
            }
        }
        if (c < tn) out[((t0 + c) * hv + h) * DV + row] = ov;
    };
    const int64_t nch = (n + kChunk - 1) / kChunk;
    if (nch > 0) issue(0, st0);
    for (int64_t ch = 0; ch < nch; ch += 2) {
        step(ch, st0, st1, nch);
        if (ch + 1 < nch) step(ch + 1, st1, st0, nch);
    }
    if (state_out) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) state_out[soff + i] = S[i];
    }
}

template <int DK, int DV>
int launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha, const float* beta,
           const float* state_in, int64_t n, int hk, int hv, float* out, float* state_out, hipStream_t s) {
    hipLaunchKernelGGL((gdn_scan<DK, DV>), dim3((unsigned)(hv * (DV / Gdn<DK, DV>::ROWS))), dim3(64 * kWaves), 0, s,
                       q, k, v, alpha, beta, state_in, n, hk, hv, out, state_out);
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
