// k_gate.hip -- gate scoring network and sequence RMSNorm of the scores.
//
// At the gate layer a small MLP reads each token's normalised post-attention
// residual and returns one scalar; the scores are then RMSNorm-normalised
// along the sequence (fluxbbs.com TokenGate article, section on where the
// gate sits; slinene.github.io digest, method key points; aiwillknow.com,
// Figure 1(a)(b)).
//
// Kernel 1 (gate_mlp): one workgroup takes 64 residual rows, or 128 once the
// prompt still gives every CU a workgroup that way (each W1 tile read from L2
// then serves twice the rows); eight waves for 256 hidden units, two per
// SIMD, so one wave's load latency hides behind the other's products; four
// below.  The residual
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

#include <mutex>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

using tgd::f32x16;
using tgd::u32x4;

constexpr int kKC = 64;  // d-columns per LDS tile

// HD hidden units, BT residual rows per workgroup (64, or 128 on prompts long
// enough to give every CU a workgroup: each W1 tile read from L2 then serves
// twice the rows).
template <int HD, int BT>
struct Cfg {
    // 256 hidden units: eight waves (two per SIMD, so one wave's LDS and
    // direct-load latency hides behind the other's products); fewer: four
    static constexpr int WAVES = HD >= 256 ? 8 : 4;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WAVES_H = HD >= 128 ? 4 : 2;  // waves along hidden units
    static constexpr int WAVES_T = WAVES / WAVES_H;     // waves along tokens
    static constexpr int WH = HD / WAVES_H;             // hidden units per wave
    static constexpr int WT = BT / WAVES_T;             // tokens per wave
    static constexpr int MB = WH / 32;                  // 32-row blocks of hidden units
    static constexpr int NB = WT / 32;                  // 32-column blocks of tokens
    static_assert(MB >= 1 && NB >= 1, "tile shape");
};

// GELU(a) = a * Phi(a) = a/2 * (1 + erf(a / sqrt 2)).  erf by the rational
// approximation of Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (|error| <= 1.5e-7 for x >= 0; odd extension):
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x).
// With E = erf(|a| / sqrt 2) and erf odd, 2 GELU(a) = a + |a| E, which is
// what this returns (the caller folds in the 1/2); exp(-x^2) with
// x^2 = a^2 / 2 is exp2(a * (a * -log2(e)/2)).  Over the 256 hidden units of a
// score this moves the normalised score by about 1e-5 at most.
__device__ __forceinline__ float gelu2_erf(float a) {
    constexpr float p = 0.3275911f;
    constexpr float a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f, a4 = -1.453152027f,
                    a5 = 1.061405429f;
    constexpr float kHalfLog2e = 0.72134752044448170368f;  // log2(e) / 2
    const float ax = fabsf(a);
    const float t = __builtin_amdgcn_rcpf(fmaf(p * 0.70710678118654752440f, ax, 1.0f));
    const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
    const float e = __builtin_amdgcn_exp2f(a * (a * -kHalfLog2e));
    return fmaf(ax, fmaf(-poly, e, 1.0f), a);
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

// Fourth word of a raw buffer resource on gfx9-family parts: 32-bit data
// format, no swizzle; with a zero stride, offsets at or past num_records read
// as zero.
constexpr int kBufferWord3 = 0x00020000;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over `bytes` bytes from base (zero stride).
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{(int32_t)(uint32_t)a, (int32_t)((uint32_t)(a >> 32) & 0xffffu), bytes, kBufferWord3};
}

// Direct load of 16 bytes per lane from the resource at voff + soff into LDS
// at lds + 16 * lane.  Issued from inline assembly so the compiler does not
// track these LDS writes: it would otherwise make the operand reads of one
// stage wait for the loads in flight into the others.  The instruction writes
// no register; the tile loop orders it with explicit vector-memory waits and
// the workgroup barrier.
// (m0 is set right before each use of it, so clobbering it here is safe.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void buffer_to_lds16(i32x4 rs, const TG_LDS uint8_t* lds, uint32_t voff, uint32_t soff) {
    const uint32_t m = (uint32_t)(uintptr_t)lds;
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(m), "v"(voff), "s"(rs), "s"(soff)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define TG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

template <int HD, int BT>
__global__ __launch_bounds__((Cfg<HD, BT>::THREADS)) void gate_mlp(const uint16_t* __restrict__ resid,
                                                     const uint16_t* __restrict__ w1,
                                                     const uint16_t* __restrict__ b1,
                                                     const uint16_t* __restrict__ w2, float b2,
                                                     int64_t n, int d, float eps_row,
                                                     float* __restrict__ s_out,
                                                     float* __restrict__ block_ss) {
    using C = Cfg<HD, BT>;
    constexpr int kBT = BT;
    constexpr int H_BYTES = kBT * kKC * 2;            // residual tile: BT rows x 128 bytes
    constexpr int W_BYTES = HD * kKC * 2;             // W1 tile: HD rows x 128 bytes
    constexpr int STAGE = H_BYTES + W_BYTES;
    constexpr int H_LOADS = H_BYTES / 1024 / C::WAVES;  // 1 KB direct-load instructions per wave
    constexpr int W_LOADS = W_BYTES / 1024 / C::WAVES;
    static_assert(H_LOADS >= 1 && H_BYTES % (1024 * C::WAVES) == 0 && W_BYTES % (1024 * C::WAVES) == 0, "loads");
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

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
    const int wh = wave % C::WAVES_H, wt = wave / C::WAVES_H;
    const int l32 = lane & 31, g = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.x * kBT;
    const int nchunks = d / kKC;

    for (int j = tid; j < HD; j += C::THREADS) {
        sB1[j] = b1 ? tgd::bf16lo(b1[j]) : 0.0f;
        sW2[j] = 0.5f * tgd::bf16lo(w2[j]);
    }

    // Direct loads of one 64-column tile into LDS, through buffer resources:
    // each wave instruction fills one 1 KB block = 8 rows of 128 bytes; lane l
    // writes slot l%8 of row l/8 with the piece (l%8) ^ swz8(row).  A lane's
    // byte offset within the rows is fixed for the kernel and the tile start is
    // a scalar offset.  Residual rows past n repeat row n-1 (their scores are
    // never written).  The residual blocks of a tile come first, then W1's.
    const int rows_ok = (int)min((int64_t)kBT, n - row0);
    const uint16_t* rbase = resid + row0 * d;
    const i32x4 r_rs = buffer_rsrc(rbase, rows_ok * d * 2);
    const i32x4 w_rs = buffer_rsrc(w1, HD * d * 2);
    uint32_t voff[VM_PER_TILE];
#pragma unroll
    for (int r = 0; r < VM_PER_TILE; ++r) {
        const int slot = lane & 7;
        const int blk = (r < H_LOADS ? r : r - H_LOADS) * C::WAVES + wave, row = blk * 8 + (lane >> 3);
        const int src_row = r < H_LOADS ? min(row, rows_ok - 1) : row;
        voff[r] = (uint32_t)(src_row * d + 8 * (slot ^ swz8(row))) * 2u;
    }
    // instructions [i0, i1) of the tile's direct loads
    auto issue_part = [&](int c, uint8_t* __restrict__ stg, int i0, int i1) {
        const int soff = c * kKC * 2;
#pragma unroll
        for (int r = 0; r < VM_PER_TILE; ++r) {
            if (r < i0 || r >= i1) continue;
            if (r < H_LOADS)
                buffer_to_lds16(r_rs, (TG_LDS uint8_t*)stg + (r * C::WAVES + wave) * 1024, voff[r], soff);
            else
                buffer_to_lds16(w_rs, (TG_LDS uint8_t*)stg + H_BYTES + ((r - H_LOADS) * C::WAVES + wave) * 1024, voff[r],
                                soff);
        }
    };
    auto issue = [&](int c, uint8_t* __restrict__ stg) { issue_part(c, stg, 0, VM_PER_TILE); };

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
    constexpr int NOP = C::NB + C::MB;  // operand reads per k-step
    uint32_t roff[NOP];
    int rswz[NOP];
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

    // One tile: wait for its loads (the next tile's stay in flight); the
    // barrier also means every wave finished the previous step, so the loads
    // two tiles ahead can go into the stage it read; then all operand reads of
    // the tile, and its products with those loads in between.  k-step s of half-wave g reads piece 2s+g of
    // a row.  The current and the ahead stage are distinct restrict pointers
    // of one scope.
    auto step = [&](int c, const uint8_t* __restrict__ cur, uint8_t* __restrict__ ahead) {
        if (c + 1 < nchunks) {
            TG_WAIT_VMCNT(VM_PER_TILE);
        } else {
            TG_WAIT_VMCNT(0);
        }
        // barrier that the compiler also treats as a memory fence for its own
        // scheduling (no LDS read moves above it)
        asm volatile("s_barrier" ::: "memory");
        const bool more = c + 2 < nchunks;
        u32x4 op[kKC / 16][NOP];
#pragma unroll
        for (int s = 0; s < kKC / 16; ++s)
#pragma unroll
            for (int i = 0; i < NOP; ++i)
                op[s][i] = *reinterpret_cast<const u32x4*>(cur + roff[i] + 16 * ((2 * s + g) ^ rswz[i]));
        constexpr int KS = kKC / 16;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = tgd::mfma32(op[s][C::NB + mb], op[s][nb], acc[mb][nb]);
            // the loads two tiles ahead go out in slices between the k-steps,
            // so the address unit works while the matrix cores do
            if (more) {
                constexpr int per = (VM_PER_TILE + KS - 1) / KS;
                issue_part(c + 2, ahead, s * per, (s + 1) * per);
            }
            // row sums of squares: the waves sharing a token block split the k-steps
            if (s % C::WAVES_H == wh) {
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float lo = tgd::bf16lo(op[s][nb][q]), hi = tgd::bf16hi(op[s][nb][q]);
                        ssq[nb] = fmaf(lo, lo, ssq[nb]);
                        ssq[nb] = fmaf(hi, hi, ssq[nb]);
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

    // GELU and the w2 dot product over this wave's hidden units (sW2 holds
    // w2 / 2, the factor that gelu2_erf leaves out).
    float part[C::NB];
    float b1r[C::MB][16], w2r[C::MB][16];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = wh * C::WH + mb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            b1r[mb][i] = sB1[j];
            w2r[mb][i] = sW2[j];
        }
    }
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
        const float r = sR[wt * C::WT + nb * 32 + l32];
        float p = 0.0f;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) p = fmaf(w2r[mb][i], gelu2_erf(fmaf(r, acc[mb][nb][i], b1r[mb][i])), p);
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
        float v = sS[lane];  // one or two values per lane, fixed-order tree
        if constexpr (kBT == 128) v += sS[lane + 64];
        v = tgd::wave_sum(v);
        if (lane == 0) block_ss[blockIdx.x] = v;
    }
}

constexpr int kNormThreads = 256;
constexpr int kNormPerThread = 4;

__global__ __launch_bounds__(kNormThreads) void gate_seqnorm(const float* s_raw,
                                                             const float* __restrict__ block_ss,
                                                             int64_t nblocks, int64_t n, float eps_seq,
                                                             float* s_norm) {
    static_assert(kNormThreads == tgd::kSeqSumThreads, "every thread takes part in the fixed-order sum");
    __shared__ double red[kNormThreads / 64];
    const int tid = threadIdx.x;
    // this thread's raw scores first: their loads overlap the reduction.  A
    // workgroup whose slice is all in range loads and stores with no branch
    // between the accesses (a branch per access made the compiler wait for
    // each store before the next); only the last one takes the guarded path.
    const int64_t base = (int64_t)blockIdx.x * kNormThreads * kNormPerThread;
    const bool full = base + kNormThreads * kNormPerThread <= n;
    float x[kNormPerThread];
    if (full) {
#pragma unroll
        for (int e = 0; e < kNormPerThread; ++e) x[e] = s_raw[base + e * kNormThreads + tid];
    } else {
#pragma unroll
        for (int e = 0; e < kNormPerThread; ++e) {
            const int64_t i = base + (int64_t)e * kNormThreads + tid;
            x[e] = i < n ? s_raw[i] : 0.0f;
        }
    }
    tgd::seq_ss_partial(block_ss, nblocks, red);
    __syncthreads();
    const float inv = tgd::seq_inv_rho(red, n, eps_seq);
    if (full) {
#pragma unroll
        for (int e = 0; e < kNormPerThread; ++e) s_norm[base + e * kNormThreads + tid] = x[e] * inv;
    } else {
#pragma unroll
        for (int e = 0; e < kNormPerThread; ++e) {
            const int64_t i = base + (int64_t)e * kNormThreads + tid;
            if (i < n) s_norm[i] = x[e] * inv;
        }
    }
}


template <int HD>
int launch_gate_hd(const uint16_t* resid, const uint16_t* w1, const uint16_t* b1, const uint16_t* w2,
                   float b2, int64_t n, int d, float eps_row, float* s_out, float* block_ss, int64_t nb,
                   hipStream_t s) {
    if (tgi::gate_rows_per_block(n) == 128)
        hipLaunchKernelGGL((gate_mlp<HD, 128>), dim3((unsigned)nb), dim3(Cfg<HD, 128>::THREADS), 0, s, resid, w1, b1,
                           w2, b2, n, d, eps_row, s_out, block_ss);
    else
        hipLaunchKernelGGL((gate_mlp<HD, 64>), dim3((unsigned)nb), dim3(Cfg<HD, 64>::THREADS), 0, s, resid, w1, b1,
                           w2, b2, n, d, eps_row, s_out, block_ss);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

}  // namespace

// Scratch of tg_gate_score_noalloc: the scorer's per-workgroup sums of
// squared raw scores, for prompts of up to kNoAllocMaxTokens tokens (256 KB,
// held on every device the library runs on until the process ends).  In host
// code `scratch` names a host-side stand-in: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) float scratch[tgi::kNoAllocMaxTokens / tgi::kGateRowsPerBlock];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices];  // per device: the address of its copy of `scratch`

// The device address of `scratch` on the calling thread's current device
// (looked up on the first call there), or nullptr on a runtime error.
float* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_dev[dev] = static_cast<float*>(p);
    }
    return g_scratch_dev[dev];
}

}  // namespace

namespace tgi {

int launch_gate_score_noalloc(const uint16_t* resid, const uint16_t* w1, const uint16_t* b1, const uint16_t* w2,
                              float b2, int64_t n, int d, int hd, float eps_row, float eps_seq, float* score_norm,
                              float* score_raw, void* stream) {
    float* ws = scratch_on_current_device();
    if (!ws) return TG_EDEVICE;
    // every workgroup overwrites its own partial: nothing to clear
    return launch_gate_score(resid, w1, b1, w2, b2, n, d, hd, eps_row, eps_seq, score_norm, score_raw, ws, stream);
}

int launch_gate_mlp(const uint16_t* resid, const uint16_t* w1, const uint16_t* b1, const uint16_t* w2, float b2,
                    int64_t n, int d, int hd, float eps_row, float* s_raw, float* block_ss, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const int64_t nb = gate_partials(n);
    switch (hd) {
        case 64: return launch_gate_hd<64>(resid, w1, b1, w2, b2, n, d, eps_row, s_raw, block_ss, nb, s);
        case 128: return launch_gate_hd<128>(resid, w1, b1, w2, b2, n, d, eps_row, s_raw, block_ss, nb, s);
        case 256: return launch_gate_hd<256>(resid, w1, b1, w2, b2, n, d, eps_row, s_raw, block_ss, nb, s);
        default: return TG_EUNSUPPORTED;
    }
}

int launch_gate_seqnorm(const float* s_raw, const float* block_ss, int64_t n, float eps_seq, float* score_norm,
                        void* stream) {
    const int64_t per = (int64_t)kNormThreads * kNormPerThread;
    hipLaunchKernelGGL(gate_seqnorm, dim3((unsigned)((n + per - 1) / per)), dim3(kNormThreads), 0,
                       (hipStream_t)stream, s_raw, block_ss, gate_partials(n), n, eps_seq, score_norm);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_EDEVICE;
}

int launch_gate_score(const uint16_t* resid, const uint16_t* w1, const uint16_t* b1,
                      const uint16_t* w2, float b2, int64_t n, int d, int hd, float eps_row,
                      float eps_seq, float* score_norm, float* score_raw, void* ws, void* stream) {
    float* block_ss = reinterpret_cast<float*>(ws);
    float* s_out = score_raw ? score_raw : score_norm;
    const int rc = launch_gate_mlp(resid, w1, b1, w2, b2, n, d, hd, eps_row, s_out, block_ss, stream);
    if (rc != TG_OK) return rc;
    return launch_gate_seqnorm(s_out, block_ss, n, eps_seq, score_norm, stream);
}

}  // namespace tgi
