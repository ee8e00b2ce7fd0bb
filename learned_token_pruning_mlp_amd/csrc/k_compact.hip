// k_compact.hip -- gather of the kept rows (residual truncation and compaction).
//
// Pruned tokens stop at the gate layer and the kept ones continue with their
// original position ids; per-token streams such as KV rows are carried for
// the kept tokens only (fluxbbs.com TokenGate article, section on where the
// gate sits; news.farwalk.ai, "How does TokenGate learned token pruning
// work?"; aiwillknow.com, Figure 1(a)(b)).
//
// HBM-bound copy: every byte is read once and written once.  One workgroup
// moves kRows rows of one stream with 16-byte vector loads/stores, all loads
// of a thread issued before its stores.  One row per workgroup measured
// fastest (a 4 KB row per 256 threads; 2048 rows: 4.8 us against 5.4 with two
// rows and 6.2 with four): the launch is a few microseconds long, and more,
// smaller workgroups start sooner and spread the kept-index loads.
#include <hip/hip_runtime.h>

#include "tg_device.h"
#include "tg_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 1;

struct Stream {
    const char* src;
    char* dst;
    int64_t row_bytes, src_stride, dst_stride;
};

struct StreamSet {
    Stream s[TG_MAX_GATHER + 1];
};

__global__ __launch_bounds__(kThreads) void compact_rows(const int32_t* __restrict__ idx, int64_t k,
                                                         int64_t n, StreamSet set,
                                                         const int32_t* __restrict__ pos,
                                                         int32_t* __restrict__ pos_out,
                                                         const float* __restrict__ score,
                                                         float* __restrict__ score_out) {
    const Stream st = set.s[blockIdx.y];
    const int64_t t0 = (int64_t)blockIdx.x * kRows;
    const int64_t vecs = st.row_bytes >> 4;  // 16-byte pieces per row
    int32_t rows[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        int64_t t = t0 + r;
        int32_t i = (t < k) ? idx[t] : -1;
        rows[r] = (i >= 0 && (int64_t)i < n) ? i : -1;
    }
    // the first stream's blocks also carry the per-token scalars
    if (blockIdx.y == 0 && threadIdx.x < kRows) {
        int r = threadIdx.x;
        if (rows[r] >= 0) {
            if (pos_out) pos_out[t0 + r] = pos ? pos[rows[r]] : rows[r];
            if (score_out) score_out[t0 + r] = score[rows[r]];
        }
    }
    for (int64_t v0 = 0; v0 < vecs; v0 += kThreads) {
        int64_t v = v0 + threadIdx.x;
        tgd::u32x4 buf[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            if (rows[r] >= 0 && v < vecs)
                buf[r] = *reinterpret_cast<const tgd::u32x4*>(st.src + (int64_t)rows[r] * st.src_stride + (v << 4));
        }
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            if (rows[r] >= 0 && v < vecs)
                *reinterpret_cast<tgd::u32x4*>(st.dst + (t0 + r) * st.dst_stride + (v << 4)) = buf[r];
        }
    }
}

}  // namespace

namespace tgi {

int launch_compact(const int32_t* kept_idx, int64_t k, int64_t n, const uint16_t* resid,
                   uint16_t* resid_out, int d, const int32_t* pos, int32_t* pos_out,
                   const float* score, float* score_out, const tg_gather* extra, int n_extra,
                   void* stream) {
    hipStream_t s = (hipStream_t)stream;
    StreamSet set{};
    int ns = 0;
    if (resid) {
        set.s[ns++] = Stream{(const char*)resid, (char*)resid_out, (int64_t)d * 2, (int64_t)d * 2,
                             (int64_t)d * 2};
    }
    for (int e = 0; e < n_extra; ++e) {
        if (extra[e].row_bytes == 0) continue;
        set.s[ns++] = Stream{(const char*)extra[e].src, (char*)extra[e].dst, extra[e].row_bytes,
                             extra[e].src_stride, extra[e].dst_stride};
    }
    if (ns == 0) set.s[ns++] = Stream{nullptr, nullptr, 0, 0, 0};  // scalars only
    dim3 grid((unsigned)((k + kRows - 1) / kRows), (unsigned)ns);
    hipLaunchKernelGGL(compact_rows, grid, dim3(kThreads), 0, s, kept_idx, k, n, set, pos, pos_out,
                       score, score_out);
    if (hipGetLastError() != hipSuccess) return TG_EDEVICE;
    return TG_OK;
}

}  // namespace tgi
