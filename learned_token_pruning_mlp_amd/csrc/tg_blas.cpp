// tg_blas.cpp -- the projections of an upper decoder layer: plain bf16 GEMMs
// through rocBLAS (a library GEMM; the row-wise work around them is in
// k_layer.hip).
//
//   y[rows, out] = x[rows, in] . W[out, in]^T  (+ residual[rows, out])
//
// All matrices row-major, W in the usual [out_features, in_features] layout.
// gemm_bf16_f32 is the general form (bf16 operands, fp32 result, optional
// accumulation into the result) used by the scorer's backward.
// rocBLAS is column-major, where a row-major [r, c] matrix is its transpose
// [c, r] with leading dimension c; so y^T = W . x^T is the column-major
// product D[out x rows] = op(A) . B with A = W seen as [in x out] (op =
// transpose, lda = in) and B = x seen as [in x rows] (ldb = in).  bf16
// inputs and output, fp32 accumulation; the residual enters as C with
// beta = 1 (D = y, C = residual, ldc = ldd = out).
#include <rocblas/rocblas.h>

#include "tg_internal.h"

namespace tgi {

int blas_create(void** handle) {
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) return TG_EDEVICE;
    // no atomics: every GEMM through the handle gives the same bits run to run
    if (rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed) != rocblas_status_success) {
        rocblas_destroy_handle(h);
        return TG_EDEVICE;
    }
    *handle = (void*)h;
    return TG_OK;
}

int blas_destroy(void* handle) {
    return rocblas_destroy_handle((rocblas_handle)handle) == rocblas_status_success ? TG_OK : TG_EDEVICE;
}

int linear(void* handle, const uint16_t* x, const uint16_t* w, const uint16_t* residual, uint16_t* y, int64_t rows,
           int in_dim, int out_dim, void* stream) {
    rocblas_handle h = (rocblas_handle)handle;
    if (rocblas_set_stream(h, (hipStream_t)stream) != rocblas_status_success) return TG_EDEVICE;
    const float alpha = 1.0f, beta = residual ? 1.0f : 0.0f;
    const void* c = residual ? (const void*)residual : (const void*)y;
    const rocblas_status st = rocblas_gemm_ex(
        h, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)out_dim, (rocblas_int)rows,
        (rocblas_int)in_dim, &alpha, w, rocblas_datatype_bf16_r, (rocblas_int)in_dim, x, rocblas_datatype_bf16_r,
        (rocblas_int)in_dim, &beta, c, rocblas_datatype_bf16_r, (rocblas_int)out_dim, y, rocblas_datatype_bf16_r,
        (rocblas_int)out_dim, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, rocblas_gemm_flags_none);
    return st == rocblas_status_success ? TG_OK : TG_EDEVICE;
}

int gemm_bf16_f32(void* handle, bool trans_a, bool trans_b, int m, int n, int k, const uint16_t* a, int lda,
                  const uint16_t* b, int ldb, float beta, float* d, int ldd, void* stream) {
    rocblas_handle h = (rocblas_handle)handle;
    if (rocblas_set_stream(h, (hipStream_t)stream) != rocblas_status_success) return TG_EDEVICE;
    const float alpha = 1.0f;
    const rocblas_status st = rocblas_gemm_ex(
        h, trans_a ? rocblas_operation_transpose : rocblas_operation_none,
        trans_b ? rocblas_operation_transpose : rocblas_operation_none, m, n, k, &alpha, a, rocblas_datatype_bf16_r,
        lda, b, rocblas_datatype_bf16_r, ldb, &beta, d, rocblas_datatype_f32_r, ldd, d, rocblas_datatype_f32_r, ldd,
        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, rocblas_gemm_flags_none);
    return st == rocblas_status_success ? TG_OK : TG_EDEVICE;
}

int gemm_bf16_f32_batched(void* handle, bool trans_a, bool trans_b, int m, int n, int k, const uint16_t* a,
                          int lda, int64_t stride_a, const uint16_t* b, int ldb, int64_t stride_b, float* d, int ldd,
                          int64_t stride_d, int batch, void* stream) {
    rocblas_handle h = (rocblas_handle)handle;
    if (rocblas_set_stream(h, (hipStream_t)stream) != rocblas_status_success) return TG_EDEVICE;
    const float alpha = 1.0f, beta = 0.0f;
    const rocblas_status st = rocblas_gemm_strided_batched_ex(
        h, trans_a ? rocblas_operation_transpose : rocblas_operation_none,
        trans_b ? rocblas_operation_transpose : rocblas_operation_none, m, n, k, &alpha, a, rocblas_datatype_bf16_r,
        lda, stride_a, b, rocblas_datatype_bf16_r, ldb, stride_b, &beta, d, rocblas_datatype_f32_r, ldd, stride_d, d,
        rocblas_datatype_f32_r, ldd, stride_d, batch, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
        rocblas_gemm_flags_none);
    return st == rocblas_status_success ? TG_OK : TG_EDEVICE;
}

}  // namespace tgi
