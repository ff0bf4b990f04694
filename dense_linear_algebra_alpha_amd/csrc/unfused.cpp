// Unfused comparator: the same result from operator-level library kernels.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract)
// measures its fused kernel against launching several operator-level kernels
// from GPU-accelerated libraries. On MI355X those are rocBLAS (dense GEMV) and
// rocSPARSE (SpMV), with one elementwise kernel for v .* t in between:
//   t   = X y                      (sgemv / spmv, reads X once)
//   t   = v .* t                   (elementwise kernel; skipped when v is absent)
//   out = z                        (device copy, when beta != 0 and out != z)
//   out = alpha X^T t + beta out   (sgemv / spmv on the transpose, reads X again)
// so X crosses HBM twice and t makes a round trip, against once for the fused path. rocBLAS's
// sgemv without transpose on the column-major view of a row-major X (the last step) is slow when
// X has few columns and many rows; xtvxy_dense_f32_unfused_reference_explicit takes a caller-made
// copy of X^T (xtvxy_dense_f32_transpose) so that both steps are transposed sgemvs. rocSPARSE's
// transposed SpMV serialises on output columns that many rows share; the plan option
// XTVXY_UNFUSED_EXPLICIT_TRANSPOSE keeps a CSR copy of X^T (made once with csr2csc) so that the
// last step is a forward SpMV: the stronger operator-level baseline.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <rocsparse/rocsparse.h>

#include <cstdint>
#include <mutex>

#include "internal.h"

using namespace xtvxy;

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_blas_mutex;
rocblas_handle g_blas[kMaxDevices];

xtvxy_status blas_handle(rocblas_handle* h) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return XTVXY_ERROR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_blas_mutex);
  if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
    g_blas[dev] = nullptr;
    return XTVXY_ERROR_LIBRARY;
  }
  *h = g_blas[dev];
  return XTVXY_SUCCESS;
}

}  // namespace

struct xtvxy_csr_unfused_plan_s {
  int device = 0;
  int64_t m = 0, n = 0, nnz = 0;
  const int32_t* row_ptr = nullptr;
  const int32_t* col_idx = nullptr;
  const float* values = nullptr;
  rocsparse_handle handle = nullptr;
  rocsparse_spmat_descr A = nullptr;
  rocsparse_dnvec_descr vec_n = nullptr;  // n-length operand (y, or out)
  rocsparse_dnvec_descr vec_m = nullptr;  // m-length operand (t)
  rocsparse_dnvec_descr vec_n2 = nullptr; // n-length result (out)
  void* buf_fwd = nullptr;
  void* buf_tr = nullptr;
  size_t buf_fwd_bytes = 0, buf_tr_bytes = 0;
  float* t = nullptr;       // m floats
  float* dummy_n = nullptr; // n floats, stands in for y/out while the plan is analysed
  // explicit transpose: X^T as a CSR matrix (n x m), so that X^T t is a forward SpMV
  bool explicit_t = false;
  rocsparse_spmat_descr AT = nullptr;
  int32_t* at_ptr = nullptr;  // n + 1
  int32_t* at_idx = nullptr;  // nnz
  float* at_val = nullptr;    // nnz
  void* buf_at = nullptr;
  size_t buf_at_bytes = 0;
};

namespace {

void destroy_plan(xtvxy_csr_unfused_plan p) {
  if (!p) return;
  if (p->A) rocsparse_destroy_spmat_descr(p->A);
  if (p->vec_n) rocsparse_destroy_dnvec_descr(p->vec_n);
  if (p->vec_m) rocsparse_destroy_dnvec_descr(p->vec_m);
  if (p->vec_n2) rocsparse_destroy_dnvec_descr(p->vec_n2);
  if (p->handle) rocsparse_destroy_handle(p->handle);
  if (p->buf_fwd) (void)hipFree(p->buf_fwd);
  if (p->buf_tr) (void)hipFree(p->buf_tr);
  if (p->t) (void)hipFree(p->t);
  if (p->dummy_n) (void)hipFree(p->dummy_n);
  if (p->AT) rocsparse_destroy_spmat_descr(p->AT);
  if (p->at_ptr) (void)hipFree(p->at_ptr);
  if (p->at_idx) (void)hipFree(p->at_idx);
  if (p->at_val) (void)hipFree(p->at_val);
  if (p->buf_at) (void)hipFree(p->buf_at);
  delete p;
}

constexpr rocsparse_spmv_alg kAlg = rocsparse_spmv_alg_default;

rocsparse_status spmv_with(xtvxy_csr_unfused_plan p, rocsparse_spmat_descr mat, rocsparse_operation op,
                           const float* alpha, rocsparse_dnvec_descr x, const float* beta, rocsparse_dnvec_descr y,
                           rocsparse_spmv_stage stage, size_t* bytes, void* buf) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wdeprecated-declarations"
  return rocsparse_spmv(p->handle, op, alpha, mat, x, beta, y, rocsparse_datatype_f32_r, kAlg, stage, bytes, buf);
#pragma clang diagnostic pop
}

rocsparse_status spmv(xtvxy_csr_unfused_plan p, rocsparse_operation op, const float* alpha,
                      rocsparse_dnvec_descr x, const float* beta, rocsparse_dnvec_descr y, rocsparse_spmv_stage stage,
                      size_t* bytes, void* buf) {
  return spmv_with(p, p->A, op, alpha, x, beta, y, stage, bytes, buf);
}

// alpha X^T x + beta y: the library's transposed SpMV, or a forward SpMV with the explicit X^T.
rocsparse_status spmv_transposed(xtvxy_csr_unfused_plan p, const float* alpha, rocsparse_dnvec_descr x,
                                 const float* beta, rocsparse_dnvec_descr y) {
  if (p->explicit_t) {
    size_t bytes = p->buf_at_bytes;
    return spmv_with(p, p->AT, rocsparse_operation_none, alpha, x, beta, y, rocsparse_spmv_stage_compute, &bytes,
                     p->buf_at);
  }
  size_t bytes = p->buf_tr_bytes;
  return spmv(p, rocsparse_operation_transpose, alpha, x, beta, y, rocsparse_spmv_stage_compute, &bytes, p->buf_tr);
}

// Builds X^T (the CSC form of X read as CSR) and analyses the forward SpMV with it.
xtvxy_status build_transpose(xtvxy_csr_unfused_plan p) {
  const int64_t m = p->m, n = p->n, nnz = p->nnz;
  if (hipMalloc(&p->at_ptr, (size_t)(n + 1) * sizeof(int32_t)) != hipSuccess ||
      hipMalloc(&p->at_idx, (size_t)nnz * sizeof(int32_t)) != hipSuccess ||
      hipMalloc(&p->at_val, (size_t)nnz * sizeof(float)) != hipSuccess)
    return XTVXY_ERROR_LAUNCH;
  size_t tmp_bytes = 0;
  if (rocsparse_csr2csc_buffer_size(p->handle, (rocsparse_int)m, (rocsparse_int)n, (rocsparse_int)nnz, p->row_ptr,
                                    p->col_idx, rocsparse_action_numeric, &tmp_bytes) != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  void* tmp = nullptr;
  if (hipMalloc(&tmp, tmp_bytes > 0 ? tmp_bytes : 256) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  const rocsparse_status cs =
      rocsparse_scsr2csc(p->handle, (rocsparse_int)m, (rocsparse_int)n, (rocsparse_int)nnz, p->values, p->row_ptr,
                         p->col_idx, p->at_val, p->at_idx, p->at_ptr, rocsparse_action_numeric,
                         rocsparse_index_base_zero, tmp);
  hipStream_t s = nullptr;
  rocsparse_get_stream(p->handle, &s);
  const hipError_t sync = hipStreamSynchronize(s);
  (void)hipFree(tmp);
  if (cs != rocsparse_status_success) return XTVXY_ERROR_LIBRARY;
  if (sync != hipSuccess) return XTVXY_ERROR_LAUNCH;
  if (rocsparse_create_csr_descr(&p->AT, n, m, nnz, p->at_ptr, p->at_idx, p->at_val, rocsparse_indextype_i32,
                                 rocsparse_indextype_i32, rocsparse_index_base_zero,
                                 rocsparse_datatype_f32_r) != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  const float one = 1.0f, zero = 0.0f;
  if (spmv_with(p, p->AT, rocsparse_operation_none, &one, p->vec_m, &zero, p->vec_n2,
                rocsparse_spmv_stage_buffer_size, &p->buf_at_bytes, nullptr) != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  if (hipMalloc(&p->buf_at, p->buf_at_bytes > 0 ? p->buf_at_bytes : 256) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  if (spmv_with(p, p->AT, rocsparse_operation_none, &one, p->vec_m, &zero, p->vec_n2,
                rocsparse_spmv_stage_preprocess, &p->buf_at_bytes, p->buf_at) != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  p->explicit_t = true;
  return XTVXY_SUCCESS;
}

}  // namespace

extern "C" {

xtvxy_status xtvxy_dense_f32_unfused_reference_workspace_size(int64_t m, int64_t n, size_t* bytes) {
  if (!bytes) return XTVXY_ERROR_NULL_POINTER;
  if (m < 0 || n < 0) return XTVXY_ERROR_INVALID_VALUE;
  *bytes = (m > 0 && n > 0) ? align_up((size_t)m * sizeof(float)) : 0;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_dense_f32_unfused_reference(int64_t m, int64_t n, float alpha, const float* X, int64_t ldx,
                                               const float* v, const float* y, float beta, const float* z,
                                               float* out, void* workspace, size_t workspace_bytes,
                                               hipStream_t stream) {
  bool quick = false;
  xtvxy_status st = check_dense_args(m, n, alpha, X, ldx, v, y, beta, z, out, &quick);
  if (st != XTVXY_SUCCESS) return st;
  if (quick) return n == 0 ? XTVXY_SUCCESS
                           : (launch_beta_only(n, beta, z, out, stream) == hipSuccess ? XTVXY_SUCCESS
                                                                                      : XTVXY_ERROR_LAUNCH);
  if (m > INT32_MAX || n > INT32_MAX || ldx > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  if (!workspace || workspace_bytes < (size_t)m * sizeof(float)) return XTVXY_ERROR_WORKSPACE;
  rocblas_handle h;
  st = blas_handle(&h);
  if (st != XTVXY_SUCCESS) return st;
  if (rocblas_set_stream(h, stream) != rocblas_status_success ||
      rocblas_set_pointer_mode(h, rocblas_pointer_mode_host) != rocblas_status_success)
    return XTVXY_ERROR_LIBRARY;
  float* t = static_cast<float*>(workspace);
  const float one = 1.0f, zero = 0.0f;
  // Row-major X (m x n, leading dimension ldx) is the column-major n x m matrix A = X^T:
  // X y = A^T y and X^T t = A t.
  if (rocblas_sgemv(h, rocblas_operation_transpose, (rocblas_int)n, (rocblas_int)m, &one, X, (rocblas_int)ldx, y, 1,
                    &zero, t, 1) != rocblas_status_success)
    return XTVXY_ERROR_LIBRARY;
  if (v && launch_scale(m, v, t, stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  if (beta != 0.0f && out != z &&
      hipMemcpyAsync(out, z, (size_t)n * sizeof(float), hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return XTVXY_ERROR_LAUNCH;
  if (rocblas_sgemv(h, rocblas_operation_none, (rocblas_int)n, (rocblas_int)m, &alpha, X, (rocblas_int)ldx, t, 1,
                    &beta, out, 1) != rocblas_status_success)
    return XTVXY_ERROR_LIBRARY;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_dense_f32_transpose(int64_t m, int64_t n, const float* X, int64_t ldx, float* Xt, int64_t ldxt,
                                       hipStream_t stream) {
  if (m < 0 || n < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (m == 0 || n == 0) return XTVXY_SUCCESS;
  if (ldx < n || ldxt < m) return XTVXY_ERROR_INVALID_VALUE;
  if (m > INT32_MAX || n > INT32_MAX || ldx > INT32_MAX || ldxt > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  if (!X || !Xt) return XTVXY_ERROR_NULL_POINTER;
  const size_t xb = ((size_t)(m - 1) * ldx + n) * sizeof(float), tb = ((size_t)(n - 1) * ldxt + m) * sizeof(float);
  if (reinterpret_cast<uintptr_t>(X) < reinterpret_cast<uintptr_t>(Xt) + tb &&
      reinterpret_cast<uintptr_t>(Xt) < reinterpret_cast<uintptr_t>(X) + xb)
    return XTVXY_ERROR_ALIASING;
  rocblas_handle h;
  xtvxy_status st = blas_handle(&h);
  if (st != XTVXY_SUCCESS) return st;
  if (rocblas_set_stream(h, stream) != rocblas_status_success ||
      rocblas_set_pointer_mode(h, rocblas_pointer_mode_host) != rocblas_status_success)
    return XTVXY_ERROR_LIBRARY;
  // Column-major: X is the n x m matrix A (lda = ldx), Xt the m x n matrix C (ldc = ldxt), C = A^T
  // (beta = 0: the second operand, C itself, is not read).
  const float one = 1.0f, zero = 0.0f;
  if (rocblas_sgeam(h, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)m, (rocblas_int)n, &one, X,
                    (rocblas_int)ldx, &zero, Xt, (rocblas_int)ldxt, Xt, (rocblas_int)ldxt) != rocblas_status_success)
    return XTVXY_ERROR_LIBRARY;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_dense_f32_unfused_reference_explicit(int64_t m, int64_t n, float alpha, const float* X, int64_t ldx,
                                                        const float* Xt, int64_t ldxt, const float* v, const float* y,
                                                        float beta, const float* z, float* out, void* workspace,
                                                        size_t workspace_bytes, hipStream_t stream) {
  bool quick = false;
  xtvxy_status st = check_dense_args(m, n, alpha, X, ldx, v, y, beta, z, out, &quick);
  if (st != XTVXY_SUCCESS) return st;
  if (quick) return n == 0 ? XTVXY_SUCCESS
                           : (launch_beta_only(n, beta, z, out, stream) == hipSuccess ? XTVXY_SUCCESS
                                                                                      : XTVXY_ERROR_LAUNCH);
  if (ldxt < m) return XTVXY_ERROR_INVALID_VALUE;
  if (m > INT32_MAX || n > INT32_MAX || ldx > INT32_MAX || ldxt > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  if (!Xt) return XTVXY_ERROR_NULL_POINTER;
  const size_t tb = ((size_t)(n - 1) * ldxt + m) * sizeof(float);
  if (reinterpret_cast<uintptr_t>(out) < reinterpret_cast<uintptr_t>(Xt) + tb &&
      reinterpret_cast<uintptr_t>(Xt) < reinterpret_cast<uintptr_t>(out) + (size_t)n * sizeof(float))
    return XTVXY_ERROR_ALIASING;
  if (!workspace || workspace_bytes < (size_t)m * sizeof(float)) return XTVXY_ERROR_WORKSPACE;
  rocblas_handle h;
  st = blas_handle(&h);
  if (st != XTVXY_SUCCESS) return st;
  if (rocblas_set_stream(h, stream) != rocblas_status_success ||
      rocblas_set_pointer_mode(h, rocblas_pointer_mode_host) != rocblas_status_success)
    return XTVXY_ERROR_LIBRARY;
  float* t = static_cast<float*>(workspace);
  const float one = 1.0f, zero = 0.0f;
  // X y = A^T y with A the column-major n x m view of X; X^T t = B^T t with B the column-major
  // m x n view of Xt. Both are transposed products, each reading its matrix along its rows.
  if (rocblas_sgemv(h, rocblas_operation_transpose, (rocblas_int)n, (rocblas_int)m, &one, X, (rocblas_int)ldx, y, 1,
                    &zero, t, 1) != rocblas_status_success)
    return XTVXY_ERROR_LIBRARY;
  if (v && launch_scale(m, v, t, stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  if (beta != 0.0f && out != z &&
      hipMemcpyAsync(out, z, (size_t)n * sizeof(float), hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return XTVXY_ERROR_LAUNCH;
  if (rocblas_sgemv(h, rocblas_operation_transpose, (rocblas_int)m, (rocblas_int)n, &alpha, Xt, (rocblas_int)ldxt, t,
                    1, &beta, out, 1) != rocblas_status_success)
    return XTVXY_ERROR_LIBRARY;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_csr_f32_unfused_plan_create(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr,
                                               const int32_t* col_idx, const float* values, hipStream_t stream,
                                               xtvxy_csr_unfused_plan* out_plan) {
  return xtvxy_csr_f32_unfused_plan_create_ex(m, n, nnz, row_ptr, col_idx, values, XTVXY_UNFUSED_TRANSPOSE_OP,
                                              stream, out_plan);
}

xtvxy_status xtvxy_csr_f32_unfused_plan_create_ex(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr,
                                                  const int32_t* col_idx, const float* values, int32_t options,
                                                  hipStream_t stream, xtvxy_csr_unfused_plan* out_plan) {
  if (!out_plan) return XTVXY_ERROR_NULL_POINTER;
  *out_plan = nullptr;
  if (m < 0 || n < 0 || nnz < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (options != XTVXY_UNFUSED_TRANSPOSE_OP && options != XTVXY_UNFUSED_EXPLICIT_TRANSPOSE)
    return XTVXY_ERROR_INVALID_VALUE;
  if (nnz > INT32_MAX || m >= INT32_MAX || n > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  if (!row_ptr || (nnz > 0 && (!col_idx || !values))) return XTVXY_ERROR_NULL_POINTER;
  xtvxy_csr_unfused_plan p = new xtvxy_csr_unfused_plan_s;
  p->m = m;
  p->n = n;
  p->nnz = nnz;
  p->row_ptr = row_ptr;
  p->col_idx = col_idx;
  p->values = values;
  auto fail = [&](xtvxy_status s) {
    destroy_plan(p);
    return s;
  };
  if (hipGetDevice(&p->device) != hipSuccess) return fail(XTVXY_ERROR_LAUNCH);
  if (m == 0 || n == 0 || nnz == 0) {  // nothing for the libraries to do: out = beta z
    *out_plan = p;
    return XTVXY_SUCCESS;
  }
  if (hipMalloc(&p->t, (size_t)m * sizeof(float)) != hipSuccess ||
      hipMalloc(&p->dummy_n, (size_t)n * sizeof(float)) != hipSuccess)
    return fail(XTVXY_ERROR_LAUNCH);
  if (rocsparse_create_handle(&p->handle) != rocsparse_status_success ||
      rocsparse_set_stream(p->handle, stream) != rocsparse_status_success ||
      rocsparse_set_pointer_mode(p->handle, rocsparse_pointer_mode_host) != rocsparse_status_success)
    return fail(XTVXY_ERROR_LIBRARY);
  if (rocsparse_create_csr_descr(&p->A, m, n, nnz, const_cast<int32_t*>(row_ptr), const_cast<int32_t*>(col_idx),
                                 const_cast<float*>(values), rocsparse_indextype_i32, rocsparse_indextype_i32,
                                 rocsparse_index_base_zero, rocsparse_datatype_f32_r) != rocsparse_status_success ||
      rocsparse_create_dnvec_descr(&p->vec_n, n, p->dummy_n, rocsparse_datatype_f32_r) != rocsparse_status_success ||
      rocsparse_create_dnvec_descr(&p->vec_m, m, p->t, rocsparse_datatype_f32_r) != rocsparse_status_success ||
      rocsparse_create_dnvec_descr(&p->vec_n2, n, p->dummy_n, rocsparse_datatype_f32_r) != rocsparse_status_success)
    return fail(XTVXY_ERROR_LIBRARY);
  const float one = 1.0f, zero = 0.0f;
  if (spmv(p, rocsparse_operation_none, &one, p->vec_n, &zero, p->vec_m, rocsparse_spmv_stage_buffer_size,
           &p->buf_fwd_bytes, nullptr) != rocsparse_status_success ||
      spmv(p, rocsparse_operation_transpose, &one, p->vec_m, &zero, p->vec_n2, rocsparse_spmv_stage_buffer_size,
           &p->buf_tr_bytes, nullptr) != rocsparse_status_success)
    return fail(XTVXY_ERROR_LIBRARY);
  if (hipMalloc(&p->buf_fwd, p->buf_fwd_bytes > 0 ? p->buf_fwd_bytes : 256) != hipSuccess ||
      hipMalloc(&p->buf_tr, p->buf_tr_bytes > 0 ? p->buf_tr_bytes : 256) != hipSuccess)
    return fail(XTVXY_ERROR_LAUNCH);
  if (spmv(p, rocsparse_operation_none, &one, p->vec_n, &zero, p->vec_m, rocsparse_spmv_stage_preprocess,
           &p->buf_fwd_bytes, p->buf_fwd) != rocsparse_status_success ||
      spmv(p, rocsparse_operation_transpose, &one, p->vec_m, &zero, p->vec_n2, rocsparse_spmv_stage_preprocess,
           &p->buf_tr_bytes, p->buf_tr) != rocsparse_status_success)
    return fail(XTVXY_ERROR_LIBRARY);
  if (options == XTVXY_UNFUSED_EXPLICIT_TRANSPOSE) {
    const xtvxy_status st = build_transpose(p);
    if (st != XTVXY_SUCCESS) return fail(st);
  }
  if (hipStreamSynchronize(stream) != hipSuccess) return fail(XTVXY_ERROR_LAUNCH);
  *out_plan = p;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_csr_f32_unfused_plan_destroy(xtvxy_csr_unfused_plan plan) {
  destroy_plan(plan);
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_csr_f32_unfused_reference(xtvxy_csr_unfused_plan p, float alpha, const float* v,
                                             const float* y, float beta, const float* z, float* out,
                                             hipStream_t stream) {
  if (!p) return XTVXY_ERROR_NULL_POINTER;
  bool quick = false;
  xtvxy_status st = check_csr_args(p->m, p->n, p->nnz, alpha, p->row_ptr, p->col_idx, p->values, v, y, beta, z,
                                   out, &quick);
  if (st != XTVXY_SUCCESS) return st;
  if (quick) return p->n == 0 ? XTVXY_SUCCESS
                              : (launch_beta_only(p->n, beta, z, out, stream) == hipSuccess ? XTVXY_SUCCESS
                                                                                           : XTVXY_ERROR_LAUNCH);
  if (rocsparse_set_stream(p->handle, stream) != rocsparse_status_success) return XTVXY_ERROR_LIBRARY;
  if (rocsparse_dnvec_set_values(p->vec_n, const_cast<float*>(y)) != rocsparse_status_success ||
      rocsparse_dnvec_set_values(p->vec_m, p->t) != rocsparse_status_success ||
      rocsparse_dnvec_set_values(p->vec_n2, out) != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  const float one = 1.0f, zero = 0.0f;
  size_t bytes = p->buf_fwd_bytes;
  if (spmv(p, rocsparse_operation_none, &one, p->vec_n, &zero, p->vec_m, rocsparse_spmv_stage_compute, &bytes,
           p->buf_fwd) != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  if (v && launch_scale(p->m, v, p->t, stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  if (beta != 0.0f) {
    if (out != z &&
        hipMemcpyAsync(out, z, (size_t)p->n * sizeof(float), hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return XTVXY_ERROR_LAUNCH;
  } else if (launch_zero(out, (size_t)p->n * sizeof(float), stream) != hipSuccess) {
    return XTVXY_ERROR_LAUNCH;  // the transposed product scales out by beta: start from zeros
  }
  if (spmv_transposed(p, &alpha, p->vec_m, &beta, p->vec_n2) != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  return XTVXY_SUCCESS;
}

}  // extern "C"

namespace xtvxy {

// t = X y with the comparator's rocSPARSE SpMV (the margins step of an unfused solver).
xtvxy_status unfused_rowdot(xtvxy_csr_unfused_plan p, const float* y, float* t, hipStream_t stream) {
  if (!p) return XTVXY_ERROR_NULL_POINTER;
  if (p->m == 0) return XTVXY_SUCCESS;
  if (!t) return XTVXY_ERROR_NULL_POINTER;
  if (!p->handle)  // n == 0 or nnz == 0: every row product is empty
    return launch_zero(t, (size_t)p->m * sizeof(float), stream) == hipSuccess ? XTVXY_SUCCESS : XTVXY_ERROR_LAUNCH;
  if (!y) return XTVXY_ERROR_NULL_POINTER;
  if (rocsparse_set_stream(p->handle, stream) != rocsparse_status_success ||
      rocsparse_dnvec_set_values(p->vec_n, const_cast<float*>(y)) != rocsparse_status_success ||
      rocsparse_dnvec_set_values(p->vec_m, t) != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  const float one = 1.0f, zero = 0.0f;
  size_t bytes = p->buf_fwd_bytes;
  const rocsparse_status r = spmv(p, rocsparse_operation_none, &one, p->vec_n, &zero, p->vec_m,
                                  rocsparse_spmv_stage_compute, &bytes, p->buf_fwd);
  if (rocsparse_dnvec_set_values(p->vec_m, p->t) != rocsparse_status_success || r != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  return XTVXY_SUCCESS;
}

// out = alpha X^T u + beta z with the comparator's transposed rocSPARSE SpMV (the gradient step
// of an unfused solver); z is read only when beta != 0 and may equal out.
xtvxy_status unfused_tmv(xtvxy_csr_unfused_plan p, float alpha, const float* u, float beta, const float* z,
                         float* out, hipStream_t stream) {
  if (!p) return XTVXY_ERROR_NULL_POINTER;
  if (p->n == 0) return XTVXY_SUCCESS;
  if (!out || (beta != 0.0f && !z)) return XTVXY_ERROR_NULL_POINTER;
  if (!p->handle || alpha == 0.0f)
    return launch_beta_only(p->n, beta, z, out, stream) == hipSuccess ? XTVXY_SUCCESS : XTVXY_ERROR_LAUNCH;
  if (!u) return XTVXY_ERROR_NULL_POINTER;
  if (beta != 0.0f) {
    if (out != z &&
        hipMemcpyAsync(out, z, (size_t)p->n * sizeof(float), hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return XTVXY_ERROR_LAUNCH;
  } else if (launch_zero(out, (size_t)p->n * sizeof(float), stream) != hipSuccess) {
    return XTVXY_ERROR_LAUNCH;
  }
  if (rocsparse_set_stream(p->handle, stream) != rocsparse_status_success ||
      rocsparse_dnvec_set_values(p->vec_m, const_cast<float*>(u)) != rocsparse_status_success ||
      rocsparse_dnvec_set_values(p->vec_n2, out) != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  const rocsparse_status r = spmv_transposed(p, &alpha, p->vec_m, &beta, p->vec_n2);
  if (rocsparse_dnvec_set_values(p->vec_m, p->t) != rocsparse_status_success || r != rocsparse_status_success)
    return XTVXY_ERROR_LIBRARY;
  return XTVXY_SUCCESS;
}

// The plan's shape and matrix, for callers that check that a plan belongs to their matrix.
void unfused_plan_shape(xtvxy_csr_unfused_plan p, int64_t* m, int64_t* n, int64_t* nnz, const int32_t** row_ptr,
                        const int32_t** col_idx, const float** values) {
  *m = p->m;
  *n = p->n;
  *nnz = p->nnz;
  *row_ptr = p->row_ptr;
  *col_idx = p->col_idx;
  *values = p->values;
}

}  // namespace xtvxy
