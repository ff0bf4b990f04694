// CPU oracle for out = alpha * X^T (v .* (X y)) + beta * z.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
// load or call this file: it exists so that tests, the smoke check and the
// benchmark's CPU baseline have an independent, obviously correct value to
// compare the GPU library against. It shares no header, helper or constant
// with the library under dense_linear_algebra_alpha_amd/.
//
// What is computed ("On optimizing machine learning workloads via kernel
// fusion", abstract: the generic pattern alpha * X^T (v * (X * y)) + beta * z,
// with dense and sparse X). The pattern is read as
//     X        m x n matrix (dense row-major with leading dimension ldx, or CSR)
//     y        n-vector,  X y is the ordinary matrix-vector product (m-vector)
//     v        m-vector,  v * (X y) is the elementwise product (the only product
//                         of two m-vectors that gives an m-vector)
//     X^T (.)  ordinary transposed matrix-vector product (n-vector)
//     z        n-vector,  alpha, beta scalars.
// Every input is the exact array given to the GPU; each element is promoted
// to fp64 exactly and all arithmetic below is fp64, evaluated in the plain
// order of the definition. Dense X may also be stored as bf16 (reduced-precision
// storage of X): a bf16 element is the upper 16 bits of an fp32 bit pattern,
// so it widens exactly by appending 16 zero bits; the rest is unchanged.
//     step 1  t_i = sum_k X_ik y_k             (k ascending; CSR: storage order)
//     step 2  u_i = v_i t_i                    (v absent => v_i = 1)
//     step 3  S_j = sum_i X_ij u_i             (i ascending)
//     step 4  out_j = alpha S_j + beta z_j     (beta == 0 => z is not read)
// The two halves of the pattern are also exported on their own for CSR X
// (oracle_csr_rowdot: steps 1-2, oracle_csr_tmv: steps 3-4 with u given).
// Special cases (BLAS conventions, the plainest reading where the page is
// silent): n == 0 does nothing; alpha == 0 or m == 0 gives out_j = beta z_j
// (0 when beta == 0) without reading X, v or y. Rows with v_i == 0 are not
// skipped, so IEEE NaN/Inf propagate exactly as the formula says.
//
// The "bound" entry points evaluate the same steps on absolute values,
//     D_j = |alpha| sum_i |X_ij| |v_i| sum_k |X_ik| |y_k| + |beta| |z_j|,
// which is the normaliser of the elementwise relative error used to judge the
// fp32 GPU result (a first-order bound on its rounding error, up to a factor
// of the summation length times the fp32 unit roundoff).
//
// Parallelism never changes an operation or its order: step 1 runs rows in
// parallel (each dot product is one sequential loop), dense step 3 gives each
// thread a contiguous range of output columns (each S_j is still accumulated
// over i in ascending order), CSR step 3 is one sequential scatter in row
// order. Results are therefore bitwise identical for any thread count.
//
// Build: g++ -O2 -fopenmp -fPIC -shared (no -ffast-math, no FMA contraction).

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>
#include <omp.h>

namespace {

enum { ORACLE_OK = 0, ORACLE_BAD_SIZE = 1, ORACLE_NULL = 2 };

inline double val(double x, bool absolute) { return absolute ? std::fabs(x) : x; }

// An element of X as a double: fp32 promoted exactly; bf16 widened to the fp32 with these
// upper 16 bits and zero lower bits, then promoted.
inline double elem(float x) { return (double)x; }
inline double elem(uint16_t h) {
  const uint32_t b = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &b, sizeof f);
  return (double)f;
}

// step 4 for the cases where the sum S is not formed (alpha == 0 or m == 0):
// out_j = beta z_j, and 0 when beta == 0 (z unread).
void beta_only(int64_t n, float beta, const float* z, bool absolute, double* out) {
  for (int64_t j = 0; j < n; ++j)
    out[j] = (beta == 0.0f) ? 0.0 : val((double)beta, absolute) * val((double)z[j], absolute);
}

// step 4: out_j = alpha S_j + beta z_j
void epilogue(int64_t n, float alpha, const std::vector<double>& S, float beta, const float* z,
              bool absolute, double* out) {
  for (int64_t j = 0; j < n; ++j) {
    double r = val((double)alpha, absolute) * S[j];
    if (beta != 0.0f) r += val((double)beta, absolute) * val((double)z[j], absolute);
    out[j] = r;
  }
}

template <class Elem>
int dense_impl(int64_t m, int64_t n, float alpha, const Elem* X, int64_t ldx, const float* v,
               const float* y, float beta, const float* z, double* out, bool absolute) {
  if (m < 0 || n < 0) return ORACLE_BAD_SIZE;
  if (n == 0) return ORACLE_OK;
  if (out == nullptr) return ORACLE_NULL;
  if (beta != 0.0f && z == nullptr) return ORACLE_NULL;
  if (alpha == 0.0f || m == 0) {
    beta_only(n, beta, z, absolute, out);
    return ORACLE_OK;
  }
  if (ldx < n) return ORACLE_BAD_SIZE;
  if (X == nullptr || y == nullptr) return ORACLE_NULL;

  // steps 1 and 2
  std::vector<double> u((size_t)m);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    const Elem* row = X + i * ldx;
    double t = 0.0;
    for (int64_t k = 0; k < n; ++k) t += val(elem(row[k]), absolute) * val((double)y[k], absolute);
    const double vi = (v == nullptr) ? 1.0 : val((double)v[i], absolute);
    u[(size_t)i] = vi * t;
  }

  // step 3: S_j = sum_i X_ij u_i, i ascending; threads own disjoint column ranges
  std::vector<double> S((size_t)n, 0.0);
#pragma omp parallel
  {
    const int64_t T = omp_get_num_threads(), me = omp_get_thread_num();
    const int64_t j0 = n * me / T, j1 = n * (me + 1) / T;
    for (int64_t i = 0; i < m; ++i) {
      const Elem* row = X + i * ldx;
      const double ui = u[(size_t)i];
      for (int64_t j = j0; j < j1; ++j) S[(size_t)j] += val(elem(row[j]), absolute) * ui;
    }
  }

  epilogue(n, alpha, S, beta, z, absolute, out);
  return ORACLE_OK;
}

int csr_impl(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
             const int32_t* col_idx, const float* values, const float* v, const float* y, float beta,
             const float* z, double* out, bool absolute) {
  if (m < 0 || n < 0 || nnz < 0) return ORACLE_BAD_SIZE;
  if (n == 0) return ORACLE_OK;
  if (out == nullptr) return ORACLE_NULL;
  if (beta != 0.0f && z == nullptr) return ORACLE_NULL;
  if (alpha == 0.0f || m == 0) {
    beta_only(n, beta, z, absolute, out);
    return ORACLE_OK;
  }
  if (row_ptr == nullptr || y == nullptr) return ORACLE_NULL;
  if (nnz > 0 && (col_idx == nullptr || values == nullptr)) return ORACLE_NULL;
  // structure check: zero-based, monotone row pointers ending at nnz, columns in range
  if (row_ptr[0] != 0 || (int64_t)row_ptr[m] != nnz) return ORACLE_BAD_SIZE;
  for (int64_t i = 0; i < m; ++i)
    if (row_ptr[i + 1] < row_ptr[i]) return ORACLE_BAD_SIZE;
  for (int64_t p = 0; p < nnz; ++p)
    if (col_idx[p] < 0 || (int64_t)col_idx[p] >= n) return ORACLE_BAD_SIZE;

  // steps 1 and 2: t_i over the stored entries of row i, in storage order
  // (a column stored twice contributes twice)
  std::vector<double> u((size_t)m);
#pragma omp parallel for schedule(dynamic, 4096)
  for (int64_t i = 0; i < m; ++i) {
    double t = 0.0;
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)
      t += val((double)values[p], absolute) * val((double)y[col_idx[p]], absolute);
    const double vi = (v == nullptr) ? 1.0 : val((double)v[i], absolute);
    u[(size_t)i] = vi * t;
  }

  // step 3: S_j = sum over stored entries (i, j) of X_ij u_i, rows ascending
  std::vector<double> S((size_t)n, 0.0);
  for (int64_t i = 0; i < m; ++i) {
    const double ui = u[(size_t)i];
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)
      S[(size_t)col_idx[p]] += val((double)values[p], absolute) * ui;
  }

  epilogue(n, alpha, S, beta, z, absolute, out);
  return ORACLE_OK;
}

// The two halves of the pattern, each on its own, for iterative solvers that need them
// separately (a generalized linear model's margins X w and gradient X^T r are the same two
// products the pattern chains):
//   rowdot  t_i   = alpha v_i (X y)_i + beta t0_i   (steps 1-2, then an epilogue on rows)
//   tmv     out_j = alpha (X^T u)_j + beta z_j      (steps 3-4 with u given)
// Same conventions as the full pattern: beta == 0 leaves t0 / z unread, alpha == 0 (or an
// empty dimension) reads no X, y, v or u.
int csr_check(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
              const float* values) {
  if (row_ptr == nullptr) return ORACLE_NULL;
  if (nnz > 0 && (col_idx == nullptr || values == nullptr)) return ORACLE_NULL;
  if (row_ptr[0] != 0 || (int64_t)row_ptr[m] != nnz) return ORACLE_BAD_SIZE;
  for (int64_t i = 0; i < m; ++i)
    if (row_ptr[i + 1] < row_ptr[i]) return ORACLE_BAD_SIZE;
  for (int64_t p = 0; p < nnz; ++p)
    if (col_idx[p] < 0 || (int64_t)col_idx[p] >= n) return ORACLE_BAD_SIZE;
  return ORACLE_OK;
}

int csr_rowdot_impl(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                    const int32_t* col_idx, const float* values, const float* v, const float* y,
                    float beta, const float* t0, double* out, bool absolute) {
  if (m < 0 || n < 0 || nnz < 0) return ORACLE_BAD_SIZE;
  if (m == 0) return ORACLE_OK;
  if (out == nullptr) return ORACLE_NULL;
  if (beta != 0.0f && t0 == nullptr) return ORACLE_NULL;
  const bool reads_x = alpha != 0.0f && n > 0;
  if (reads_x) {
    if (y == nullptr) return ORACLE_NULL;
    const int rc = csr_check(m, n, nnz, row_ptr, col_idx, values);
    if (rc != ORACLE_OK) return rc;
  }
#pragma omp parallel for schedule(dynamic, 4096)
  for (int64_t i = 0; i < m; ++i) {
    double r = 0.0;
    if (reads_x) {
      double t = 0.0;
      for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)
        t += val((double)values[p], absolute) * val((double)y[col_idx[p]], absolute);
      const double vi = (v == nullptr) ? 1.0 : val((double)v[i], absolute);
      r = val((double)alpha, absolute) * (vi * t);
    }
    if (beta != 0.0f) r += val((double)beta, absolute) * val((double)t0[i], absolute);
    out[i] = r;
  }
  return ORACLE_OK;
}

int csr_tmv_impl(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                 const int32_t* col_idx, const float* values, const float* u, float beta, const float* z,
                 double* out, bool absolute) {
  if (m < 0 || n < 0 || nnz < 0) return ORACLE_BAD_SIZE;
  if (n == 0) return ORACLE_OK;
  if (out == nullptr) return ORACLE_NULL;
  if (beta != 0.0f && z == nullptr) return ORACLE_NULL;
  if (alpha == 0.0f || m == 0) {
    beta_only(n, beta, z, absolute, out);
    return ORACLE_OK;
  }
  if (u == nullptr) return ORACLE_NULL;
  const int rc = csr_check(m, n, nnz, row_ptr, col_idx, values);
  if (rc != ORACLE_OK) return rc;
  // S_j = sum over stored entries (i, j) of X_ij u_i, rows ascending
  std::vector<double> S((size_t)n, 0.0);
  for (int64_t i = 0; i < m; ++i) {
    const double ui = val((double)u[i], absolute);
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)
      S[(size_t)col_idx[p]] += val((double)values[p], absolute) * ui;
  }
  epilogue(n, alpha, S, beta, z, absolute, out);
  return ORACLE_OK;
}

}  // namespace

extern "C" {

// Sets the OpenMP thread count for later calls (<= 0 keeps the current one);
// returns the number of threads a parallel region will use.
int oracle_set_threads(int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
  int used = 1;
#pragma omp parallel
  {
#pragma omp single
    used = omp_get_num_threads();
  }
  return used;
}

// ref_j = alpha S_j + beta z_j for dense row-major X (element (i,k) at X[i*ldx + k]).
int oracle_dense(int64_t m, int64_t n, float alpha, const float* X, int64_t ldx, const float* v,
                 const float* y, float beta, const float* z, double* ref) {
  return dense_impl(m, n, alpha, X, ldx, v, y, beta, z, ref, false);
}

// D_j, the same steps on absolute values.
int oracle_dense_bound(int64_t m, int64_t n, float alpha, const float* X, int64_t ldx,
                       const float* v, const float* y, float beta, const float* z, double* bound) {
  return dense_impl(m, n, alpha, X, ldx, v, y, beta, z, bound, true);
}

// The same for dense X stored as bf16 bit patterns (row-major, leading dimension ldx).
int oracle_dense_bf16(int64_t m, int64_t n, float alpha, const uint16_t* X, int64_t ldx, const float* v,
                      const float* y, float beta, const float* z, double* ref) {
  return dense_impl(m, n, alpha, X, ldx, v, y, beta, z, ref, false);
}

int oracle_dense_bf16_bound(int64_t m, int64_t n, float alpha, const uint16_t* X, int64_t ldx,
                            const float* v, const float* y, float beta, const float* z, double* bound) {
  return dense_impl(m, n, alpha, X, ldx, v, y, beta, z, bound, true);
}

// ref_j for CSR X: zero-based int32 row_ptr[m+1], col_idx[nnz], fp32 values[nnz].
int oracle_csr(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
               const int32_t* col_idx, const float* values, const float* v, const float* y,
               float beta, const float* z, double* ref) {
  return csr_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, ref, false);
}

int oracle_csr_bound(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                     const int32_t* col_idx, const float* values, const float* v, const float* y,
                     float beta, const float* z, double* bound) {
  return csr_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, bound, true);
}


// t_i = alpha v_i (X y)_i + beta t0_i for CSR X (the first half of the pattern), and its bound.
int oracle_csr_rowdot(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                      const int32_t* col_idx, const float* values, const float* v, const float* y, float beta,
                      const float* t0, double* ref) {
  return csr_rowdot_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, ref, false);
}
int oracle_csr_rowdot_bound(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                            const int32_t* col_idx, const float* values, const float* v, const float* y,
                            float beta, const float* t0, double* bound) {
  return csr_rowdot_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, bound, true);
}

// out_j = alpha (X^T u)_j + beta z_j for CSR X (the second half of the pattern), and its bound.
int oracle_csr_tmv(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                   const int32_t* col_idx, const float* values, const float* u, float beta, const float* z,
                   double* ref) {
  return csr_tmv_impl(m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, ref, false);
}
int oracle_csr_tmv_bound(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                         const int32_t* col_idx, const float* values, const float* u, float beta,
                         const float* z, double* bound) {
  return csr_tmv_impl(m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, bound, true);
}

}  // extern "C"
