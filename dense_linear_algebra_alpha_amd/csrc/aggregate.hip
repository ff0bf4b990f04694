// Second level of the hierarchical aggregation ("On optimizing machine learning
// workloads via kernel fusion", abstract: partial results are aggregated
// hierarchically) and the small helper kernels of the library.
//
// aggregate: out_j = alpha * S_j + beta * z_j with S_j the sum of the fused
// kernel's per-workgroup partials (plus, for the CSR path, the columns outside
// the LDS window: a global accumulator, or the partial rows of the units of the
// column's bin written by csr_bins.hip). Each 1024-thread workgroup owns COLS columns
// (64; 16 for outputs of at most 4096 columns, so that a narrow output still spreads
// over several CUs; 256 for outputs wider than 65536 columns, whose binned columns have
// few partial rows each, so that fewer, fuller workgroups cover them); 1024 / COLS thread
// rows each sum a strided subset of the partials in fp64, and their results are combined
// in a fixed order, so the result is bitwise reproducible for a given plan.
// The epilogue is also evaluated in fp64 and rounded once. beta == 0 never
// reads z; out may alias z (each element is read before it is written by the
// same thread). After a CSR structure analysis the columns are relabelled by
// frequency: the sums of relabelled column j then go to out[perm[j]], with
// z[perm[j]] (perm a permutation, so each element is still read and written by
// one thread).
#include "internal.h"

namespace xtvxy {
namespace {

constexpr int kAggThreads = 1024;
constexpr int64_t kNarrowOutput = 4096;  // outputs up to this width use 16 columns per workgroup
constexpr int64_t kWideOutput = 65536;   // outputs beyond this width use 256 columns per workgroup

template <int kAggCols>
__global__ __launch_bounds__(kAggThreads) void aggregate_kernel(const float* __restrict__ partial, int64_t rows,
                                                                int64_t ldp, const float* __restrict__ acc,
                                                                int64_t n, float alpha, float beta, const float* z,
                                                                float* out, BinPartials bins,
                                                                const uint32_t* __restrict__ error,
                                                                const int32_t* __restrict__ out_perm) {
  constexpr int kAggRows = kAggThreads / kAggCols;
  __shared__ double sh[kAggRows][kAggCols];
  const int tx = threadIdx.x % kAggCols, ty = threadIdx.x / kAggCols;
  const int64_t j = (int64_t)blockIdx.x * kAggCols + tx;
  double s = 0.0;
  if (j < ldp) {
#pragma unroll 8
    for (int64_t r = ty; r < rows; r += kAggRows) s += (double)partial[r * ldp + j];
  } else if (bins.partial2 != nullptr && j >= bins.first_col && j < n) {
    const int64_t rel = j - bins.first_col;
    const int64_t b = rel >> bins.bin_shift, off = rel & ((1 << bins.bin_shift) - 1);
    const int64_t u1 = bins.unit_start[b + 1];
#pragma unroll 4
    for (int64_t u = bins.unit_start[b] + ty; u < u1; u += kAggRows)
      s += (double)bins.partial2[(u << bins.bin_shift) + off];
  }
  sh[ty][tx] = s;
  __syncthreads();
  if (ty == 0 && j < n) {
    double t = sh[0][tx];
#pragma unroll
    for (int k = 1; k < kAggRows; ++k) t += sh[k][tx];
    if (acc) t += (double)acc[j];
    // relabelled columns: sum j belongs to column out_perm[j]
    const int64_t oj = out_perm != nullptr ? (int64_t)out_perm[j] : j;
    double o = (double)alpha * t;
    if (beta != 0.0f) o += (double)beta * (double)z[oj];
    // a group-row wait that gave up left some partial sums incomplete: the result is NaN
    out[oj] = (error != nullptr && *error != 0u) ? __builtin_nanf("") : (float)o;
  }
}

__global__ void beta_only_kernel(int64_t n, float beta, const float* z, float* out) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (int64_t)gridDim.x * blockDim.x)
    out[j] = (beta != 0.0f) ? beta * z[j] : 0.0f;
}

__global__ void zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ void scale_kernel(int64_t m, const float* __restrict__ v, float* t) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < m; i += (int64_t)gridDim.x * blockDim.x)
    t[i] = v[i] * t[i];
}

// flag: 0 ok, 1 row_ptr ends wrong, 2 row_ptr decreases, 3 column out of range (largest code wins)
__global__ void csr_check_kernel(int64_t m, int64_t n, int64_t nnz, const int32_t* __restrict__ rp,
                                 const int32_t* __restrict__ ci, int32_t* flag) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid == 0 && (rp[0] != 0 || (int64_t)rp[m] != nnz)) atomicMax(flag, 1);
  for (int64_t i = tid; i < m; i += stride)
    if (rp[i + 1] < rp[i]) atomicMax(flag, 2);
  for (int64_t p = tid; p < nnz; p += stride)
    if (ci[p] < 0 || (int64_t)ci[p] >= n) atomicMax(flag, 3);
}

unsigned grid_for(int64_t count, int block) {
  int64_t g = (count + block - 1) / block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_aggregate(const float* partial, int64_t rows, int64_t ldp, const float* acc, int64_t n,
                            float alpha, float beta, const float* z, float* out, hipStream_t s,
                            const BinPartials* bins, const uint32_t* error, const int32_t* out_perm) {
  if (n <= 0) return hipSuccess;
  const BinPartials none{nullptr, nullptr, 0, 0};
  if (n <= kNarrowOutput) {
    hipLaunchKernelGGL(aggregate_kernel<16>, dim3((unsigned)((n + 15) / 16)), dim3(kAggThreads), 0, s, partial,
                       rows, ldp, acc, n, alpha, beta, z, out, bins ? *bins : none, error, out_perm);
  } else if (n <= kWideOutput) {
    hipLaunchKernelGGL(aggregate_kernel<64>, dim3((unsigned)((n + 63) / 64)), dim3(kAggThreads), 0, s, partial,
                       rows, ldp, acc, n, alpha, beta, z, out, bins ? *bins : none, error, out_perm);
  } else {
    hipLaunchKernelGGL(aggregate_kernel<256>, dim3((unsigned)((n + 255) / 256)), dim3(kAggThreads), 0, s, partial,
                       rows, ldp, acc, n, alpha, beta, z, out, bins ? *bins : none, error, out_perm);
  }
  return hipGetLastError();
}

hipError_t launch_beta_only(int64_t n, float beta, const float* z, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(beta_only_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, n, beta, z, out);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(words, 256)), dim3(256), 0, s, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

hipError_t launch_scale(int64_t m, const float* v, float* t, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(scale_kernel, dim3(grid_for(m, 256)), dim3(256), 0, s, m, v, t);
  return hipGetLastError();
}

hipError_t launch_csr_check(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                            int32_t* flag, hipStream_t s) {
  hipError_t e = launch_zero(flag, sizeof(int32_t), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csr_check_kernel, dim3(grid_for(m > nnz ? m : nnz, 256)), dim3(256), 0, s, m, n, nnz,
                     row_ptr, col_idx, flag);
  return hipGetLastError();
}

}  // namespace xtvxy
