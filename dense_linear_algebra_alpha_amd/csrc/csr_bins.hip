// Second level of the CSR scatter for the columns outside the LDS window.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract):
// partial results are aggregated hierarchically. For the columns the fused
// kernel cannot hold in LDS, it does not add into global memory with atomics;
// it appends each product u_i * x_ij, with its column, to workspace chunks of
// the column's bin (bins of 2^bin_shift columns). These two kernels finish the
// sum:
//   bin_sort        one workgroup groups the handed-out chunks by bin (a
//                   counting sort of chunk ids) and cuts every bin into units
//                   of at most kBinUnitChunks chunks;
//   bin_accumulate  one workgroup per unit adds the unit's items into an LDS
//                   copy of the bin's columns and writes it as one partial row.
// aggregate.hip then sums, for each binned column, the partial rows of its
// bin's units in a fixed order.
#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

constexpr int kSortThreads = 1024;
constexpr int kAccThreads = 1024;

__global__ __launch_bounds__(kSortThreads) void bin_sort_kernel(CsrBinArgs a) {
  __shared__ uint32_t hist[kMaxBins];
  __shared__ uint32_t cursor[kMaxBins];
  const int tid = threadIdx.x;
  const int64_t handed = (int64_t)*a.pool_next;
  const int64_t chunks = handed < a.pool_chunks ? handed : a.pool_chunks;
  for (int b = tid; b < kMaxBins; b += kSortThreads) hist[b] = 0;
  __syncthreads();
  for (int64_t c = tid; c < chunks; c += kSortThreads) {
    const int32_t b = a.chunk_bin[c];
    if ((uint32_t)b < (uint32_t)a.bins) atomicAdd(&hist[b], 1u);
  }
  __syncthreads();
  if (tid == 0) {
    // exclusive prefix sums: chunk positions and units per bin
    int64_t pos = 0, units = 0;
    for (int b = 0; b < a.bins; ++b) {
      a.bin_start[b] = (int32_t)pos;
      cursor[b] = (uint32_t)pos;
      a.unit_start[b] = (int32_t)units;
      pos += hist[b];
      units += (hist[b] + kBinUnitChunks - 1) / kBinUnitChunks;
    }
    a.bin_start[a.bins] = (int32_t)pos;
    a.unit_start[a.bins] = (int32_t)(units < a.max_units ? units : a.max_units);
  }
  __syncthreads();
  for (int64_t c = tid; c < chunks; c += kSortThreads) {
    const int32_t b = a.chunk_bin[c];
    if ((uint32_t)b < (uint32_t)a.bins) a.order[atomicAdd(&cursor[b], 1u)] = (int32_t)c;
  }
}

__global__ __launch_bounds__(kAccThreads) void bin_accumulate_kernel(CsrBinArgs a) {
  extern __shared__ float win[];  // [2^bin_shift]
  const int64_t u = blockIdx.x;
  const int32_t units = a.unit_start[a.bins];
  if (u >= units) return;
  // the unit's bin: the last b with unit_start[b] <= u
  int lo = 0, hi = a.bins - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)a.unit_start[mid] <= u) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int64_t c0 = (int64_t)a.bin_start[b] + (u - a.unit_start[b]) * kBinUnitChunks;
  const int64_t c1 = min(c0 + kBinUnitChunks, (int64_t)a.bin_start[b + 1]);
  const int width = 1 << a.bin_shift;
  const int64_t first_col = a.lds_window + ((int64_t)b << a.bin_shift);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kWavesAcc = kAccThreads / 64;
  constexpr int kPerLane = kBinChunkItems / 64;
  for (int j = tid; j < width; j += kAccThreads) win[j] = 0.0f;
  __syncthreads();
  // a wavefront takes every kWavesAcc-th chunk of the unit; a lane its items lane + 64 i
  for (int64_t ci = c0 + wave; ci < c1; ci += kWavesAcc) {
    const int32_t ch = a.order[ci];
    const int32_t fill = a.chunk_fill[ch];
    const int2* items = a.pool + (int64_t)ch * kBinChunkItems;
    int2 e[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) e[i] = items[lane + 64 * i];  // inside the chunk; masked below
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int64_t rel = (int64_t)e[i].x - first_col;
      if (lane + 64 * i < fill && rel >= 0 && rel < width) lds_add_f32(win + rel, __int_as_float(e[i].y));
    }
  }
  __syncthreads();
  float* dst = a.partial2 + u * width;
  for (int j = tid; j < width; j += kAccThreads) dst[j] = win[j];
}

}  // namespace

hipError_t launch_csr_bins(const CsrBinArgs& a, hipStream_t s) {
  if (a.bins <= 0 || a.bins > kMaxBins || a.bin_shift < 10 || a.bin_shift > 15 || a.max_units <= 0 ||
      a.max_units > INT32_MAX)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(bin_sort_kernel, dim3(1), dim3(kSortThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(float) << a.bin_shift;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bin_accumulate_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bin_accumulate_kernel, dim3((unsigned)a.max_units), dim3(kAccThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace xtvxy
