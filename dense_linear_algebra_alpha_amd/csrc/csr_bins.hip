// Second level of the CSR scatter for the columns outside the LDS window.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract):
// partial results are aggregated hierarchically. For the columns the fused
// kernel cannot hold in LDS, it does not add into global memory with atomics;
// it appends each product u_i * x_ij, with its column, to workspace chunks of
// the column's bin (bins of 2^bin_shift columns). These kernels finish the
// sum:
//   bin_count, bin_scan, bin_place
//                   a counting sort of the handed-out chunk ids by bin (per
//                   workgroup counts, one scan, placement), which also cuts
//                   every bin into units of at most kBinUnitChunks chunks;
//   bin_accumulate  one workgroup per unit adds the unit's items into an LDS
//                   copy of the bin's columns and writes it as one partial row.
// aggregate.hip then sums, for each binned column, the partial rows of its
// bin's units in a fixed order.
#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

constexpr int kSortThreads = 1024;
constexpr int kCountThreads = 256;
constexpr int kAccThreads = 1024;

// The handed-out chunks split evenly over the sorting workgroups (the same split in both passes).
__device__ inline void sort_range(const CsrBinArgs& a, int64_t* c0, int64_t* c1) {
  const int64_t handed = (int64_t)*a.pool_next;
  const int64_t chunks = handed < a.pool_chunks ? handed : a.pool_chunks;
  const int64_t per = (chunks + kBinSortGroups - 1) / kBinSortGroups;
  *c0 = min((int64_t)blockIdx.x * per, chunks);
  *c1 = min(*c0 + per, chunks);
}

// Pass 1: chunks of each bin in this workgroup's range -> counts[bin][group].
__global__ __launch_bounds__(kCountThreads) void bin_count_kernel(CsrBinArgs a) {
  __shared__ uint32_t hist[kMaxBins];
  int64_t c0, c1;
  sort_range(a, &c0, &c1);
  for (int b = threadIdx.x; b < a.bins; b += kCountThreads) hist[b] = 0;
  __syncthreads();
  for (int64_t c = c0 + threadIdx.x; c < c1; c += kCountThreads) {
    const int32_t b = a.chunk_bin[c];
    if ((uint32_t)b < (uint32_t)a.bins) atomicAdd(&hist[b], 1u);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < a.bins; b += kCountThreads) a.counts[b * kBinSortGroups + blockIdx.x] = (int32_t)hist[b];
}

// Pass 2 (one workgroup): counts -> exclusive offsets in (bin, group) order, the first position
// of every bin, and the units of every bin (an exclusive scan of the bins' unit counts).
// The counts pass through LDS in chunks of kScanChunk, loaded and stored coalesced; each thread
// scans a contiguous segment of a chunk.
constexpr int kScanChunk = 8192;

// Inclusive sum of x over the threads 0..tid of a kSortThreads workgroup: a scan within each
// wavefront by lane shuffles, then the wavefronts' totals (two barriers; every thread calls it).
__device__ int32_t block_inclusive_scan(int32_t x, int32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t t = __shfl_up(x, d, 64);
    if (lane >= d) x += t;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  __syncthreads();  // wsum may be reused by the next call
  return x + before;
}
__global__ __launch_bounds__(kSortThreads) void bin_scan_kernel(CsrBinArgs a) {
  __shared__ int32_t chunk_total;
  __shared__ int32_t bstart[kMaxBins + 1];
  __shared__ int32_t ucount[kMaxBins];
  __shared__ int32_t cs[kScanChunk];
  __shared__ int32_t wsum[kSortThreads / 64];
  const int tid = threadIdx.x;
  const int total = a.bins * kBinSortGroups;
  int32_t carry = 0;  // counts of the chunks before
  for (int c0 = 0; c0 < total; c0 += kScanChunk) {
    const int len = min(kScanChunk, total - c0);
    for (int i = tid; i < len; i += kSortThreads) cs[i] = a.counts[c0 + i];
    __syncthreads();
    const int per = (len + kSortThreads - 1) / kSortThreads;
    const int s0 = min(tid * per, len), s1 = min(s0 + per, len);
    int32_t sum = 0;
    for (int i = s0; i < s1; ++i) sum += cs[i];
    const int32_t incl = block_inclusive_scan(sum, wsum);  // of the per-thread sums
    if (tid == kSortThreads - 1) chunk_total = incl;
    int32_t run = carry + incl - sum;  // exclusive start of this thread's segment
    for (int i = s0; i < s1; ++i) {
      const int32_t c = cs[i];
      cs[i] = run;
      if ((c0 + i) % kBinSortGroups == 0) bstart[(c0 + i) / kBinSortGroups] = run;  // first position of a bin
      run += c;
    }
    __syncthreads();
    carry += chunk_total;
    for (int i = tid; i < len; i += kSortThreads) a.counts[c0 + i] = cs[i];
    __syncthreads();
  }
  const int32_t placed = carry;
  if (tid == 0) bstart[a.bins] = placed;
  __syncthreads();
  // units of every bin, then their exclusive scan over the bins (at most kMaxBins <= kSortThreads)
  const int32_t mine = tid < a.bins ? (bstart[tid + 1] - bstart[tid] + kBinUnitChunks - 1) / kBinUnitChunks : 0;
  const int32_t uincl = block_inclusive_scan(mine, wsum);
  if (tid < kMaxBins) ucount[tid] = uincl;
  __syncthreads();
  if (tid < a.bins) {
    a.bin_start[tid] = bstart[tid];
    a.unit_start[tid] = ucount[tid] - mine;
  }
  if (tid == 0) {
    const int64_t units = a.bins > 0 ? ucount[a.bins - 1] : 0;
    a.bin_start[a.bins] = placed;
    a.unit_start[a.bins] = (int32_t)(units < a.max_units ? units : a.max_units);
  }
}

// Pass 3: every chunk id to its place in `order` (ranks within a workgroup from LDS counters).
__global__ __launch_bounds__(kCountThreads) void bin_place_kernel(CsrBinArgs a) {
  __shared__ uint32_t cursor[kMaxBins];
  int64_t c0, c1;
  sort_range(a, &c0, &c1);
  for (int b = threadIdx.x; b < a.bins; b += kCountThreads)
    cursor[b] = (uint32_t)a.counts[b * kBinSortGroups + blockIdx.x];
  __syncthreads();
  for (int64_t c = c0 + threadIdx.x; c < c1; c += kCountThreads) {
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
  hipLaunchKernelGGL(bin_count_kernel, dim3(kBinSortGroups), dim3(kCountThreads), 0, s, a);
  hipLaunchKernelGGL(bin_scan_kernel, dim3(1), dim3(kSortThreads), 0, s, a);
  hipLaunchKernelGGL(bin_place_kernel, dim3(kBinSortGroups), dim3(kCountThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(float) << a.bin_shift;
  e = allow_dynamic_lds(reinterpret_cast<const void*>(&bin_accumulate_kernel));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bin_accumulate_kernel, dim3((unsigned)a.max_units), dim3(kAccThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace xtvxy
