// Fused CSR kernels for out = alpha * X^T (v .* (X y)) + beta * z.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract): one
// fused kernel with techniques specific to sparse X; each stored entry is
// loaded once and used for both the row dot product and the transposed
// scatter, and partial outputs are aggregated hierarchically.
//
// Work split: workgroup w owns the rows whose first entry lies in
// [w q, (w + 1) q), q = ceil(nnz / grid), so every workgroup streams about the
// same number of entries (found by a 64-way search of row_ptr by one
// wavefront). A workgroup walks its rows in tiles of at most
// 256 * entries_per_thread entries and kCsrRowsPerTile rows:
//   1. row_ptr of the tile's rows is staged in LDS;
//   2. each thread loads a run of consecutive entries (value, column), gathers
//      y[column], and adds its per-row runs of products into LDS dots with LDS
//      atomics (t_i = sum of the row's entries times y);
//   3. t_i becomes u_i = v_i t_i;
//   4. each thread scatters u_row * value for the entries still in its registers:
//      into an LDS copy of the output (LDS path: the workgroup's partial output,
//      written to the workspace at the end and summed by aggregate.hip), or
//      straight into a global fp32 accumulator with hardware float atomics
//      (global path, any n).
// A row with more entries than a tile is handled by the whole workgroup in two
// sweeps over its entries (dot, then scatter).
#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

constexpr int kMaxEntries = 8;  // entries per thread per tile

// Smallest r in [0, m] with rp[r] >= target (m when none), by one full wavefront.
__device__ int64_t wave_lower_bound(const int32_t* __restrict__ rp, int64_t m, int64_t target) {
  const int lane = threadIdx.x & 63;
  if (target <= 0) return 0;
  int64_t lo = 0, hi = m;  // the answer lies in [lo, hi]; position hi counts as ">= target"
  while (hi - lo > 64) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t probe = min(lo + (int64_t)(lane + 1) * step, hi);
    const bool ge = (probe >= hi) || ((int64_t)rp[probe] >= target);
    const uint64_t mask = __ballot(ge);
    const int k = __ffsll((unsigned long long)mask) - 1;  // lane 63 always qualifies
    const int64_t nhi = __shfl(probe, k, 64);
    const int64_t nlo = (k == 0) ? lo : __shfl(probe, k - 1, 64) + 1;
    lo = nlo;
    hi = nhi;
  }
  const int64_t probe = lo + lane;
  const bool ge = (probe >= hi) || ((int64_t)rp[probe] >= target);
  const uint64_t mask = __ballot(ge);
  if (mask == 0) return hi;
  return min(lo + (int64_t)(__ffsll((unsigned long long)mask) - 1), hi);
}

template <bool LDS_OUT>
__device__ __forceinline__ void scatter_add(const CsrArgs& a, float* out_s, int32_t col, float c) {
  if constexpr (LDS_OUT) {
    atomicAdd(out_s + col, c);
  } else {
    unsafeAtomicAdd(a.partial + col, c);
  }
}

template <bool LDS_OUT>
__global__ __launch_bounds__(kBlock) void csr_tiles(CsrArgs a) {
  constexpr int RM = kCsrRowsPerTile;
  __shared__ int32_t rp_s[RM + 1];
  __shared__ float t_s[RM];
  __shared__ float lred[kWaves];
  __shared__ int64_t range_s[2];
  extern __shared__ float out_s[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.entries_per_thread;
  const int T = kBlock * K;

  if constexpr (LDS_OUT) {
    for (int64_t j = tid; j < a.n; j += kBlock) out_s[j] = 0.0f;
  }
  if (wave == 0) {
    const int64_t q = (a.nnz + gridDim.x - 1) / gridDim.x;
    const int64_t rb = wave_lower_bound(a.row_ptr, a.m, (int64_t)blockIdx.x * q);
    const int64_t re = (blockIdx.x + 1 == gridDim.x) ? a.m : wave_lower_bound(a.row_ptr, a.m, (int64_t)(blockIdx.x + 1) * q);
    if (lane == 0) {
      range_s[0] = rb;
      range_s[1] = re;
    }
  }
  __syncthreads();
  const int64_t rb = range_s[0], re = range_s[1];

  for (int64_t ra = rb; ra < re;) {
    const int cnt = (int)min((int64_t)RM, re - ra);
    __syncthreads();  // the previous tile is done with rp_s, t_s, lred
    for (int k = tid; k <= cnt; k += kBlock) rp_s[k] = a.row_ptr[ra + k];
    __syncthreads();
    const int32_t pa = rp_s[0];
    int j;  // rows [ra, ra + j) form the tile: the largest j with rp_s[j] - pa <= T
    {
      int lo = 0, hi = cnt;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rp_s[mid] - pa <= T) lo = mid; else hi = mid - 1;
      }
      j = lo;
    }
    if (j == 0) {
      // row ra alone holds more than T entries: dot sweep, then scatter sweep
      const int32_t p0 = rp_s[0], p1 = rp_s[1];
      float s = 0.0f;
      for (int64_t p = p0 + tid; p < p1; p += kBlock) s = fmaf(a.values[p], a.y[a.col_idx[p]], s);
      s = group_sum(s, 64);
      if (lane == 0) lred[wave] = s;
      __syncthreads();
      float t = lred[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) t += lred[w];
      const float u = (a.v ? a.v[ra] : 1.0f) * t;
      for (int64_t p = p0 + tid; p < p1; p += kBlock) scatter_add<LDS_OUT>(a, out_s, a.col_idx[p], u * a.values[p]);
      ra += 1;
      continue;
    }
    const int32_t pb = rp_s[j];
    for (int k = tid; k < j; k += kBlock) t_s[k] = 0.0f;
    __syncthreads();

    const int32_t e0 = pa + tid * K;
    float val[kMaxEntries];
    int32_t col[kMaxEntries];
    int row0 = 0;
    if (e0 < pb) {
      int lo = 0, hi = j - 1;  // row of entry e0: the largest r with rp_s[r] <= e0
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rp_s[mid] <= e0) lo = mid; else hi = mid - 1;
      }
      row0 = lo;
#pragma unroll
      for (int k = 0; k < kMaxEntries; ++k) {
        const int32_t e = e0 + k;
        const bool ok = k < K && e < pb;
        val[k] = ok ? __builtin_nontemporal_load(a.values + e) : 0.0f;
        col[k] = ok ? __builtin_nontemporal_load(a.col_idx + e) : 0;
      }
      int r = row0;
      float run = 0.0f;
      bool any = false;
#pragma unroll
      for (int k = 0; k < kMaxEntries; ++k) {
        const int32_t e = e0 + k;
        if (k < K && e < pb) {
          while (e >= rp_s[r + 1]) {
            if (any) atomicAdd(t_s + r, run);
            run = 0.0f;
            any = false;
            ++r;
          }
          run = fmaf(val[k], a.y[col[k]], run);
          any = true;
        }
      }
      if (any) atomicAdd(t_s + r, run);
    }
    __syncthreads();
    for (int k = tid; k < j; k += kBlock) t_s[k] = (a.v ? a.v[ra + k] : 1.0f) * t_s[k];
    __syncthreads();
    if (e0 < pb) {
      int r = row0;
#pragma unroll
      for (int k = 0; k < kMaxEntries; ++k) {
        const int32_t e = e0 + k;
        if (k < K && e < pb) {
          while (e >= rp_s[r + 1]) ++r;
          scatter_add<LDS_OUT>(a, out_s, col[k], t_s[r] * val[k]);
        }
      }
    }
    ra += j;
  }

  if constexpr (LDS_OUT) {
    __syncthreads();
    float* dst = a.partial + (int64_t)blockIdx.x * a.n;
    for (int64_t c = tid; c < a.n; c += kBlock) dst[c] = out_s[c];
  }
}

}  // namespace

hipError_t launch_csr(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if (p.block_threads != kBlock || p.grid <= 0 || p.grid > INT32_MAX) return hipErrorInvalidValue;
  if (p.entries_per_thread < 1 || p.entries_per_thread > kMaxEntries) return hipErrorInvalidValue;
  const dim3 grid((unsigned)p.grid), block(kBlock);
  switch (p.kernel) {
    case XTVXY_CSR_LDS_TILES: {
      const size_t lds = (size_t)a.n * sizeof(float);
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&csr_tiles<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(csr_tiles<true>, grid, block, lds, s, a);
      return hipGetLastError();
    }
    case XTVXY_CSR_GLOBAL_TILES:
      hipLaunchKernelGGL(csr_tiles<false>, grid, block, 0, s, a);
      return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace xtvxy
