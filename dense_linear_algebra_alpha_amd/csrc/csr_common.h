// Device-side pieces shared by the two fused CSR kernels (csr.hip: workgroup tiles;
// csr_waves.hip: wavefront tiles): where the columns outside the LDS window go, where y is
// gathered from, and the 64-way search of row_ptr that splits the entries between workgroups
// or wavefronts.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace xtvxy {

typedef __attribute__((address_space(1))) float global_float;
typedef __attribute__((address_space(1))) uint32_t global_uint;

// Columns outside the LDS window: none (the window holds all of them), global float atomics,
// or binned (csr_bins.hip).
enum CsrColdMode { kColdNone = 0, kColdAtomic = 1, kColdBinned = 2 };
// Where y is gathered from: global memory, an LDS copy of all of it, or an LDS copy of
// y[0, y_window) and global memory beyond.
enum CsrYMode { kYGlobal = 0, kYLds = 1, kYSplit = 2 };

// The wavefront's LDS writes made visible to its own later LDS reads: a wavefront's LDS
// operations complete in order, so only the compiler has to be kept from moving accesses
// across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Smallest r in [0, m] with rp[r] >= target (m when none), by one full wavefront: each round
// probes 64 evenly spaced positions and keeps the span between the last probe below the target
// and the first at or above it.
__device__ inline int64_t wave_lower_bound(const int32_t* __restrict__ rp, int64_t m, int64_t target) {
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

}  // namespace xtvxy
