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

// wave_lower_bound for two targets at once: both searches take their rounds together, so each
// round's two probes are requested before either is waited for (one latency per round, not two).
__device__ inline void wave_lower_bound_pair(const int32_t* __restrict__ rp, int64_t m, int64_t ta, int64_t tb,
                                             int64_t& ra, int64_t& rb) {
  const int lane = threadIdx.x & 63;
  int64_t lo[2] = {0, 0}, hi[2] = {m, m};
  const int64_t target[2] = {ta, tb};
  while (hi[0] - lo[0] > 64 || hi[1] - lo[1] > 64) {
    int64_t probe[2];
    int32_t v[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t step = hi[s] - lo[s] > 64 ? (hi[s] - lo[s] + 63) / 64 : 0;  // 0: this one is done
      probe[s] = min(lo[s] + (int64_t)(lane + 1) * step, hi[s]);
      v[s] = rp[probe[s]];  // probe <= hi <= m: inside row_ptr
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (hi[s] - lo[s] <= 64) continue;  // wavefront-uniform
      const uint64_t mask = __ballot(probe[s] >= hi[s] || (int64_t)v[s] >= target[s]);
      const int k = __ffsll((unsigned long long)mask) - 1;  // lane 63 always qualifies
      const int64_t nhi = __shfl(probe[s], k, 64);
      const int64_t nlo = (k == 0) ? lo[s] : __shfl(probe[s], k - 1, 64) + 1;
      lo[s] = nlo;
      hi[s] = nhi;
    }
  }
  int64_t res[2];
  int64_t probe[2];
  int32_t v[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    probe[s] = min(lo[s] + (int64_t)lane, hi[s]);
    v[s] = rp[probe[s]];
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint64_t mask = __ballot(probe[s] >= hi[s] || (int64_t)v[s] >= target[s]);
    res[s] = target[s] <= 0 ? 0 : mask == 0 ? hi[s] : min(lo[s] + (int64_t)(__ffsll((unsigned long long)mask) - 1), hi[s]);
  }
  ra = res[0];
  rb = res[1];
}

}  // namespace xtvxy
