// Device-side helpers shared by the xtvxy kernels (wavefront reductions, loads).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace xtvxy {

typedef float f4 __attribute__((ext_vector_type(4)));

// Sum over aligned groups of `width` lanes (power of two, <= 64) of a wavefront,
// by a butterfly of lane exchanges; every lane of a group ends with the same
// (bitwise identical) group total.
__device__ __forceinline__ float group_sum(float x, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// `VEC` consecutive floats of row `xr` starting at column `col`, zero past column n.
// X is streamed exactly once, so the loads carry the non-temporal hint.
template <int VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ xr, int64_t col, int64_t n,
                                           float (&o)[VEC]) {
  if constexpr (VEC == 4) {
    if (col + 4 <= n) {
      f4 t = __builtin_nontemporal_load(reinterpret_cast<const f4*>(xr + col));
      o[0] = t.x;
      o[1] = t.y;
      o[2] = t.z;
      o[3] = t.w;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = (col + k < n) ? __builtin_nontemporal_load(xr + col + k) : 0.0f;
    }
  } else {
    o[0] = (col < n) ? __builtin_nontemporal_load(xr + col) : 0.0f;
  }
}

}  // namespace xtvxy
