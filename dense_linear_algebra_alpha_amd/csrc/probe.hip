// Measurement probes, not part of the fused path:
//   - the streaming-read ceiling: how fast this GPU reads a large buffer from HBM when the reads
//     are as simple as they get (16-byte non-temporal loads, every workgroup a contiguous
//     stretch, one add per load); benchmarks report the fused kernels against it beside the
//     published HBM peak;
//   - the streaming ceiling of the wavefront CSR kernel's access pattern: two arrays of 4-byte
//     entries (column indices and values) read in tiles of 512 entries, 8 per lane as two
//     16-byte loads per array, the next tile requested before the current one is used, with
//     each wavefront walking a contiguous stretch of its own (as that kernel does) or with the
//     4 wavefronts of a workgroup taking alternate tiles of the workgroup's stretch;
//   - the rates of the primitives a scatter of products to columns outside an LDS window could
//     be built on (fp32 atomics into one copy of the output or into one copy per XCD, scattered
//     8-byte item stores, random 4-byte gathers), on synthetic hashed column streams, so the
//     choice of binning for those columns rests on measured rates.
#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const f4* __restrict__ p, int64_t quads,
                                                                   float* sink) {
  const int64_t per_wg = (quads + gridDim.x - 1) / gridDim.x;
  const int64_t q0 = (int64_t)blockIdx.x * per_wg;
  const int64_t q1 = min(q0 + per_wg, quads);
  float acc = 0.0f;
  int64_t q = q0 + threadIdx.x;
  for (; q + (kProbeUnroll - 1) * kProbeThreads < q1; q += kProbeUnroll * kProbeThreads) {
    f4 t[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) t[u] = __builtin_nontemporal_load(p + q + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc += t[u].x + t[u].y + t[u].z + t[u].w;
  }
  for (; q < q1; q += kProbeThreads) {
    const f4 t = __builtin_nontemporal_load(p + q);
    acc += t.x + t.y + t.z + t.w;
  }
  if (acc == 1.2345678e-30f) sink[0] = acc;  // keeps the loads; never true for the probe's zeroed buffer
}

typedef int32_t i4p __attribute__((ext_vector_type(4)));
constexpr int kTileEntries = 512;  // 64 lanes x 8 entries

// `tiles` tiles of kTileEntries entries per wavefront (workgroups of 4 wavefronts); the arrays
// hold gridDim.x * 4 * tiles * kTileEntries entries, every index below that by construction.
template <bool INTERLEAVE>
__global__ __launch_bounds__(kProbeThreads) void tile_stream_kernel(const int32_t* __restrict__ a,
                                                                    const float* __restrict__ b, int64_t tiles,
                                                                    float* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  auto first = [&](int64_t t) -> int64_t {  // first entry of this lane in tile t (t < tiles)
    const int64_t tile = INTERLEAVE ? (int64_t)blockIdx.x * 4 * tiles + t * 4 + wave : gw * tiles + t;
    return tile * kTileEntries + lane * 8;
  };
  float acc = 0.0f;
  int64_t e = first(0);
  i4p c0 = *reinterpret_cast<const i4p*>(a + e), c1 = *reinterpret_cast<const i4p*>(a + e + 4);
  f4 v0 = *reinterpret_cast<const f4*>(b + e), v1 = *reinterpret_cast<const f4*>(b + e + 4);
  for (int64_t t = 1; t <= tiles; ++t) {
    e = first(t < tiles ? t : tiles - 1);  // after the last tile the last one again (cached)
    const i4p n0 = *reinterpret_cast<const i4p*>(a + e), n1 = *reinterpret_cast<const i4p*>(a + e + 4);
    const f4 w0 = *reinterpret_cast<const f4*>(b + e), w1 = *reinterpret_cast<const f4*>(b + e + 4);
    acc += (float)(c0.x + c0.y + c0.z + c0.w + c1.x + c1.y + c1.z + c1.w) *
           (v0.x + v0.y + v0.z + v0.w + v1.x + v1.y + v1.z + v1.w);
    c0 = n0; c1 = n1; v0 = w0; v1 = w1;
  }
  if (acc == 1.2345678e-30f) sink[0] = acc;  // keeps the loads; never true for zeroed arrays
}

// Column of update k: a hash of k, uniform over [0, n) (skew 0) or n u^3 for a uniform u (skew 1,
// a quarter of the updates on the first 1.6% of the columns).
__device__ __forceinline__ uint32_t probe_column(uint32_t k, uint32_t n, int skew) {
  uint32_t h = k * 2654435761u + 12345u;
  h ^= h >> 16;
  h *= 0x7feb352du;
  h ^= h >> 15;
  h *= 0x846ca68bu;
  h ^= h >> 16;
  if (!skew) return h % n;
  const float u = (float)(h >> 8) * (1.0f / 16777216.0f);
  const uint32_t c = (uint32_t)(u * u * u * (float)n);
  return c < n ? c : n - 1;
}

// The XCD (accelerator complex die) the wavefront runs on, 0..7 on MI355X.
__device__ __forceinline__ uint32_t probe_xcd() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7u;  // hwreg(HW_REG_XCC_ID, 0, 4)
}

__global__ __launch_bounds__(kProbeThreads) void scatter_probe_kernel(int kind, float* f, int2* pool, uint32_t n,
                                                                      uint32_t items, int skew, float* sink) {
  float acc = 0.0f;
  const float* gf = f;
  float* mine = kind == XTVXY_PROBE_ATOMIC_PER_XCD ? f + (size_t)probe_xcd() * n : f;
  for (uint32_t k = blockIdx.x * kProbeThreads + threadIdx.x; k < items; k += gridDim.x * kProbeThreads) {
    const uint32_t c = probe_column(k, n, skew);
    if (kind == XTVXY_PROBE_ATOMIC_PER_XCD)
      __hip_atomic_fetch_add(mine + c, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    else if (kind == XTVXY_PROBE_ATOMIC_DEVICE)
      __hip_atomic_fetch_add(mine + c, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else if (kind == XTVXY_PROBE_ITEM_STORES)
      pool[c] = make_int2((int)k, 1);
    else
      acc += gf[c];
  }
  if (acc == 1.2345678e-30f) sink[0] = acc;  // keeps the gathers
}

}  // namespace
}  // namespace xtvxy

extern "C" xtvxy_status xtvxy_scatter_probe(int kind, void* buffer, size_t bytes, uint32_t n, uint32_t items,
                                            int skew, int64_t grid, float* sink, hipStream_t stream) {
  using namespace xtvxy;
  if (!buffer || !sink) return XTVXY_ERROR_NULL_POINTER;
  if (kind < XTVXY_PROBE_ATOMIC_PER_XCD || kind > XTVXY_PROBE_GATHERS || n == 0 || (skew != 0 && skew != 1) ||
      grid <= 0 || grid > INT32_MAX || reinterpret_cast<uintptr_t>(buffer) % 16 != 0)
    return XTVXY_ERROR_INVALID_VALUE;
  // the columns index n floats (8 copies of them per XCD), or n 8-byte items
  const size_t need = kind == XTVXY_PROBE_ATOMIC_PER_XCD ? (size_t)8 * n * sizeof(float)
                      : kind == XTVXY_PROBE_ITEM_STORES  ? (size_t)n * sizeof(int2)
                                                         : (size_t)n * sizeof(float);
  if (bytes < need) return XTVXY_ERROR_WORKSPACE;
  if (items == 0) return XTVXY_SUCCESS;
  hipLaunchKernelGGL(scatter_probe_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream, kind,
                     static_cast<float*>(buffer), static_cast<int2*>(buffer), n, items, skew, sink);
  return hipGetLastError() == hipSuccess ? XTVXY_SUCCESS : XTVXY_ERROR_LAUNCH;
}

extern "C" xtvxy_status xtvxy_read_probe(const void* buffer, size_t bytes, int64_t grid, float* sink,
                                         hipStream_t stream) {
  using namespace xtvxy;
  if (!buffer || !sink) return XTVXY_ERROR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(buffer) % 16 != 0 || bytes % 16 != 0 || grid <= 0 || grid > INT32_MAX)
    return XTVXY_ERROR_INVALID_VALUE;
  if (bytes == 0) return XTVXY_SUCCESS;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const f4*>(buffer), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? XTVXY_SUCCESS : XTVXY_ERROR_LAUNCH;
}

extern "C" xtvxy_status xtvxy_tile_stream_probe(const void* indices, const void* values, int64_t entries,
                                                int64_t grid, int32_t interleave, float* sink, hipStream_t stream) {
  using namespace xtvxy;
  if (!indices || !values || !sink) return XTVXY_ERROR_NULL_POINTER;
  const int64_t per_wg = 4 * (int64_t)kTileEntries;
  if (reinterpret_cast<uintptr_t>(indices) % 16 != 0 || reinterpret_cast<uintptr_t>(values) % 16 != 0 ||
      grid <= 0 || grid > INT32_MAX || entries <= 0 || entries % (grid * per_wg) != 0 ||
      (interleave != 0 && interleave != 1))
    return XTVXY_ERROR_INVALID_VALUE;
  const int64_t tiles = entries / (grid * per_wg);
  const int32_t* a = static_cast<const int32_t*>(indices);
  const float* b = static_cast<const float*>(values);
  if (interleave)
    hipLaunchKernelGGL(tile_stream_kernel<true>, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream, a, b, tiles, sink);
  else
    hipLaunchKernelGGL(tile_stream_kernel<false>, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream, a, b, tiles, sink);
  return hipGetLastError() == hipSuccess ? XTVXY_SUCCESS : XTVXY_ERROR_LAUNCH;
}
