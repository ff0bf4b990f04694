// Fused dense kernels for out = alpha * X^T (v .* (X y)) + beta * z.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract):
// the fused kernel loads each element of X once and uses it twice — for the
// row dot product t_i = x_i . y and, after the scale u_i = v_i t_i, for the
// accumulation of u_i x_i into the transposed product — and aggregates partial
// results hierarchically. Here the two uses of a row happen while the row is
// still in registers; each workgroup sums its rows into one partial n-vector
// (registers -> LDS -> workspace), and aggregate.hip sums the workgroups'
// partials and applies alpha and beta. Thread coarsening: a workgroup walks a
// contiguous block of rows_per_unit rows.
//
// Three layouts of a row over the threads (chosen by the launch model):
//   wave rows  (n <= 1024): `lanes_per_row` lanes of a wavefront share a row,
//              each holding `chunks` pieces of `VEC` columns; a wavefront keeps
//              UNR rows per row group in flight and reduces their dots with DPP
//              and permlane-swap lane exchanges (no LDS round trips).
//   block rows (n <= 8192): the 256 threads of a workgroup share a row; the dot
//              is reduced across the four wavefronts through LDS.
//   group rows (wider):     `group` workgroups split a row into column
//              slices (fp32: each thread's column sums in LDS, 4 rows of 8
//              chunks per exchange). Each member publishes its slice dots in 64-bit slots
//              that carry the value and the step number together, so a reader
//              needs no fence: it waits until a slot shows the step it expects.
//              The grid never exceeds what the device holds at once and the
//              library runs group-row launches of a device one after another,
//              so every member gets a slot; a bounded wait flags an error
//              instead of hanging, and a member whose wait gave up waits no more.
//
// X is fp32, or bf16 (reduced-precision storage: each element widened to fp32 as it is
// loaded, all arithmetic fp32). A chunk is VEC consecutive elements read by one load: 4 fp32 or
// 8 bf16 per 16-byte load, or 1 element when X is not aligned for that.
//
// Every loop runs the same number of iterations in all lanes of a workgroup
// (rows past the end are masked to zero), so cross-lane exchanges never execute
// under divergent control flow.
#include <map>
#include <mutex>

#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

constexpr uint32_t kSpinLimit = 1u << 24;  // a barrier wait gives up (and flags an error) after this
                                           // many polls, unless the call sets a smaller bound

template <class E, int VEC, int NCH, int UNR>
__global__ __launch_bounds__(kBlock) void dense_wave_rows(DenseArgs a) {
  constexpr int W = 64 * VEC * NCH;  // widest row a wavefront covers
  __shared__ float red[kWaves][W];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lpr = a.lanes_per_row;
  const int sub = lane & (lpr - 1);  // lane within its row group
  const int slot = lane / lpr;       // row group within the wavefront
  const int slots = 64 / lpr;
  const int units = kWaves * slots;  // row groups per workgroup
  const int unit = wave * slots + slot;
  const int64_t n = a.n;
  const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_unit;
  const int64_t r1 = min(a.m, r0 + a.rows_per_unit);
  const int64_t per_batch = (int64_t)units * UNR;  // rows of the workgroup per batch

  float yv[NCH][VEC], acc[NCH][VEC];
  bool cok[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int64_t col0 = ((int64_t)c * lpr + sub) * VEC;
    cok[c] = col0 < n;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      yv[c][k] = (col0 + k < n) ? a.y[col0 + k] : 0.0f;
      acc[c][k] = 0.0f;
    }
  }

  // Row u of a batch for this lane's group: r0 + batch_start + u * units + unit.
  auto process = [&](int64_t start, bool check) {
    XChunk<E, VEC> xv[UNR][NCH];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t row = start + (int64_t)u * units + unit;
      const bool rok = !check || row < r1;
      const E* xr = static_cast<const E*>(a.X) + (rok ? row : r0) * a.ldx;
#pragma unroll
      for (int c = 0; c < NCH; ++c) load_x<E, VEC>(xr, ((int64_t)c * lpr + sub) * VEC, cok[c] && rok, xv[u][c]);
    }
    float s[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      s[u] = 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int k = 0; k < VEC; ++k) s[u] = fmaf(xv[u][c].get(k), yv[c][k], s[u]);
    }
    if constexpr (UNR == 8) {
      if (lpr == 64) {
        // lane i ends with the dot of row i >> 3 of the batch; scale it there, then broadcast
        const float t = wave_sum8_transposed(s);
        const int64_t row = start + (lane >> 3) * (int64_t)units + unit;
        const bool rok = !check || row < r1;
        const float vv = a.v ? (rok ? a.v[row] : 0.0f) : 1.0f;
        const float uu = rok ? vv * t : 0.0f;
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const float uu_b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(uu), 8 * u));
#pragma unroll
          for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[c][k] = fmaf(uu_b, xv[u][c].get(k), acc[c][k]);
        }
        return;
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const float t = group_sum(s[u], lpr);
      const int64_t row = start + (int64_t)u * units + unit;
      const bool rok = !check || row < r1;
      const float vv = a.v ? (rok ? a.v[row] : 0.0f) : 1.0f;
      const float uu = rok ? vv * t : 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[c][k] = fmaf(uu, xv[u][c].get(k), acc[c][k]);
    }
  };

  int64_t start = r0;
  for (; start + per_batch <= r1; start += per_batch) process(start, false);
  if (start < r1) process(start, true);

  // Row groups of a wavefront that own the same columns are combined by lane exchanges,
  // the four wavefronts through LDS, in a fixed order.
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[c][k] = slot_sum(acc[c][k], lpr);
  if (slot == 0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int k = 0; k < VEC; ++k) red[wave][(c * lpr + sub) * VEC + k] = acc[c][k];
  }
  __syncthreads();
  float* dst = a.partial + (int64_t)blockIdx.x * n;
  for (int64_t j = threadIdx.x; j < n; j += kBlock) {
    float t = red[0][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += red[w][j];
    dst[j] = t;
  }
}

// 64-bit exchange slot: the float's bits in the low word, the step tag (step + 1) in the high word.
__device__ __forceinline__ uint64_t pack_slot(float v, uint32_t tag) {
  return ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
}

template <class E, int VEC, int NCH, bool GROUP>
__global__ __launch_bounds__(kBlock) void dense_block_rows(DenseArgs a) {
  constexpr int R = GROUP ? group_rows_per_step(NCH, VEC, (int)sizeof(E)) : block_rows_per_step(NCH, VEC, (int)sizeof(E));
  constexpr int kMaxGroup = kGroupMaxMembers;
  // Group rows (and fp32 block rows of 8 chunks of 4) keep each thread's column sums in LDS, in
  // words no other thread touches (so no barrier guards them); the registers they free hold more
  // rows per exchange of dots (per barrier, for block rows).
  constexpr bool kSumsInLds = GROUP || block_sums_in_lds(NCH, VEC, (int)sizeof(E));
  __shared__ float red[2][R][kWaves];
  __shared__ float gx[GROUP ? R : 1][GROUP ? kMaxGroup : 1];
  __shared__ __align__(16) float acc_s[kSumsInLds ? NCH * kBlock * VEC : 1];  // [chunk][thread][VEC]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = a.n;
  const int gsz = GROUP ? a.group : 1;
  const int64_t unit = GROUP ? blockIdx.x / gsz : blockIdx.x;
  const int member = GROUP ? (int)(blockIdx.x % gsz) : 0;
  const int64_t c0 = (int64_t)member * ((int64_t)kBlock * VEC * NCH);  // first column of this slice
  const int64_t r0 = unit * a.rows_per_unit;
  const int64_t r1 = min(a.m, r0 + a.rows_per_unit);

  float yv[NCH][VEC], acc[kSumsInLds ? 1 : NCH][VEC];
  auto acc_word = [&](int c, int k) -> float& { return acc_s[(c * kBlock + (int)threadIdx.x) * VEC + k]; };
  bool cok[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int64_t col0 = c0 + ((int64_t)c * kBlock + threadIdx.x) * VEC;
    cok[c] = col0 < n;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      yv[c][k] = (col0 + k < n) ? a.y[col0 + k] : 0.0f;
      if constexpr (kSumsInLds) {
        acc_word(c, k) = 0.0f;
      } else {
        acc[c][k] = 0.0f;
      }
    }
  }
  uint64_t* slots = GROUP ? reinterpret_cast<uint64_t*>(a.xchg) + unit * 2 * gsz * R : nullptr;

  // Rows base .. base+R-1 into x (rows past r1 masked to zero, address clamped to row r0).
  auto load_rows = [&](int64_t base, XChunk<E, VEC> (&x)[R][NCH]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = base + r;
      const bool rok = row < r1;
      const E* xr = static_cast<const E*>(a.X) + (rok ? row : r0) * a.ldx;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        load_x<E, VEC>(xr, c0 + ((int64_t)c * kBlock + threadIdx.x) * VEC, cok[c] && rok, x[r][c]);
    }
  };
  // Block rows: when a second set of the step's rows fits in 32 more registers, the next step's
  // rows are requested as soon as this step's dots are formed, so their latency overlaps the
  // barrier and the accumulation instead of adding to them. Group rows do not prefetch: the
  // lanes that wait for the other members' dots would first wait for their own prefetch (the
  // vector-memory counter completes in order), and the second set costs a wave per SIMD
  // (measured slower on 8192 x 65536).
  constexpr int kWordsPerChunk = (VEC * (int)sizeof(E) + 3) / 4;
  constexpr bool kPrefetch = !GROUP && R * NCH * kWordsPerChunk <= 32;
  XChunk<E, VEC> xv[R][NCH];
  XChunk<E, VEC> xn[kPrefetch ? R : 1][kPrefetch ? NCH : 1];
  if constexpr (kPrefetch) {
    if (r0 < r1) load_rows(r0, xv);
  }

  int parity = 0;
  uint32_t step = 0;
  bool gave_up = false;
  for (int64_t base = r0; base < r1; base += R) {
    if constexpr (!kPrefetch) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = base + r;
        const bool rok = row < r1;
        const E* xr = static_cast<const E*>(a.X) + (rok ? row : r0) * a.ldx;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          load_x<E, VEC>(xr, c0 + ((int64_t)c * kBlock + threadIdx.x) * VEC, cok[c] && rok, xv[r][c]);
      }
    }
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s[r] = 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int k = 0; k < VEC; ++k) s[r] = fmaf(xv[r][c].get(k), yv[c][k], s[r]);
      s[r] = group_sum(s[r], 64);
    }
    if constexpr (kPrefetch) {
      if (base + R < r1) load_rows(base + R, xn);  // uniform across the workgroup
    }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) red[parity][r][wave] = s[r];
    }
    __syncthreads();
    float t[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      t[r] = red[parity][r][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) t[r] += red[parity][r][w];
    }
    if constexpr (GROUP) {
      // Publish this slice's dots, then collect every member's for this step. Slot parity
      // lets a member run one step ahead without overwriting values still being read.
      uint64_t* sl = slots + parity * gsz * R;
      const uint32_t tag = step + 1;
      if (threadIdx.x < R) {
        float mine = t[0];
#pragma unroll
        for (int r = 1; r < R; ++r)
          if (threadIdx.x == r) mine = t[r];
        __hip_atomic_store(sl + member * R + threadIdx.x, pack_slot(mine, tag), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      for (int j = threadIdx.x; j < gsz * R; j += kBlock) {  // every member's dot of every row
        const int c = j / R, r = j % R;
        uint64_t w = __hip_atomic_load(sl + c * R + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t spins = 0;
        const uint32_t limit = gave_up ? 0u : a.wait_polls ? a.wait_polls : kSpinLimit;
        const uint32_t want = tag + a.wait_tag_skew;  // skew 0 except under the failure-path test hook
        while ((uint32_t)(w >> 32) != want) {
          if (++spins > limit) {
            gave_up = true;  // the result is flagged as failed: later steps do not wait again
            __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          w = __hip_atomic_load(sl + c * R + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        gx[r][c] = __uint_as_float((uint32_t)w);
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float tr = gx[r][0];
        for (int c = 1; c < gsz; ++c) tr += gx[r][c];
        t[r] = tr;
      }
      ++step;
    }
    float uu[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = base + r;
      const bool rok = row < r1;
      const float vv = a.v ? (rok ? a.v[row] : 0.0f) : 1.0f;
      uu[r] = rok ? vv * t[r] : 0.0f;
    }
    if constexpr (GROUP && sizeof(E) == 2) {
      // 16-bit group rows are widened again for the accumulation rather than kept widened since
      // the dots: the packed words take half the registers, which hold twice the rows per
      // exchange of dots, and the widening is one operation per element
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NCH; ++c) xv[r][c].opaque();
    }
    if constexpr (kSumsInLds) {  // one read and one write of each sum per step, rows in order
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          float s_ck = acc_word(c, k);
#pragma unroll
          for (int r = 0; r < R; ++r) s_ck = fmaf(uu[r], xv[r][c].get(k), s_ck);
          acc_word(c, k) = s_ck;
        }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
          for (int k = 0; k < VEC; ++k) acc[c][k] = fmaf(uu[r], xv[r][c].get(k), acc[c][k]);
    }
    if constexpr (kPrefetch) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NCH; ++c) xv[r][c] = xn[r][c];
    }
    parity ^= 1;
  }

  float* dst = a.partial + unit * n;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      const int64_t col = c0 + ((int64_t)c * kBlock + threadIdx.x) * VEC + k;
      if constexpr (kSumsInLds) {
        if (col < n) dst[col] = acc_word(c, k);
      } else {
        if (col < n) dst[col] = acc[c][k];
      }
    }
}

template <class E, int VEC>
hipError_t launch_wave(const DenseArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  const dim3 grid((unsigned)p.grid), block(kBlock);
  switch (p.chunks) {
    case 1: hipLaunchKernelGGL((dense_wave_rows<E, VEC, 1, 8>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((dense_wave_rows<E, VEC, 2, 4>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((dense_wave_rows<E, VEC, 4, 2>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The wave-row kernel for an element size, chunk width and chunk count (nullptr: none).
const void* wave_kernel_for(int elem_bytes, int vec, int chunks, bool f16 = false) {
#define XTVXY_WAVE(E, V)                                                                       \
  switch (chunks) {                                                                          \
    case 1: return reinterpret_cast<const void*>(&dense_wave_rows<E, V, 1, 8>);              \
    case 2: return reinterpret_cast<const void*>(&dense_wave_rows<E, V, 2, 4>);              \
    case 4: return reinterpret_cast<const void*>(&dense_wave_rows<E, V, 4, 2>);              \
  }                                                                                          \
  return nullptr;
  if (elem_bytes == 4 && vec == 4) { XTVXY_WAVE(float, 4) }
  if (elem_bytes == 4 && vec == 1) { XTVXY_WAVE(float, 1) }
  if (elem_bytes == 2 && vec == 8 && !f16) { XTVXY_WAVE(bf16_t, 8) }
  if (elem_bytes == 2 && vec == 1 && !f16) { XTVXY_WAVE(bf16_t, 1) }
  if (elem_bytes == 2 && vec == 8 && f16) { XTVXY_WAVE(f16_t, 8) }
  if (elem_bytes == 2 && vec == 1 && f16) { XTVXY_WAVE(f16_t, 1) }
#undef XTVXY_WAVE
  return nullptr;
}

template <class E, int VEC, int NCH>
const void* block_kernel(bool group) {
  return group ? reinterpret_cast<const void*>(&dense_block_rows<E, VEC, NCH, true>)
               : reinterpret_cast<const void*>(&dense_block_rows<E, VEC, NCH, false>);
}

template <class E16>
const void* block_kernel_16(int vec, int chunks, bool group) {
  if (vec == 8) {
    switch (chunks) {
      case 1: return block_kernel<E16, 8, 1>(group);
      case 2: return block_kernel<E16, 8, 2>(group);
      case 4: return block_kernel<E16, 8, 4>(group);
    }
  } else if (vec == 1) {
    switch (chunks) {
      case 1: return block_kernel<E16, 1, 1>(group);
      case 2: return block_kernel<E16, 1, 2>(group);
      case 4: return block_kernel<E16, 1, 4>(group);
      case 8: return block_kernel<E16, 1, 8>(group);
    }
  }
  return nullptr;
}

// The block/group-row kernel for an element size (and, for 16-bit elements, bf16 or fp16), chunk
// width and chunk count (nullptr: none). 16-bit chunks of 8 stop at 4 chunks per thread, the same
// registers as 8 fp32 chunks of 4.
const void* block_kernel_for(int elem_bytes, int vec, int chunks, bool group, bool f16 = false) {
  if (elem_bytes == 4 && vec == 4) {
    switch (chunks) {
      case 1: return block_kernel<float, 4, 1>(group);
      case 2: return block_kernel<float, 4, 2>(group);
      case 4: return block_kernel<float, 4, 4>(group);
      case 8: return block_kernel<float, 4, 8>(group);
    }
  } else if (elem_bytes == 4 && vec == 1) {
    switch (chunks) {
      case 1: return block_kernel<float, 1, 1>(group);
      case 2: return block_kernel<float, 1, 2>(group);
      case 4: return block_kernel<float, 1, 4>(group);
      case 8: return block_kernel<float, 1, 8>(group);
    }
  } else if (elem_bytes == 2) {
    return f16 ? block_kernel_16<f16_t>(vec, chunks, group) : block_kernel_16<bf16_t>(vec, chunks, group);
  }
  return nullptr;
}

}  // namespace

namespace {

// Workgroups of kernel k resident per CU, and the device's CU count, cached per (device, kernel):
// the plan queries run on every fused call.
std::mutex g_occ_mutex;
std::map<std::pair<int, const void*>, int> g_occ;

int resident_per_cu(const void* k, int* cus) {
  int dev = 0;
  if (!k || hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(g_occ_mutex);
  auto it = g_occ.find({dev, k});
  auto cu_it = g_occ.find({dev, nullptr});
  if (it != g_occ.end() && cu_it != g_occ.end()) {
    if (cus) *cus = cu_it->second;
    return it->second;
  }
  int per_cu = 0;
  hipDeviceProp_t prop;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kBlock, 0) != hipSuccess ||
      hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return 0;
  g_occ[{dev, k}] = per_cu;
  g_occ[{dev, nullptr}] = prop.multiProcessorCount;
  if (cus) *cus = prop.multiProcessorCount;
  return per_cu;
}

// Group-row launches of one device run one after another, whatever their streams: each waits
// for the previous one to finish, so two grids that each fit the device never hold the slots
// the other's members need. A stream under graph capture keeps the graph's own order.
std::mutex g_group_mutex;
struct GroupLast {
  hipEvent_t done = nullptr;     // recorded after the device's latest group-row launch
  hipStream_t stream = nullptr;  // the stream it was recorded on
};
std::map<int, GroupLast> g_group_last;

hipError_t launch_group_ordered(const void* k, unsigned grid, void** params, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(s, &capture);
  if (e != hipSuccess) return e;
  if (capture != hipStreamCaptureStatusNone) return hipLaunchKernel(k, dim3(grid), dim3(kBlock), params, 0, s);
  std::lock_guard<std::mutex> lock(g_group_mutex);
  GroupLast& last = g_group_last[dev];
  if (!last.done) {
    e = hipEventCreateWithFlags(&last.done, hipEventDisableTiming);
    if (e != hipSuccess) {
      last.done = nullptr;
      return e;
    }
  } else if (last.stream != s) {  // on the same stream, stream order already serialises them
    e = hipStreamWaitEvent(s, last.done, 0);
    if (e != hipSuccess) return e;
  }
  e = hipLaunchKernel(k, dim3(grid), dim3(kBlock), params, 0, s);
  if (e != hipSuccess) return e;
  e = hipEventRecord(last.done, s);
  last.stream = e == hipSuccess ? s : nullptr;
  return e;
}

}  // namespace

// (16-bit elements: the bf16 kernels stand for the fp16 ones, which differ only in the conversion
// at each use; their register counts differ by one at most, which leaves the residency unchanged.)
int dense_resident_per_cu(const xtvxy_launch_params& p, int elem_bytes) {
  const void* k = p.kernel == XTVXY_DENSE_WAVE_ROWS ? wave_kernel_for(elem_bytes, p.vec, p.chunks)
                                                    : block_kernel_for(elem_bytes, p.vec, p.chunks,
                                                                       p.kernel == XTVXY_DENSE_GROUP_ROWS);
  return resident_per_cu(k, nullptr);
}

int64_t dense_group_max_resident(const xtvxy_launch_params& p, int elem_bytes) {
  int cus = 0;
  const int per_cu = resident_per_cu(block_kernel_for(elem_bytes, p.vec, p.chunks, true), &cus);
  return (int64_t)per_cu * cus;
}

hipError_t launch_dense(const DenseArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if (p.block_threads != kBlock || p.grid <= 0 || p.grid > INT32_MAX) return hipErrorInvalidValue;
  switch (p.kernel) {
    case XTVXY_DENSE_WAVE_ROWS:
      if (a.elem_bytes == 4 && p.vec == 4) return launch_wave<float, 4>(a, p, s);
      if (a.elem_bytes == 4 && p.vec == 1) return launch_wave<float, 1>(a, p, s);
      if (a.elem_bytes == 2 && p.vec == 8) return a.f16 ? launch_wave<f16_t, 8>(a, p, s) : launch_wave<bf16_t, 8>(a, p, s);
      if (a.elem_bytes == 2 && p.vec == 1) return a.f16 ? launch_wave<f16_t, 1>(a, p, s) : launch_wave<bf16_t, 1>(a, p, s);
      return hipErrorInvalidValue;
    case XTVXY_DENSE_BLOCK_ROWS: {
      const void* k = block_kernel_for(a.elem_bytes, p.vec, p.chunks, false, a.f16 != 0);
      if (!k) return hipErrorInvalidValue;
      DenseArgs args = a;
      void* params[] = {&args};
      return hipLaunchKernel(k, dim3((unsigned)p.grid), dim3(kBlock), params, 0, s);
    }
    case XTVXY_DENSE_GROUP_ROWS: {
      if (p.group < 1 || p.group > kGroupMaxMembers) return hipErrorInvalidValue;
      const void* k = block_kernel_for(a.elem_bytes, p.vec, p.chunks, true, a.f16 != 0);
      if (!k) return hipErrorInvalidValue;
      DenseArgs args = a;
      void* params[] = {&args};
      return launch_group_ordered(k, (unsigned)p.grid, params, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace xtvxy
