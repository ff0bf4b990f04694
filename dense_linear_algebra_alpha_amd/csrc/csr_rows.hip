// Fused CSR kernel by row classes, for out = alpha * X^T (v .* (X y)) + beta * z, and the
// kernels of the structure analysis it runs on.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract): one fused kernel with
// techniques specific to sparse X, launch parameters chosen from the input's characteristics.
// Here the characteristics are taken from the matrix's structure once (xtvxy_csr_f32_analyse):
//   - columns are relabelled by how many entries they hold, the most frequent first, so that the
//     LDS windows (output columns [0, W), y [0, Wy)) hold the hottest columns of any matrix;
//   - nonempty rows are grouped by length class c: a class-c row has at most 16 * 2^c - 3
//     entries, so a group of 2^c lanes holding 16 entry slots each (four 16-byte quads, the
//     quads of a group interleaved so that its lanes read consecutive quads) covers all of the
//     row's quads whatever its first entry mod 4; rows of more than 1021 entries form the "very
//     long" class, taken by a whole wavefront in slices of 1024 slots;
//   - the rows of each class are cut into work units of about kRowsUnitEntries entries (one row
//     per unit for very long rows), and unit_prefix counts the entries before each unit.
// Every wavefront works alone: wavefront g of G takes the units that start in the g-th of G equal
// parts of the entries (a 64-way search of unit_prefix). A batch of a class-c unit is 64 / 2^c rows,
// one per lane group:
//   1. the group's lanes load the row's quads (only quads that hold entries of the row), and
//      gather y at each entry's column from the LDS copy of y (columns < Wy) or global memory;
//   2. each lane sums its products, the group sums its lanes (DPP butterflies), and
//      u_row = v_row * dot is in every lane of the group; every slot outside the row is masked
//      out of the product itself, so values of neighbouring rows never enter;
//   3. the products u_row * value are scattered from registers: columns < W into the
//      workgroup's LDS copy of the output (compare-and-swap adds), the others into the
//      wavefront's bins (the chunk pool and bin passes of csr_bins.hip) or global atomics.
// A very long row is swept twice: the dot over all its slices (the first slice kept in registers),
// then the scatter (the other slices loaded again, from L2 by then).
#include "csr_common.h"
#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

typedef int32_t i4 __attribute__((ext_vector_type(4)));

constexpr int kQuads = kRowsSlots / 4;  // 16-byte quads per lane

template <int BLK, int YMODE, int COLD>
__global__ __launch_bounds__(BLK) void csr_rows(CsrArgs a) {
  static_assert(BLK == 256 || BLK == 512 || BLK == 1024, "workgroups of 256, 512 or 1024 threads");
  constexpr int NW = BLK / 64;
  constexpr int K = kRowsSlots;
  constexpr bool BINNED = COLD == kColdBinned;
  constexpr uint32_t S = kBinChunkItems;
  extern __shared__ __align__(16) float dyn[];
  float* out_s = dyn;                 // [lds_window], shared by the wavefronts
  float* y_s = dyn + a.lds_window;    // [y_window]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t nnz = (uint32_t)a.nnz;
  const int32_t window = (int32_t)a.lds_window;
  const int32_t y_window = YMODE == kYGlobal ? 0 : (int32_t)a.y_window;
  const bool aligned = a.aligned;
  const float* __restrict__ values = a.values;
  const int32_t* __restrict__ cols = a.col_idx;

  for (int32_t j = tid; j < window; j += BLK) out_s[j] = 0.0f;
  for (int32_t j = tid; j < y_window; j += BLK) y_s[j] = a.y[j];
  // This wavefront's bins (columns >= window), as in the wavefront kernel: per bin the ranks
  // handed out in the current batch, the current chunk and its fill, and for the batch's writers
  // the chunk and fill the batch started from and the first of the new chunks it took.
  const int bins = BINNED ? a.bins : 0;
  const uint64_t pool_items = (uint64_t)a.pool_chunks * S;
  uint32_t* cnt_w = nullptr;
  int32_t* cur_w = nullptr;
  uint32_t* fill_w = nullptr;
  int32_t* oc_w = nullptr;
  uint32_t* of_w = nullptr;
  uint32_t* first_w = nullptr;
  if constexpr (BINNED) {
    uint32_t* bs = reinterpret_cast<uint32_t*>(dyn + a.lds_window + y_window) + (size_t)wave * 6 * bins;
    cnt_w = bs;
    cur_w = reinterpret_cast<int32_t*>(bs + bins);
    fill_w = bs + 2 * bins;
    oc_w = reinterpret_cast<int32_t*>(bs + 3 * bins);
    of_w = bs + 4 * bins;
    first_w = bs + 5 * bins;
    for (int t = lane; t < bins; t += 64) {
      cnt_w[t] = 0u;
      cur_w[t] = -1;
      fill_w[t] = S;
    }
  }
  __syncthreads();

  auto gather_y = [&](int32_t col) -> float {
    if constexpr (YMODE == kYGlobal) return a.y[col];
    if constexpr (YMODE == kYLds) return y_s[col];
    return col < y_window ? y_s[col] : a.y[col];
  };
  // The four entries of the quad at p (p a multiple of 4, p < nnz): one 16-byte load of values and
  // one of columns when the arrays are 16-byte aligned and the quad is whole, else element loads
  // clamped to the last entry (their slots past nnz are outside every row).
  auto load_quad = [&](uint32_t p, float* v4, int32_t* c4) {
    if (aligned && p + 4u <= nnz) {
      const f4 vv = *reinterpret_cast<const f4*>(values + p);
      const i4 cc = *reinterpret_cast<const i4*>(cols + p);
      v4[0] = vv.x; v4[1] = vv.y; v4[2] = vv.z; v4[3] = vv.w;
      c4[0] = cc.x; c4[1] = cc.y; c4[2] = cc.z; c4[3] = cc.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t q = min(p + (uint32_t)i, nnz - 1u);
        v4[i] = values[q];
        c4[i] = cols[q];
      }
    }
  };
  // The K slots of this lane for the row [s, e): quad k starts at qbase + 4 (j + stride k); only
  // quads that hold entries of the row are loaded; on[] marks the slots inside the row.
  auto load_slots = [&](uint32_t qbase, int j, int stride, uint32_t s, uint32_t e, float (&val)[K],
                        int32_t (&col)[K], bool (&on)[K]) {
#pragma unroll
    for (int k = 0; k < kQuads; ++k) {
      const uint32_t p = qbase + 4u * (uint32_t)(j + stride * k);
      if (p < e) {
        load_quad(p, &val[4 * k], &col[4 * k]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          val[4 * k + i] = 0.0f;
          col[4 * k + i] = 0;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) on[4 * k + i] = p + (uint32_t)i >= s && p + (uint32_t)i < e;
    }
  };
  // This lane's share of the row's dot product (slots outside the row contribute nothing, not
  // even a NaN or Inf of a neighbouring row).
  auto lane_dot = [&](const float (&val)[K], const int32_t (&col)[K], const bool (&on)[K]) -> float {
    float yv[K];
#pragma unroll
    for (int t = 0; t < K; ++t) yv[t] = on[t] ? gather_y(col[t]) : 0.0f;
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < K; ++t) part += on[t] ? val[t] * yv[t] : 0.0f;
    return part;
  };

  // Scatter of the products u * val[t] of the slots inside the row.
  auto scatter = [&](float u, const float (&val)[K], const int32_t (&col)[K], const bool (&on)[K]) {
    if constexpr (COLD == kColdNone) {
#pragma unroll
      for (int t = 0; t < K; ++t)
        if (on[t]) lds_add_f32(out_s + col[t], u * val[t]);
    } else if constexpr (COLD == kColdAtomic) {
#pragma unroll
      for (int t = 0; t < K; ++t) {
        if (on[t]) {
          if (col[t] < window)
            lds_add_f32(out_s + col[t], u * val[t]);
          else
            __hip_atomic_fetch_add((global_float*)a.acc + col[t], u * val[t], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    } else {
      // ranks within the wavefront's batch of each bin
      uint32_t rank[K];
#pragma unroll
      for (int t = 0; t < K; ++t) {
        rank[t] = 0u;
        if (on[t] && col[t] >= window) {
          const int bin = (col[t] - window) >> a.bin_shift;
          rank[t] = __hip_atomic_fetch_add((lds_uint*)(cnt_w + bin), 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WAVEFRONT);
        }
      }
      wave_lds_sync();
      // room for the batch: one lane per bin; a bin that spills takes new consecutive chunks
      // from the pool with one global atomic
      for (int t = lane; t < bins; t += 64) {
        const uint32_t cnt = cnt_w[t];
        if (cnt == 0u) continue;
        cnt_w[t] = 0u;
        const int32_t cur = cur_w[t];
        const uint32_t fill = fill_w[t];
        oc_w[t] = cur;
        of_w[t] = fill;
        const uint32_t room = cur >= 0 ? S - fill : 0u;
        if (cnt <= room) {
          fill_w[t] = fill + cnt;
          continue;
        }
        const uint32_t need = cnt - room, kc = (need + S - 1u) / S;
        const uint32_t first =
            __hip_atomic_fetch_add((global_uint*)a.pool_next, kc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int64_t)first + kc > a.pool_chunks) {  // cannot happen with the pool sized for the plan
          first_w[t] = (uint32_t)a.pool_chunks;   // the items are dropped rather than written out of bounds
          cur_w[t] = -1;
          fill_w[t] = S;
          continue;
        }
        for (uint32_t q = 0; q < kc; ++q) {
          a.chunk_bin[first + q] = t;
          a.chunk_fill[first + q] = (int32_t)S;  // the last one is corrected when it stops filling
        }
        first_w[t] = first;
        cur_w[t] = (int32_t)(first + kc - 1u);
        fill_w[t] = need - (kc - 1u) * S;
      }
      // the window's products while the chunk hand-out completes
#pragma unroll
      for (int t = 0; t < K; ++t)
        if (on[t] && col[t] < window) lds_add_f32(out_s + col[t], u * val[t]);
      wave_lds_sync();
#pragma unroll
      for (int t = 0; t < K; ++t) {
        if (on[t] && col[t] >= window) {
          const int bin = (col[t] - window) >> a.bin_shift;
          const int32_t oc = oc_w[bin];
          const uint32_t of = of_w[bin];
          const uint32_t room = oc >= 0 ? S - of : 0u;
          const uint64_t pos = rank[t] < room ? (uint64_t)oc * S + of + rank[t]
                                              : (uint64_t)first_w[bin] * S + (rank[t] - room);
          if (pos < pool_items) a.pool[pos] = make_int2(col[t], __float_as_int(u * val[t]));
        }
      }
      wave_lds_sync();  // the batch's reads of the bin state come before the next batch's ranks
    }
  };

  // One batch of a class-c unit: row b + (lane >> c) of the unit for each group of 2^c lanes.
  auto batch = [&](int32_t first, int32_t count, int c, int32_t b) {
    const int gsz = 1 << c;
    const int j = lane & (gsz - 1);
    const int32_t idx = b + (lane >> c);
    const bool has = idx < count;
    const int32_t r = a.rows[first + (has ? idx : count - 1)];
    const uint32_t s = (uint32_t)a.row_ptr[r];
    const uint32_t e = has ? (uint32_t)a.row_ptr[r + 1] : s;  // a group without a row: no slots
    const float vr = a.v ? a.v[r] : 1.0f;
    float val[K];
    int32_t col[K];
    bool on[K];
    load_slots(s & ~3u, j, gsz, s, e, val, col, on);
    const float u = vr * group_sum(lane_dot(val, col, on), gsz);
    scatter(u, val, col, on);
  };

  // A row of more than 1021 entries, by the whole wavefront in slices of 64 K slots.
  auto very_long = [&](int32_t r) {
    const uint32_t s = (uint32_t)a.row_ptr[r], e = (uint32_t)a.row_ptr[r + 1];
    const float vr = a.v ? a.v[r] : 1.0f;
    const uint32_t base = s & ~3u;
    float val0[K];
    int32_t col0[K];
    bool on0[K];
    load_slots(base, lane, 64, s, e, val0, col0, on0);
    float part = lane_dot(val0, col0, on0);
    for (uint32_t sb = base + 64u * K; sb < e; sb += 64u * K) {
      float val[K];
      int32_t col[K];
      bool on[K];
      load_slots(sb, lane, 64, s, e, val, col, on);
      part += lane_dot(val, col, on);
    }
    const float u = vr * group_sum(part, 64);
    scatter(u, val0, col0, on0);
    for (uint32_t sb = base + 64u * K; sb < e; sb += 64u * K) {
      float val[K];
      int32_t col[K];
      bool on[K];
      load_slots(sb, lane, 64, s, e, val, col, on);
      scatter(u, val, col, on);
    }
  };

  // This wavefront's units: those that start in its share of the entries.
  const int64_t G = (int64_t)gridDim.x * NW, g = (int64_t)blockIdx.x * NW + wave;
  const int64_t total = a.unit_prefix[a.units_count];
  const int64_t q = (total + G - 1) / G;
  int32_t ub = (int32_t)wave_lower_bound(a.unit_prefix, a.units_count, g * q);
  int32_t ue = g + 1 == G ? a.units_count : (int32_t)wave_lower_bound(a.unit_prefix, a.units_count, (g + 1) * q);
  ub = __builtin_amdgcn_readfirstlane(ub);
  ue = __builtin_amdgcn_readfirstlane(ue);
  for (int32_t un = ub; un < ue; ++un) {
    const int32_t first = a.units[4 * un], count = a.units[4 * un + 1], c = a.units[4 * un + 2];
    if (c == kRowsVeryLong) {
      for (int32_t k = 0; k < count; ++k) very_long(a.rows[first + k]);
    } else {
      const int32_t per = 64 >> c;
      for (int32_t b = 0; b < count; b += per) batch(first, count, c, b);
    }
  }

  if constexpr (BINNED) {
    // the fill of each bin's last chunk (every other handed-out chunk is full)
    for (int t = lane; t < bins; t += 64)
      if (cur_w[t] >= 0) a.chunk_fill[cur_w[t]] = (int32_t)fill_w[t];
  }
  __syncthreads();
  if (window > 0) {
    float* dst = a.partial + (int64_t)blockIdx.x * window;
    for (int32_t c = tid; c < window; c += BLK) dst[c] = out_s[c];
  }
}

template <int BLK, int YMODE, int COLD>
hipError_t launch_r(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  const size_t lds = csr_waves_dynamic_lds(a.lds_window, YMODE == kYGlobal ? 0 : a.y_window, a.bins, BLK);
  const void* fn = reinterpret_cast<const void*>(&csr_rows<BLK, YMODE, COLD>);
  hipError_t e = allow_dynamic_lds(fn);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((csr_rows<BLK, YMODE, COLD>), dim3((unsigned)p.grid), dim3(BLK), lds, s, a);
  return hipGetLastError();
}

template <int BLK, int COLD>
hipError_t launch_ry(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if (a.y_window >= a.n) return launch_r<BLK, kYLds, COLD>(a, p, s);
  if (a.y_window > 0) return launch_r<BLK, kYSplit, COLD>(a, p, s);
  return launch_r<BLK, kYGlobal, COLD>(a, p, s);
}

template <int BLK>
hipError_t launch_rc(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if (a.bins > 0) return launch_ry<BLK, kColdBinned>(a, p, s);
  if (a.lds_window < a.n) return launch_ry<BLK, kColdAtomic>(a, p, s);
  return launch_ry<BLK, kColdNone>(a, p, s);
}

__global__ void col_count_kernel(const int32_t* __restrict__ col, int64_t nnz, uint32_t* counts) {
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < nnz; p += (int64_t)gridDim.x * blockDim.x)
    atomicAdd(counts + col[p], 1u);
}

__global__ void relabel_kernel(const int32_t* __restrict__ col, int64_t nnz, const int32_t* __restrict__ slot,
                               int32_t* __restrict__ out) {
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < nnz; p += (int64_t)gridDim.x * blockDim.x)
    out[p] = slot[col[p]];
}

__global__ void permute_kernel(const float* __restrict__ y, const int32_t* __restrict__ perm, int64_t n,
                               float* __restrict__ yp) {
  for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < n; s += (int64_t)gridDim.x * blockDim.x)
    yp[s] = y[perm[s]];
}

unsigned stream_grid(int64_t count) {
  int64_t g = (count + 255) / 256;
  return (unsigned)(g < 1 ? 1 : g > 8192 ? 8192 : g);
}

}  // namespace

hipError_t launch_csr_rows(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if (p.grid <= 0 || p.grid > INT32_MAX || p.kernel != XTVXY_CSR_ROWS || p.entries_per_thread != kRowsSlots)
    return hipErrorInvalidValue;
  if (a.nnz <= 0 || a.nnz > INT32_MAX || a.m <= 0 || a.m > INT32_MAX - 1024 || a.lds_window < 0 ||
      a.lds_window > a.n || a.y_window < 0 || a.y_window > a.n || a.rows == nullptr || a.units == nullptr ||
      a.unit_prefix == nullptr || a.units_count < 0)
    return hipErrorInvalidValue;
  const bool binned = a.bins > 0;
  if (binned && (a.pool == nullptr || a.pool_next == nullptr || a.chunk_bin == nullptr || a.chunk_fill == nullptr ||
                 a.bins > kMaxBins || a.acc != nullptr))
    return hipErrorInvalidValue;
  if (!binned && a.lds_window < a.n && a.acc == nullptr) return hipErrorInvalidValue;
  if (p.block_threads == 256) return launch_rc<256>(a, p, s);
  if (p.block_threads == 512) return launch_rc<512>(a, p, s);
  if (p.block_threads == 1024) return launch_rc<1024>(a, p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_col_count(const int32_t* col_idx, int64_t nnz, uint32_t* counts, hipStream_t s) {
  if (nnz <= 0) return hipSuccess;
  hipLaunchKernelGGL(col_count_kernel, dim3(stream_grid(nnz)), dim3(256), 0, s, col_idx, nnz, counts);
  return hipGetLastError();
}

hipError_t launch_relabel(const int32_t* col_idx, int64_t nnz, const int32_t* slot, int32_t* out, hipStream_t s) {
  if (nnz <= 0) return hipSuccess;
  hipLaunchKernelGGL(relabel_kernel, dim3(stream_grid(nnz)), dim3(256), 0, s, col_idx, nnz, slot, out);
  return hipGetLastError();
}

hipError_t launch_permute(const float* y, const int32_t* perm, int64_t n, float* yp, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kernel, dim3(stream_grid(n)), dim3(256), 0, s, y, perm, n, yp);
  return hipGetLastError();
}

}  // namespace xtvxy
