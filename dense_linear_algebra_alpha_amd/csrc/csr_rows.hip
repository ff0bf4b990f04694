// Fused CSR kernel by row classes, for out = alpha * X^T (v .* (X y)) + beta * z, and the
// kernels of the structure analysis it runs on.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract): one fused kernel with
// techniques specific to sparse X, launch parameters chosen from the input's characteristics.
// Here the characteristics are taken from the matrix's structure once (xtvxy_csr_f32_analyse):
//   - columns are relabelled by how many entries they hold, the most frequent first, so that the
//     LDS windows (output columns [0, W), y [0, Wy)) hold the hottest columns of any matrix;
//   - nonempty rows are grouped by length class c: a class-c row has at most 8 * 2^c - 3 entries,
//     so a group of 2^c lanes holding 8 entry slots each (two 16-byte quads, the quads of a group
//     interleaved so that its lanes read consecutive quads) covers all of the row's quads
//     whatever its first entry mod 4; rows of more than 509 entries form the "very long" class,
//     taken by a whole wavefront in slices of 512 slots;
//   - a batch is 64 / 2^c rows of one class (a row per lane group), or one very long row; each
//     batch's rows are listed with their entry bounds, and batch_prefix counts the entries
//     before each batch.
// Every wavefront works alone: wavefront g of G takes the batches that start in the g-th of G
// equal parts of the entries (a 64-way search of batch_prefix). Batches are ordered very long rows
// first, so a wavefront takes its very long rows (if any) and then its short-row batches, these in
// a software pipeline: while batch k is processed, the next batch's quads and v are in flight and
// the bounds of the one after; the next batch's y gathers are issued as soon as its quads have
// arrived. (The vector-memory counter completes in order, so the loads are issued in the order
// they are waited for, and none is issued under a branch.) For each batch:
//   1. each lane's quads (quads past the row's last quad re-read it: no other row's bytes) and
//      y at each entry's column, from the LDS copy of y (columns < Wy) and global memory;
//   2. each lane sums its products, the group sums its lanes (DPP butterflies), and
//      u_row = v_row * dot is in every lane of the group; every slot outside the row is masked
//      out of the product itself, so values of neighbouring rows never enter;
//   3. the products u_row * value are scattered from registers: columns < W into the workgroup's
//      LDS copy of the output (compare-and-swap adds, all of a lane's issued before any is
//      checked), the others into the wavefront's bins (the chunk pool and bin passes of
//      csr_bins.hip) or global atomics.
// A very long row is swept twice: the dot over all its slices (the first slice kept in registers),
// then the scatter (the other slices loaded again, from L2 by then).
#include "csr_common.h"
#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

typedef int32_t i4 __attribute__((ext_vector_type(4)));
typedef int32_t i2 __attribute__((ext_vector_type(2)));

constexpr int kQuads = kRowsSlots / 4;  // 16-byte quads per lane

template <int BLK, int YMODE, int COLD, bool ALIGNED>
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
  const uint32_t nnz_full = nnz & ~3u;  // entries in whole quads
  const float* __restrict__ values = static_cast<const float*>(a.values);  // fp32 only (checked at launch)
  const int32_t* __restrict__ cols = a.col_idx;
  const int bins = BINNED ? a.bins : 0;
  // after the windows: a sink word per thread (masked-off LDS adds), then this wavefront's bins
  float* sink = dyn + a.lds_window + y_window + tid;

  for (int32_t j = tid; j < window; j += BLK) out_s[j] = 0.0f;
  for (int32_t j = tid; j < y_window; j += BLK) y_s[j] = a.y[j];
  *sink = 0.0f;
  // This wavefront's bins (columns >= window), as in the wavefront kernel: per bin the ranks
  // handed out in the current batch, the current chunk and its fill, and for the batch's writers
  // the chunk and fill the batch started from and the first of the new chunks it took.
  const uint64_t pool_items = (uint64_t)a.pool_chunks * S;
  uint32_t* cnt_w = nullptr;
  int32_t* cur_w = nullptr;
  uint32_t* fill_w = nullptr;
  int32_t* oc_w = nullptr;
  uint32_t* of_w = nullptr;
  uint32_t* first_w = nullptr;
  if constexpr (BINNED) {
    uint32_t* bs = reinterpret_cast<uint32_t*>(dyn + a.lds_window + y_window + BLK) + (size_t)wave * 6 * bins;
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

  // y at column `col`, with no branch around the loads: from LDS and from global memory both,
  // lanes whose column is in the LDS copy reading y[0] from global memory (one line for all).
  auto gather_y = [&](int32_t col) -> float {
    if constexpr (YMODE == kYGlobal) return a.y[col];
    if constexpr (YMODE == kYLds) return y_s[col];
    const float fast = y_s[min(col, y_window - 1)];
    const float slow = a.y[col < y_window ? 0 : col];
    return col < y_window ? fast : slow;
  };

  // A batch's slots in one lane: values, columns (0 outside the row) and which slots are inside.
  struct Slots {
    float val[K];
    int32_t col[K];
    uint32_t on;  // bit t: slot t holds an entry of the row
  };
  // The K slots of this lane for the row [s, e): quad k starts at qbase + 4 (j + stride k). Every
  // quad is loaded, without a branch: quads past the row's last quad read that last quad again
  // (the same lines), so no other row's bytes are fetched. With 16-byte aligned arrays a quad is
  // two 16-byte loads, a quad at or past the last whole quad of the arrays reads the last whole
  // quad instead (the launch guarantees nnz >= 4) and its up to three entries beyond are patched
  // in by element loads (a branch taken by the lanes of the matrix's last row only); unaligned
  // arrays are read by element loads clamped to nnz - 1.
  auto load_slots = [&](uint32_t qbase, int j, int stride, uint32_t s, uint32_t e, Slots& sl) {
    const uint32_t last = e > s ? (e - 1u) & ~3u : s & ~3u;  // the row's last quad (an empty row: any)
    sl.on = 0u;
#pragma unroll
    for (int k = 0; k < kQuads; ++k) {
      const uint32_t p = qbase + 4u * (uint32_t)(j + stride * k);
      const uint32_t pq = min(p, last);
      if constexpr (ALIGNED) {
        const uint32_t pl = min(pq, nnz_full - 4u);
        const f4 vv = *reinterpret_cast<const f4*>(values + pl);
        const i4 cc = *reinterpret_cast<const i4*>(cols + pl);
        sl.val[4 * k] = vv.x; sl.val[4 * k + 1] = vv.y; sl.val[4 * k + 2] = vv.z; sl.val[4 * k + 3] = vv.w;
        sl.col[4 * k] = cc.x; sl.col[4 * k + 1] = cc.y; sl.col[4 * k + 2] = cc.z; sl.col[4 * k + 3] = cc.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t q = min(pq + (uint32_t)i, nnz - 1u);
          sl.val[4 * k + i] = values[q];
          sl.col[4 * k + i] = cols[q];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sl.on |= (p + (uint32_t)i >= s && p + (uint32_t)i < e) ? 1u << (4 * k + i) : 0u;
    }
    if constexpr (ALIGNED) {
      if (nnz != nnz_full && e > nnz_full) {  // the row holds entries after the last whole quad
#pragma unroll
        for (int k = 0; k < kQuads; ++k) {
          const uint32_t p = qbase + 4u * (uint32_t)(j + stride * k);
          if (p == nnz_full) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (p + (uint32_t)i < nnz) {
                sl.val[4 * k + i] = values[p + i];
                sl.col[4 * k + i] = cols[p + i];
              }
            }
          }
        }
      }
    }
  };
  auto slot_on = [](const Slots& sl, int t) { return ((sl.on >> t) & 1u) != 0u; };
  // y at every slot's column (slots outside the row: column 0)
  auto gather_slots = [&](const Slots& sl, float (&yv)[K]) {
#pragma unroll
    for (int t = 0; t < K; ++t) yv[t] = gather_y(slot_on(sl, t) ? sl.col[t] : 0);
  };
  // This lane's share of the row's dot product (slots outside the row contribute nothing, not even
  // a NaN or Inf of a neighbouring row).
  auto lane_dot = [&](const Slots& sl, const float (&yv)[K]) -> float {
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < K; ++t) part += slot_on(sl, t) ? sl.val[t] * yv[t] : 0.0f;
    return part;
  };
  // LDS adds of c[t] to out_s[col[t]] for the slots in `mask` (the others add 0 to this thread's
  // sink word): every compare-and-swap is issued before any is checked, and the slots that lost
  // theirs to another writer use the native LDS float add.
  auto window_adds = [&](const Slots& sl, const float (&c)[K], uint32_t mask) {
    float* adr[K];
    float add[K];
    unsigned int old[K];
#pragma unroll
    for (int t = 0; t < K; ++t) {
      const bool on = ((mask >> t) & 1u) != 0u;
      adr[t] = on ? out_s + sl.col[t] : sink;
      add[t] = on ? c[t] : 0.0f;
      old[t] = *(lds_uint*)adr[t];
    }
    bool ok[K];
#pragma unroll
    for (int t = 0; t < K; ++t) {
      unsigned int expected = old[t];
      ok[t] = __hip_atomic_compare_exchange_strong((lds_uint*)adr[t], &expected,
                                                   __float_as_uint(__uint_as_float(old[t]) + add[t]),
                                                   __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
#pragma unroll
    for (int t = 0; t < K; ++t)
      if (!ok[t]) __builtin_amdgcn_ds_faddf((lds_float*)adr[t], add[t], 0, 0, false);
  };

  // Scatter of the products u * val[t] of the slots inside the row.
  auto scatter = [&](float u, const Slots& sl) {
    float c[K];
#pragma unroll
    for (int t = 0; t < K; ++t) c[t] = u * sl.val[t];
    uint32_t hot = 0u;
#pragma unroll
    for (int t = 0; t < K; ++t) hot |= (slot_on(sl, t) && sl.col[t] < window) ? 1u << t : 0u;
    const uint32_t cold = sl.on & ~hot;
    if constexpr (COLD == kColdNone) {
      window_adds(sl, c, sl.on);
    } else if constexpr (COLD == kColdAtomic) {
      window_adds(sl, c, hot);
#pragma unroll
      for (int t = 0; t < K; ++t)
        if ((cold >> t) & 1u)
          __hip_atomic_fetch_add((global_float*)a.acc + sl.col[t], c[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // ranks within the wavefront's batch of each bin
      uint32_t rank[K];
#pragma unroll
      for (int t = 0; t < K; ++t) {
        rank[t] = 0u;
        if ((cold >> t) & 1u) {
          const int bin = (sl.col[t] - window) >> a.bin_shift;
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
      window_adds(sl, c, hot);
      wave_lds_sync();
#pragma unroll
      for (int t = 0; t < K; ++t) {
        if ((cold >> t) & 1u) {
          const int bin = (sl.col[t] - window) >> a.bin_shift;
          const int32_t oc = oc_w[bin];
          const uint32_t of = of_w[bin];
          const uint32_t room = oc >= 0 ? S - of : 0u;
          const uint64_t pos = rank[t] < room ? (uint64_t)oc * S + of + rank[t]
                                              : (uint64_t)first_w[bin] * S + (rank[t] - room);
          if (pos < pool_items) a.pool[pos] = make_int2(sl.col[t], __float_as_int(c[t]));
        }
      }
      wave_lds_sync();  // the batch's reads of the bin state come before the next batch's ranks
    }
  };

  // A row of more than 509 entries, by the whole wavefront in slices of 64 K slots.
  auto very_long = [&](int32_t r, uint32_t s, uint32_t e) {
    const float vr = a.v ? a.v[r] : 1.0f;
    const uint32_t base = s & ~3u;
    Slots s0;
    float y0[K];
    load_slots(base, lane, 64, s, e, s0);
    gather_slots(s0, y0);
    float part = lane_dot(s0, y0);
    for (uint32_t sb = base + 64u * K; sb < e; sb += 64u * K) {
      Slots sl;
      float yv[K];
      load_slots(sb, lane, 64, s, e, sl);
      gather_slots(sl, yv);
      part += lane_dot(sl, yv);
    }
    const float u = vr * group_sum(part, 64);
    scatter(u, s0);
    for (uint32_t sb = base + 64u * K; sb < e; sb += 64u * K) {
      Slots sl;
      load_slots(sb, lane, 64, s, e, sl);
      scatter(u, sl);
    }
  };

  // This wavefront's batches: those that start in its share of the entries.
  const int64_t G = (int64_t)gridDim.x * NW, g = (int64_t)blockIdx.x * NW + wave;
  const int64_t total = a.batch_prefix[a.batches_count];
  const int64_t q = (total + G - 1) / G;
  int32_t kb = (int32_t)wave_lower_bound(a.batch_prefix, a.batches_count, g * q);
  int32_t ke = g + 1 == G ? a.batches_count : (int32_t)wave_lower_bound(a.batch_prefix, a.batches_count, (g + 1) * q);
  kb = __builtin_amdgcn_readfirstlane(kb);
  ke = __builtin_amdgcn_readfirstlane(ke);
  const int32_t* __restrict__ bt = a.batches;
  // very long rows first (the batches are ordered by class, very long first)
  while (kb < ke && (bt[2 * kb + 1] >> 8) == kRowsVeryLong) {
    const int32_t pos = bt[2 * kb];
    very_long(a.rows[pos], (uint32_t)a.bounds[2 * pos], (uint32_t)a.bounds[2 * pos + 1]);
    ++kb;
  }

  // Short-row batches in a pipeline. Per batch k (A = batch k, B = batch k + 1):
  //   1. B's quads (its bounds arrived one step ago) and B's v;
  //   2. the bounds of batch k + 2 into A's bounds (A's are no longer needed);
  //   3. A's dot (its gathers were issued at the end of the previous step) and scatter;
  //   4. B's gathers, once B's quads have arrived.
  // Each wait covers only loads issued before the ones still in flight.
  struct Bounds {
    uint32_t s, e;
    int32_t r;
  };
  auto load_bounds = [&](int32_t k, Bounds& b) {
    const int32_t first = bt[2 * k], w = bt[2 * k + 1];
    const int c = w >> 8, cnt = w & 255;
    const int gi = lane >> c;
    const int32_t pos = first + min(gi, cnt - 1);
    const i2 se = *reinterpret_cast<const i2*>(a.bounds + 2 * pos);
    b.r = a.rows[pos];
    b.s = (uint32_t)se.x;
    b.e = gi < cnt ? (uint32_t)se.y : (uint32_t)se.x;  // a group without a row: no slots
  };
  auto class_of = [&](int32_t k) { return bt[2 * k + 1] >> 8; };
  auto issue = [&](int32_t k, const Bounds& b, Slots& sl, float& v) {
    const int c = class_of(k), gsz = 1 << c;
    load_slots(b.s & ~3u, lane & (gsz - 1), gsz, b.s, b.e, sl);
    v = a.v ? a.v[b.r] : 1.0f;
  };
  auto finish = [&](int32_t k, const Slots& sl, const float (&yv)[K], float v) {
    const int c = class_of(k);
    const float u = v * group_sum(lane_dot(sl, yv), 1 << c);
    scatter(u, sl);
  };
  if (kb < ke) {
    Bounds ba, bb;
    Slots sa, sb;
    float ya[K], yb[K];
    float va = 1.0f, vb = 1.0f;
    load_bounds(kb, ba);
    issue(kb, ba, sa, va);
    if (kb + 1 < ke) load_bounds(kb + 1, bb);
    gather_slots(sa, ya);
    int32_t k = kb;
    // one step: current batch in (sc, yc, vc), next in (bn -> sn, yn, vn); bc receives the bounds
    // of the batch after next
    auto step = [&](Bounds& bc, Slots& sc, float (&yc)[K], float& vc, Bounds& bn, Slots& sn, float (&yn)[K],
                    float& vn) -> bool {
      const bool next = k + 1 < ke;
      if (next) issue(k + 1, bn, sn, vn);
      if (k + 2 < ke) load_bounds(k + 2, bc);
      finish(k, sc, yc, vc);
      if (next) gather_slots(sn, yn);
      ++k;
      return next;
    };
    while (step(ba, sa, ya, va, bb, sb, yb, vb) && step(bb, sb, yb, vb, ba, sa, ya, va)) {
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

template <int BLK, int YMODE, int COLD, bool ALIGNED>
hipError_t launch_r(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  const size_t lds = csr_rows_dynamic_lds(a.lds_window, YMODE == kYGlobal ? 0 : a.y_window, a.bins, BLK);
  const void* fn = reinterpret_cast<const void*>(&csr_rows<BLK, YMODE, COLD, ALIGNED>);
  hipError_t e = allow_dynamic_lds(fn);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((csr_rows<BLK, YMODE, COLD, ALIGNED>), dim3((unsigned)p.grid), dim3(BLK), lds, s, a);
  return hipGetLastError();
}

template <int BLK, int YMODE, int COLD>
hipError_t launch_ra(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  // 16-byte loads need 16-byte aligned arrays and one whole quad of entries
  return a.aligned && a.nnz >= 4 ? launch_r<BLK, YMODE, COLD, true>(a, p, s) : launch_r<BLK, YMODE, COLD, false>(a, p, s);
}

template <int BLK, int COLD>
hipError_t launch_ry(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if (a.y_window >= a.n) return launch_ra<BLK, kYLds, COLD>(a, p, s);
  if (a.y_window > 0) return launch_ra<BLK, kYSplit, COLD>(a, p, s);
  return launch_ra<BLK, kYGlobal, COLD>(a, p, s);
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
      a.lds_window > a.n || a.y_window < 0 || a.y_window > a.n || a.rows == nullptr || a.bounds == nullptr ||
      a.batches == nullptr || a.batch_prefix == nullptr || a.batches_count < 0 || a.value_bytes != 4)
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
