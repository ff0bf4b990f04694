// Fused CSR kernel for out = alpha * X^T (v .* (X y)) + beta * z.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract): one
// fused kernel with techniques specific to sparse X; each stored entry is
// loaded once and used for both the row dot product and the transposed
// scatter, and partial outputs are aggregated hierarchically.
//
// Work split: workgroup w owns the rows whose first entry lies in
// [w q, (w + 1) q), q = ceil(nnz / grid), so every workgroup streams about the
// same number of entries (one wavefront finds the two boundaries with a 64-way
// search of row_ptr). The workgroup (BLK = 256 or 512 threads) then walks its
// rows in tiles of at most BLK rows and T = BLK K entries, the tile being the
// longest run of whole rows whose entries fit:
//   1. thread t holds the K consecutive entries starting at base + K t (base =
//      the tile's first entry rounded down to a multiple of 4), loaded as
//      vectors of 4 values (16 bytes of fp32, or 8 of bf16 widened exactly to
//      fp32: reduced-precision storage of the values) and of 4 column indices,
//      and gathers y[column] (from an LDS copy of y when it is small);
//   2. the row of each entry comes from row-start marks: every nonempty row of
//      the tile writes its index at the LDS slot of its first entry, each
//      thread reads the marks of its K slots, and a running maximum over the
//      slots, then across the wavefront, names the row of every entry;
//   3. per-row dots: a thread sums its products by row; rows complete inside
//      the thread are stored directly, the rest are finished by a segmented sum
//      across the wavefront, so every row gets one write per wavefront it
//      touches (an atomic add only where a row crosses a wavefront boundary).
//      Each write already carries the factor v_row, giving u_row = v_row t_row;
//   4. every entry still in registers is scattered as u_row * value: columns
//      below the LDS window W accumulate in the workgroup's LDS copy of the
//      output (written to the workspace at the end and summed across
//      workgroups by aggregate.hip), columns at or above W go to a global fp32
//      accumulator with hardware float atomics.
// The LDS float accumulations are compare-and-swap adds (see lds_add_f32).
// A row with more entries than a tile is handled by the whole workgroup in two
// sweeps over its entries (dot, then scatter).
//
// Software pipeline: while a tile is processed, the next tile's row_ptr, v and
// entries (which start where this tile ends) are already loading, and (when y is
// read from global memory) at the end of the step, once they have arrived, the
// next tile's y gathers are issued so that they overlap the barrier and the
// start of the next step. The loads issued ahead run without any branch around
// them (addresses clamped, slots past the tile masked where they are used): the
// counter of outstanding vector-memory operations completes in order, and a
// conditional load, or two paths that leave a prefetched value in different
// registers, anywhere in between forces a wait for everything. The per-tile LDS state
// (row_ptr, v, marks, dots) is double-buffered, so a tile costs two workgroup
// barriers: one between the dots and the scatter, one that publishes the next
// tile's state and counts its rows.
#include "csr_common.h"
#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

typedef int32_t i4 __attribute__((ext_vector_type(4)));
typedef int32_t i2 __attribute__((ext_vector_type(2)));

// What the kernel computes: the whole pattern (partials of X^T (v .* (X y))), only its first
// half (t = alpha v .* (X y) + beta t0, written per row), or only its second half (partials of
// X^T u, with u given in place of v and no y).
enum CsrMode { kModeFused = 0, kModeRowdot = 1, kModeTmv = 2 };

// The loads one tile needs, held in registers while the previous tile is processed.
template <int K>
struct TileRegs {
  float val[K];
  int32_t col[K];
  int32_t rp;   // row_ptr[r + tid] (the tile's rows start at r): first entry of this thread's row
  int32_t rp1;  // row_ptr[r + tid + 1]: its end
  float v;      // v[r + tid]
  float yv[K];  // y[col] of the entries (gathered one step ahead when y is read from global memory)
};

template <class VT, int BLK, int K, int YMODE, bool HAS_V, bool ALIGNED, int COLD, int MODE>
__global__ __launch_bounds__(BLK) void csr_fused(CsrArgs a) {
  static_assert(BLK == 256 || BLK == 512, "workgroups of 256 or 512 threads");
  static_assert(K == 4 || K == 8, "entries are loaded as vectors of 4; marks as 8 or 16 bytes");
  constexpr int T = BLK * K;  // entry slots of a tile; a tile also holds at most BLK rows
  constexpr bool BINNED = COLD == kColdBinned;
  // per-tile state, double-buffered by tile parity
  __shared__ int32_t rp_s[2][BLK + 1];  // row_ptr of the tile's rows
  __shared__ float v_s[2][BLK];         // v of the tile's rows
  __shared__ float u_s[2][BLK];         // u_row = v_row * (row dot), built by the dots
  __shared__ __align__(16) uint16_t mark_s[2][T];  // 1 + tile row whose first entry sits at slot q, else 0
  __shared__ int32_t wfirst_s[2][(BLK / 64)];     // tile row holding the first entry of each wavefront
  __shared__ int32_t rows_s[2];                    // rows of the tile
  __shared__ float sink_s[BLK];            // a private LDS word per thread for masked-off adds
  __shared__ float lred[(BLK / 64)];
  __shared__ int32_t range_s[2];
  extern __shared__ __align__(16) float dyn[];
  float* out_s = dyn;                 // [lds_window]
  float* y_s = dyn + a.lds_window;    // [y_window]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Entry positions are unsigned 32-bit (nnz < 2^31, so a position plus a tile never wraps);
  // rows are signed 32-bit (m <= 2^31 - 1025, so a row plus 256 never overflows).
  const uint32_t nnz = (uint32_t)a.nnz;
  const uint32_t nnz_full = nnz & ~3u;  // entries in whole aligned quads
  const int32_t window = (int32_t)a.lds_window;

  for (int32_t j = tid; j < window; j += BLK) out_s[j] = 0.0f;
  const int32_t y_window = YMODE == kYGlobal ? 0 : (int32_t)a.y_window;
  for (int32_t j = tid; j < y_window; j += BLK) y_s[j] = a.y[j];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int k = 0; k < K; ++k) mark_s[b][tid * K + k] = 0;
    if (tid < (BLK / 64)) wfirst_s[b][tid] = 0;
  }
  sink_s[tid] = 0.0f;
  // Binning of the columns >= window. Per bin, in LDS: the items of the current batch (a
  // tile, or a slice of a long row), the workgroup's current chunk and its fill, and where the
  // batch's items go: `room` items from pos1 on, the rest from pos2 on (new chunks, contiguous).
  constexpr uint32_t S = kBinChunkItems;
  const uint64_t pool_items = (uint64_t)a.pool_chunks * S;
  uint64_t* pos1_s = nullptr;
  uint64_t* pos2_s = nullptr;
  uint32_t* cnt_s = nullptr;
  int32_t* cur_s = nullptr;
  int32_t* fill_s = nullptr;
  uint32_t* room_s = nullptr;
  if constexpr (BINNED) {
    const int64_t words = (a.lds_window + y_window + 1) & ~(int64_t)1;  // 8-byte aligned
    pos1_s = reinterpret_cast<uint64_t*>(dyn + words);
    pos2_s = pos1_s + a.bins;
    cnt_s = reinterpret_cast<uint32_t*>(pos2_s + a.bins);
    cur_s = reinterpret_cast<int32_t*>(cnt_s + a.bins);
    fill_s = cur_s + a.bins;
    room_s = reinterpret_cast<uint32_t*>(fill_s + a.bins);
    for (int t = tid; t < a.bins; t += BLK) {
      cnt_s[t] = 0;
      cur_s[t] = -1;
      fill_s[t] = (int32_t)S;
    }
  }
  // (cold column) -> its rank among the batch's items of its bin
  auto bin_rank = [&](int32_t col) -> uint32_t {
    const int bin = (col - window) >> a.bin_shift;
    return __hip_atomic_fetch_add((lds_uint*)(cnt_s + bin), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  // After a barrier that follows the batch's ranks: one thread per bin finds room for the
  // bin's items, handing out new pool chunks (one global atomic per bin and batch that spills),
  // and resets the count. A barrier must follow before bin_write.
  auto bin_alloc = [&]() {
    for (int t = tid; t < a.bins; t += BLK) {
      const uint32_t cnt = cnt_s[t];
      if (cnt == 0) continue;
      cnt_s[t] = 0;
      const int32_t cur = cur_s[t], fill = fill_s[t];
      const uint32_t room = cur >= 0 ? S - (uint32_t)fill : 0u;
      room_s[t] = room;
      pos1_s[t] = (uint64_t)(cur >= 0 ? cur : 0) * S + (uint32_t)fill;
      if (cnt <= room) {
        fill_s[t] = fill + (int32_t)cnt;
        continue;
      }
      const uint32_t need = cnt - room, k = (need + S - 1) / S;
      const uint32_t first =
          __hip_atomic_fetch_add((global_uint*)a.pool_next, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((int64_t)first + k > a.pool_chunks) {  // cannot happen with the pool sized for the plan
        pos2_s[t] = pool_items;                  // the items are dropped rather than written out of bounds
        cur_s[t] = -1;
        fill_s[t] = (int32_t)S;
        continue;
      }
      for (uint32_t c = 0; c < k; ++c) {
        a.chunk_bin[first + c] = t;
        a.chunk_fill[first + c] = (int32_t)S;  // the last one is corrected when it stops filling
      }
      pos2_s[t] = (uint64_t)first * S;
      cur_s[t] = (int32_t)(first + k - 1);
      fill_s[t] = (int32_t)(need - (k - 1) * S);
    }
  };
  auto bin_write = [&](int32_t col, float c, uint32_t rank) {
    const int bin = (col - window) >> a.bin_shift;
    const uint32_t room = room_s[bin];
    const uint64_t pos = rank < room ? pos1_s[bin] + rank : pos2_s[bin] + (rank - room);
    if (pos < pool_items) a.pool[pos] = make_int2(col, __float_as_int(c));
  };
  // Scatter of K products c[k] to columns col[k] where on[k]. Columns in the window go to the
  // LDS copy of the output (a masked-off lane adds 0 to its own sink word, so the add needs no
  // branch); the others go to the global accumulator or to the bins. With bins, every thread of
  // the workgroup must call this together (it holds two barriers).
  auto scatter_k = [&](const float (&c)[K], const int32_t (&col)[K], const bool (&on)[K]) {
    if constexpr (COLD == kColdNone) {
#pragma unroll
      for (int k = 0; k < K; ++k) lds_add_f32(on[k] ? out_s + col[k] : sink_s + tid, on[k] ? c[k] : 0.0f);
    } else if constexpr (COLD == kColdAtomic) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const bool hot = on[k] && col[k] < window;
        lds_add_f32(hot ? out_s + col[k] : sink_s + tid, hot ? c[k] : 0.0f);
        if (on[k] && !hot)
          __hip_atomic_fetch_add((global_float*)a.acc + col[k], c[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      uint32_t rank[K];
      bool cold[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const bool hot = on[k] && col[k] < window;
        cold[k] = on[k] && !hot;
        lds_add_f32(hot ? out_s + col[k] : sink_s + tid, hot ? c[k] : 0.0f);
        if (cold[k]) rank[k] = bin_rank(col[k]);
      }
      __syncthreads();  // the batch's bin counts are complete
      bin_alloc();
      __syncthreads();  // room for every bin is known
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (cold[k]) bin_write(col[k], c[k], rank[k]);
    }
  };

  if (wave == 0) {
    const int64_t q = (a.nnz + gridDim.x - 1) / gridDim.x;
    int64_t rb, re;
    wave_lower_bound_pair(a.row_ptr, a.m, (int64_t)blockIdx.x * q, (int64_t)(blockIdx.x + 1) * q, rb, re);
    if (blockIdx.x + 1 == gridDim.x) re = a.m;
    if (lane == 0) {
      range_s[0] = (int32_t)rb;
      range_s[1] = (int32_t)re;
    }
  }
  __syncthreads();
  const int32_t rb = range_s[0], re = range_s[1];
  if (rb >= re) {
    float* dst = a.partial + (int64_t)blockIdx.x * window;
    for (int32_t c = tid; c < window; c += BLK) dst[c] = 0.0f;
    return;
  }
  // Gathers from global memory are issued a step ahead (their latency then overlaps a barrier);
  // gathers from an LDS copy of all of y measured faster at the start of the step.
  constexpr bool kGathers = MODE != kModeTmv;  // the second half alone reads no y
  constexpr bool kGatherAhead = kGathers && YMODE != kYLds;
  auto gather_y = [&](int32_t col) -> float {
    if constexpr (YMODE == kYGlobal) return a.y[col];
    if constexpr (YMODE == kYLds) return y_s[col];
    // split: both reads are issued by every lane, without a branch; lanes whose column is in
    // the LDS copy read y[0] from global memory (one cache line for all of them)
    const float fast = y_s[min(col, y_window - 1)];
    const float slow = a.y[col < y_window ? 0 : col];
    return col < y_window ? fast : slow;
  };

  auto issue_rows = [&](int32_t r, TileRegs<K>& g) {
    g.rp = a.row_ptr[min(r + tid, re)];
    g.rp1 = a.row_ptr[min(r + tid + 1, re)];
    g.v = HAS_V ? a.v[min(r + tid, re - 1)] : 1.0f;
  };
  // The K entries from base + K tid (base a multiple of 4), loaded and used at once (the slices
  // of a long row). Tiles whose T slots lie inside the whole quads of the arrays load without
  // any guard; the others load element by element with clamped addresses, entries past nnz
  // reading as zero. The branch is the same for the whole workgroup.
  auto load_entries = [&](uint32_t base, float (&val)[K], int32_t (&col)[K]) {
    const uint32_t e0 = base + (uint32_t)tid * K;
    if (base + T <= nnz_full) {
#pragma unroll
      for (int k = 0; k < K; k += 4) {
        if constexpr (ALIGNED) {
          csr_value_quad<VT>(a.values, e0 + k, val + k);
          const i4 cc = *reinterpret_cast<const i4*>(a.col_idx + e0 + k);
          col[k] = cc.x; col[k + 1] = cc.y; col[k + 2] = cc.z; col[k + 3] = cc.w;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            val[k + q] = csr_value<VT>(a.values, e0 + k + q);
            col[k + q] = a.col_idx[e0 + k + q];
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const bool in = e0 + k < nnz;
        const uint32_t p = in ? e0 + k : nnz - 1;
        const float x = csr_value<VT>(a.values, p);
        const int32_t c = a.col_idx[p];
        val[k] = in ? x : 0.0f;
        col[k] = in ? c : 0;
      }
    }
  };
  // The same entries loaded a step ahead, with no branch at all (see the top of the file): with
  // vector loads a quad at or past the last whole quad of the arrays is read at the last whole
  // quad instead (the launch guarantees nnz >= 4), element loads are clamped to nnz - 1. Slots
  // past the tile then hold entries of other positions; every use masks them, and their column
  // indices are valid. The up to three entries after the whole quads are patched in by
  // fix_tail before the tile's first use.
  const uint32_t last_quad = ALIGNED ? nnz_full - 4u : 0u;
  auto load_entries_ahead = [&](uint32_t base, float (&val)[K], int32_t (&col)[K]) {
    const uint32_t e0 = base + (uint32_t)tid * K;
#pragma unroll
    for (int k = 0; k < K; k += 4) {
      if constexpr (ALIGNED) {
        const uint32_t q = min(e0 + k, last_quad);
        csr_value_quad<VT>(a.values, q, val + k);
        const i4 cc = *reinterpret_cast<const i4*>(a.col_idx + q);
        col[k] = cc.x; col[k + 1] = cc.y; col[k + 2] = cc.z; col[k + 3] = cc.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t p = min(e0 + k + q, nnz - 1u);
          val[k + q] = csr_value<VT>(a.values, p);
          col[k + q] = a.col_idx[p];
        }
      }
    }
  };
  // Entries nnz_full .. nnz - 1 of a tile loaded by load_entries_ahead with vector loads. The
  // branch is the same for the whole workgroup and taken by the last tile or two only.
  auto fix_tail = [&](uint32_t first_entry, TileRegs<K>& g) {
    if constexpr (ALIGNED && kGatherAhead) {
      const uint32_t base = first_entry & ~3u;
      if (nnz != nnz_full && base + T > nnz_full) {
        const uint32_t e0 = base + (uint32_t)tid * K;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const uint32_t p = e0 + k;
          if (p >= nnz_full && p < nnz) {
            g.val[k] = csr_value<VT>(a.values, p);
            g.col[k] = a.col_idx[p];
          }
        }
      }
    }
  };
  // Kernels that gather y a step ahead load the entries branch-free (measured faster on the Zipf
  // workload, where the two paths of load_entries left the prefetched entries in different
  // registers and the copies waited for them at once); the others keep the guarded loads
  // (measured faster on the logistic-regression workload).
  auto issue = [&](int32_t r, uint32_t first_entry, TileRegs<K>& g) {
    issue_rows(r, g);
    if constexpr (kGatherAhead)
      load_entries_ahead(first_entry & ~3u, g.val, g.col);
    else
      load_entries(first_entry & ~3u, g.val, g.col);
  };
  // Publishes the state of the tile of at most `cnt` rows whose first entry is `first` into
  // buffer b (row_ptr, v, zeroed dots, row-start marks, the row of each wavefront's first entry,
  // the number of rows). The tile's rows are those that end inside its T entry slots: a prefix
  // of the cnt candidates, so the one thread whose row is the first that does not fit (or the
  // last candidate, when all fit) writes the count. A barrier must follow before it is read.
  auto stage = [&](int b, int cnt, uint32_t first, const TileRegs<K>& g) {
    const uint32_t base = first & ~3u;
    // the row values u: built by the dots, or (second half alone) the given vector
    u_s[b][tid] = (MODE == kModeTmv && tid < cnt) ? g.v : 0.0f;
    if (tid < cnt) {
      if (tid == 0) rp_s[b][0] = g.rp;
      rp_s[b][tid + 1] = g.rp1;
      v_s[b][tid] = g.v;
      const uint32_t s = (uint32_t)g.rp - base, e = (uint32_t)g.rp1 - base;
      if (e > s && s < T) mark_s[b][s] = (uint16_t)(tid + 1);
#pragma unroll
      for (int w = 0; w < (BLK / 64); ++w) {
        const uint32_t pw = w == 0 ? first - base : (uint32_t)(w * 64 * K);
        if (s <= pw && pw < e) wfirst_s[b][w] = tid;
      }
      const bool fits = e <= T;
      const bool prev_fits = tid == 0 || s <= T;  // the row before ends where this one starts
      if (prev_fits && !fits) rows_s[b] = tid;
      if (fits && tid == cnt - 1) rows_s[b] = cnt;
    }
  };

  TileRegs<K> ga, gb;
  int buf = 0;
  int32_t ra = rb;
  int cnt = min(BLK, re - ra);
  int j;
  {
    const uint32_t p0 = (uint32_t)a.row_ptr[ra];
    issue(ra, p0, ga);
    fix_tail(p0, ga);
    if constexpr (kGatherAhead) {
#pragma unroll
      for (int k = 0; k < K; ++k) ga.yv[k] = gather_y(ga.col[k]);
    }
    stage(0, cnt, p0, ga);
    __syncthreads();
    j = rows_s[0];
  }

  auto step = [&](TileRegs<K>& g, TileRegs<K>& gn) -> bool {
    const int b = buf;
    const uint32_t pa = (uint32_t)rp_s[b][0];
    const uint32_t base = pa & ~3u;
    const bool long_row = (j == 0);  // row ra alone holds more entries than a tile
    const uint32_t pb = (uint32_t)(long_row ? rp_s[b][1] : rp_s[b][j]);
    const int32_t ra_next = ra + (long_row ? 1 : j);
    const bool more = ra_next < re;
    const int cnt_next = more ? min(BLK, re - ra_next) : 0;
    const uint32_t e0 = base + (uint32_t)tid * K;

    // (a) this tile's y values: from LDS now, or from global memory gathered at the end of the
    // previous step
    if constexpr (kGathers && !kGatherAhead) {
#pragma unroll
      for (int k = 0; k < K; ++k) g.yv[k] = gather_y(g.col[k]);
    }
    const float (&yv)[K] = g.yv;
    // (b) the next tile's row_ptr, v and entries (they start where this tile ends)
    issue(min(ra_next, re - 1), pb, gn);

    // this thread's K row-start marks, cleared for the tile after next
    int mk[K];
    {
      uint16_t* ms = &mark_s[b][tid * K];
      if constexpr (K == 8) {
        const i4 w = *reinterpret_cast<const i4*>(ms);
        *reinterpret_cast<i4*>(ms) = i4{0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          mk[2 * q] = (int)(w[q] & 0xffff) - 1;
          mk[2 * q + 1] = (int)((uint32_t)w[q] >> 16) - 1;
        }
      } else {
        const i2 w = *reinterpret_cast<const i2*>(ms);
        *reinterpret_cast<i2*>(ms) = i2{0, 0};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          mk[2 * q] = (int)(w[q] & 0xffff) - 1;
          mk[2 * q + 1] = (int)((uint32_t)w[q] >> 16) - 1;
        }
      }
    }

    if (long_row) {
      // The whole workgroup takes the row in slices of T entries, twice: the dot, then the
      // scatter. The first slice is the one already in registers.
      const uint32_t len = pb - pa;
      float u = v_s[b][0];  // the given u of the row (second half alone), else v of the row
      if constexpr (MODE != kModeTmv) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) s += (e0 + k - pa < len) ? g.val[k] * yv[k] : 0.0f;
        for (uint32_t sb = base + T; sb < pb; sb += T) {
          float hv[K];
          int32_t hc[K];
          load_entries(sb, hv, hc);
          const uint32_t h0 = sb + (uint32_t)tid * K;
#pragma unroll
          for (int k = 0; k < K; ++k) s += (h0 + k < pb) ? hv[k] * gather_y(hc[k]) : 0.0f;
        }
        s = group_sum(s, 64);
        if (lane == 0) lred[wave] = s;
        __syncthreads();
        float t = lred[0];
#pragma unroll
        for (int w = 1; w < (BLK / 64); ++w) t += lred[w];
        u = u * t;
      }
      if constexpr (MODE == kModeRowdot) {
        if (tid == 0) a.t_out[ra] = a.alpha * u + (a.beta != 0.0f ? a.beta * a.t0[ra] : 0.0f);
      } else {
        {
          float c[K];
          bool on[K];
#pragma unroll
          for (int k = 0; k < K; ++k) {
            on[k] = e0 + k - pa < len;
            c[k] = u * g.val[k];
          }
          scatter_k(c, g.col, on);
        }
        for (uint32_t sb = base + T; sb < pb; sb += T) {
          float hv[K];
          int32_t hc[K];
          load_entries(sb, hv, hc);
          const uint32_t h0 = sb + (uint32_t)tid * K;
          float c[K];
          bool on[K];
#pragma unroll
          for (int k = 0; k < K; ++k) {
            on[k] = h0 + k < pb;
            c[k] = u * hv[k];
          }
          scatter_k(c, hc, on);
        }
      }
    } else {
      // (c) the row of each entry: the latest row-start mark at or before it, within the thread,
      // then across the wavefront, then the row that holds the wavefront's first entry
      bool ok[K];
      int rk[K];
      int run_max = -1;
      const uint32_t len = pb - pa;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        ok[k] = e0 + k - pa < len;  // unsigned: positions before pa wrap to large values
        run_max = max(run_max, mk[k]);
        mk[k] = run_max;
      }
      const int wf = wfirst_s[b][wave];
      const int before = max(wf, dpp_int<dpp::kWaveShr1>(-1, wave_max_scan(run_max)));
#pragma unroll
      for (int k = 0; k < K; ++k) rk[k] = max(before, mk[k]);  // in [0, BLK)
      // (c') with bins: the rank of each product of a column outside the window among the
      // tile's items of its bin. It depends on the column alone, so it is taken before the dots
      // and the barrier that completes the dots also completes the bins' counts.
      uint32_t crank[K];
      bool cold[K];
      if constexpr (BINNED && MODE != kModeRowdot) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          cold[k] = ok[k] && g.col[k] >= window;
          crank[k] = cold[k] ? bin_rank(g.col[k]) : 0u;
        }
      }

      if constexpr (MODE != kModeTmv) {
      // (d) per-row dots. Runs of one row inside the thread are summed in registers; a row
      // strictly inside the thread is complete and stored; the first run (head) and the last
      // (tail) may continue in neighbouring threads and are finished below.
      int r0 = -1, r1 = -1;
      float head = 0.0f, run = 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float p = ok[k] ? g.val[k] * yv[k] : 0.0f;
        const bool fresh = ok[k] && rk[k] != r1;  // a new run starts at k
        if (fresh && r1 >= 0 && r1 != r0) u_s[b][r1] = v_s[b][r1] * run;  // a row inside the thread
        head = (fresh && r1 >= 0 && r1 == r0) ? run : head;                // the first run ended
        r0 = (ok[k] && r0 < 0) ? rk[k] : r0;
        run = fresh ? p : run + p;
        r1 = ok[k] ? rk[k] : r1;
      }
      // Tails summed across the wavefront per row (keys are rows, nondecreasing with the lane;
      // lanes without entries come last with a key no row has). A lane whose tail row does not
      // continue into the next lane writes that row's sum; a lane with more than one row also
      // finishes its head row with the tail sum of the lane before when that lane ended in it.
      const bool has = r1 >= 0;
      const int key = has ? r1 : INT32_MAX;
      const float tails = wave_segmented_sum(has ? run : 0.0f, key);
      const float prev_tails = dpp_float<dpp::kWaveShr1>(0.0f, tails);
      const int prev_key = dpp_int<dpp::kWaveShr1>(-1, key);
      const int next_r0 = dpp_int<dpp::kWaveShl1>(-1, r0);
      // Only a row that also holds entries of another wavefront (its first row, or the row that
      // lane 63 ends in) can receive two writes: those are added atomically, the rest stored.
      if (has && r0 != r1) {
        const float c = v_s[b][r0] * (head + (prev_key == r0 ? prev_tails : 0.0f));
        if (r0 == wf) lds_add_f32(&u_s[b][r0], c); else u_s[b][r0] = c;
      }
      if (has && next_r0 != r1) {
        const float c = v_s[b][r1] * tails;
        if (r1 == wf || lane == 63) lds_add_f32(&u_s[b][r1], c); else u_s[b][r1] = c;
      }
      __syncthreads();  // u_s[b] complete
      }  // (with the second half alone, u_s[b] holds the given u since the tile was staged)
      if constexpr (MODE == kModeRowdot) {
        // the first half alone: t = alpha u + beta t0 for the tile's rows
        for (int r = tid; r < j; r += BLK)
          a.t_out[ra + r] = a.alpha * u_s[b][r] + (a.beta != 0.0f ? a.beta * a.t0[ra + r] : 0.0f);
      } else {
        // (e) scatter
        float c[K];
#pragma unroll
        for (int k = 0; k < K; ++k) c[k] = u_s[b][rk[k]] * g.val[k];
        if constexpr (BINNED) {
          // room for the bins' items (the threads that hand it out are busy while the others
          // add the window's products), then the items
          if constexpr (MODE == kModeTmv) __syncthreads();  // the bins' counts are complete
          bin_alloc();
#pragma unroll
          for (int k = 0; k < K; ++k) {
            const bool hot = ok[k] && !cold[k];
            lds_add_f32(hot ? out_s + g.col[k] : sink_s + tid, hot ? c[k] : 0.0f);
          }
          __syncthreads();  // room for every bin is known
#pragma unroll
          for (int k = 0; k < K; ++k)
            if (cold[k]) bin_write(g.col[k], c[k], crank[k]);
        } else {
          scatter_k(c, g.col, ok);
        }
      }
    }
    if (!more) return false;
    // the next tile's y gathers, a step ahead: its entries were issued at the start of this
    // step and have arrived by now, and the gathers overlap the barrier below and the start of
    // the next step
    if constexpr (kGatherAhead) {
      fix_tail(pb, gn);
#pragma unroll
      for (int k = 0; k < K; ++k) gn.yv[k] = gather_y(gn.col[k]);
    }
    stage(b ^ 1, cnt_next, pb, gn);
    ra = ra_next;
    buf = b ^ 1;
    cnt = cnt_next;
    __syncthreads();  // the next tile's state is published
    j = rows_s[b ^ 1];
    return true;
  };

  while (step(ga, gb) && step(gb, ga)) {
  }
  if constexpr (BINNED) {
    // the fill of each bin's last chunk (every other handed-out chunk is full)
    for (int t = tid; t < a.bins; t += BLK)
      if (cur_s[t] >= 0) a.chunk_fill[cur_s[t]] = fill_s[t];
  }

  if (window > 0) {
    __syncthreads();
    float* dst = a.partial + (int64_t)blockIdx.x * window;
    for (int32_t c = tid; c < window; c += BLK) dst[c] = out_s[c];
  }
}

template <class VT, int BLK, int K, int YMODE, bool HAS_V, bool ALIGNED, int COLD, int MODE>
hipError_t launch_k(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  size_t lds = ((size_t)a.lds_window + (YMODE == kYGlobal ? 0 : (size_t)a.y_window)) * sizeof(float);
  if (COLD == kColdBinned) lds = ((lds + 7) & ~(size_t)7) + (size_t)a.bins * kCsrBinStateBytes;
  const void* fn = reinterpret_cast<const void*>(&csr_fused<VT, BLK, K, YMODE, HAS_V, ALIGNED, COLD, MODE>);
  hipError_t e = allow_dynamic_lds(fn);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((csr_fused<VT, BLK, K, YMODE, HAS_V, ALIGNED, COLD, MODE>), dim3((unsigned)p.grid), dim3(BLK), lds,
                     s, a);
  return hipGetLastError();
}

template <class VT, int BLK, int K, int COLD, int YMODE, int MODE>
hipError_t launch_kv(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  const bool al = a.aligned && a.nnz >= 4;  // vector loads need one whole quad of entries
  if constexpr (MODE == kModeTmv) {  // u is always given
    return al ? launch_k<VT, BLK, K, YMODE, true, true, COLD, MODE>(a, p, s)
              : launch_k<VT, BLK, K, YMODE, true, false, COLD, MODE>(a, p, s);
  } else {
    if (a.v != nullptr)
      return al ? launch_k<VT, BLK, K, YMODE, true, true, COLD, MODE>(a, p, s)
                : launch_k<VT, BLK, K, YMODE, true, false, COLD, MODE>(a, p, s);
    return al ? launch_k<VT, BLK, K, YMODE, false, true, COLD, MODE>(a, p, s)
              : launch_k<VT, BLK, K, YMODE, false, false, COLD, MODE>(a, p, s);
  }
}

template <class VT, int BLK, int K, int COLD, int MODE>
hipError_t launch_kk(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if constexpr (MODE == kModeTmv) {
    return launch_kv<VT, BLK, K, COLD, kYGlobal, MODE>(a, p, s);  // no y
  } else {
    if (a.y_window >= a.n) return launch_kv<VT, BLK, K, COLD, kYLds, MODE>(a, p, s);
    if (a.y_window > 0) return launch_kv<VT, BLK, K, COLD, kYSplit, MODE>(a, p, s);
    return launch_kv<VT, BLK, K, COLD, kYGlobal, MODE>(a, p, s);
  }
}

template <int BLK, int K, int MODE, class VT = float>
hipError_t launch_cold(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if constexpr (MODE == kModeRowdot) {
    return launch_kk<VT, BLK, K, kColdNone, MODE>(a, p, s);  // no scatter
  } else {
    if (a.bins > 0) return launch_kk<VT, BLK, K, kColdBinned, MODE>(a, p, s);
    if (a.lds_window < a.n) return launch_kk<VT, BLK, K, kColdAtomic, MODE>(a, p, s);
    return launch_kk<VT, BLK, K, kColdNone, MODE>(a, p, s);
  }
}

// The launch for a mode (the whole pattern or one half) and stored value type, for checked
// arguments and binning buffers.
template <class VT>
hipError_t launch_modes(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s, int mode) {
  const bool binned = a.bins > 0;
  if (mode == kCsrRowdot) {
    // the first half alone: no output window and no scatter; t_out (and t0 when beta != 0)
    if (a.lds_window != 0 || binned || a.t_out == nullptr || (a.beta != 0.0f && a.t0 == nullptr))
      return hipErrorInvalidValue;
    if (p.block_threads == 256 && p.entries_per_thread == 8) return launch_cold<256, 8, kModeRowdot, VT>(a, p, s);
    if (p.block_threads == 512 && p.entries_per_thread == 8) return launch_cold<512, 8, kModeRowdot, VT>(a, p, s);
    return hipErrorInvalidValue;
  }
  if (!binned && a.lds_window < a.n && a.acc == nullptr) return hipErrorInvalidValue;
  if (mode == kCsrTmv) {
    if (a.v == nullptr) return hipErrorInvalidValue;  // u
    if (p.block_threads == 256 && p.entries_per_thread == 8) return launch_cold<256, 8, kModeTmv, VT>(a, p, s);
    if (p.block_threads == 512 && p.entries_per_thread == 8) return launch_cold<512, 8, kModeTmv, VT>(a, p, s);
    return hipErrorInvalidValue;
  }
  if (mode != kCsrFused) return hipErrorInvalidValue;
  // (threads, entries per thread): 256 x 4, 256 x 8 and 512 x 8
  if (p.block_threads == 256 && p.entries_per_thread == 4) return launch_cold<256, 4, kModeFused, VT>(a, p, s);
  if (p.block_threads == 256 && p.entries_per_thread == 8) return launch_cold<256, 8, kModeFused, VT>(a, p, s);
  if (p.block_threads == 512 && p.entries_per_thread == 8) return launch_cold<512, 8, kModeFused, VT>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_csr(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s, int mode) {
  if (p.grid <= 0 || p.grid > INT32_MAX || p.kernel != XTVXY_CSR_TILES) return hipErrorInvalidValue;
  if (a.nnz <= 0 || a.nnz > INT32_MAX || a.m <= 0 || a.m > INT32_MAX - 1024 || a.lds_window < 0 ||
      a.lds_window > a.n || a.y_window < 0 || a.y_window > a.n)
    return hipErrorInvalidValue;
  const bool binned = a.bins > 0;
  if (binned && (a.pool == nullptr || a.pool_next == nullptr || a.chunk_bin == nullptr || a.chunk_fill == nullptr ||
                 a.bins > kMaxBins || a.acc != nullptr))
    return hipErrorInvalidValue;
  if (a.value_bytes == 2) return launch_modes<bf16_t>(a, p, s, mode);  // bf16 values
  if (a.value_bytes != 4) return hipErrorInvalidValue;
  return launch_modes<float>(a, p, s, mode);
}

}  // namespace xtvxy
