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
// search of row_ptr). The workgroup then walks its rows in tiles of at most
// 256 rows and T = 256 K entries, the tile being the longest run of whole rows
// whose entries fit:
//   1. thread t holds the K consecutive entries starting at base + K t (base =
//      the tile's first entry rounded down to a multiple of 4), loaded as
//      16-byte vectors of values and of column indices, and gathers y[column]
//      (from an LDS copy of y when it is small);
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
// entries (which start where this tile ends) are already loading. Every one of
// these loads is issued unconditionally (addresses clamped, results selected),
// and the y gathers of a tile are issued before the prefetch of the next, so
// the compiler can wait for exactly the values it needs: the counter of
// outstanding vector-memory operations completes in order, and a conditional
// load anywhere in between forces a wait for everything. The per-tile LDS state
// (row_ptr, v, marks, dots) is double-buffered, so a tile costs two workgroup
// barriers: one between the dots and the scatter, one that publishes the next
// tile's state and counts its rows.
#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

constexpr int kTileRows = kBlock;  // rows a tile stages: one row_ptr per thread

typedef __attribute__((address_space(1))) float global_float;
typedef int32_t i4 __attribute__((ext_vector_type(4)));
typedef int32_t i2 __attribute__((ext_vector_type(2)));

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

// Scatter-add of one product. Both atomics name their address space explicitly: written as
// plain atomicAdd on float*, the compiler merges the two branches into a single flat atomic,
// which is slower and makes every later wait cover outstanding loads.
__device__ __forceinline__ void scatter(const CsrArgs& a, float* out_s, int32_t col, float c) {
  if (col < a.lds_window) {
    lds_add_f32(out_s + col, c);
  } else {
    __hip_atomic_fetch_add((global_float*)a.acc + col, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The loads one tile needs, held in registers while the previous tile is processed.
template <int K>
struct TileRegs {
  float val[K];
  int32_t col[K];
  int32_t rp;   // row_ptr[r + tid] (the tile's rows start at r): first entry of this thread's row
  int32_t rp1;  // row_ptr[r + tid + 1]: its end
  float v;      // v[r + tid]
};

template <int K, bool YLDS, bool HAS_V, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void csr_fused(CsrArgs a) {
  static_assert(K == 4 || K == 8, "entries are loaded as 16-byte vectors; marks as 8 or 16 bytes");
  constexpr int T = kBlock * K;
  // per-tile state, double-buffered by tile parity
  __shared__ int32_t rp_s[2][kTileRows + 1];  // row_ptr of the tile's rows
  __shared__ float v_s[2][kTileRows];         // v of the tile's rows
  __shared__ float u_s[2][kTileRows];         // u_row = v_row * (row dot), built by the dots
  __shared__ __align__(16) uint16_t mark_s[2][T];  // 1 + tile row whose first entry sits at slot q, else 0
  __shared__ int32_t wfirst_s[2][kWaves];     // tile row holding the first entry of each wavefront
  __shared__ float lred[kWaves];
  __shared__ int64_t range_s[2];
  extern __shared__ float dyn[];
  float* out_s = dyn;                 // [lds_window]
  float* y_s = dyn + a.lds_window;    // [n] when YLDS
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nnz = a.nnz;

  for (int64_t j = tid; j < a.lds_window; j += kBlock) out_s[j] = 0.0f;
  if constexpr (YLDS) {
    for (int64_t j = tid; j < a.n; j += kBlock) y_s[j] = a.y[j];
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int k = 0; k < K; ++k) mark_s[b][tid * K + k] = 0;
    if (tid < kWaves) wfirst_s[b][tid] = 0;
  }
  if (wave == 0) {
    const int64_t q = (nnz + gridDim.x - 1) / gridDim.x;
    const int64_t rb = wave_lower_bound(a.row_ptr, a.m, (int64_t)blockIdx.x * q);
    const int64_t re =
        (blockIdx.x + 1 == gridDim.x) ? a.m : wave_lower_bound(a.row_ptr, a.m, (int64_t)(blockIdx.x + 1) * q);
    if (lane == 0) {
      range_s[0] = rb;
      range_s[1] = re;
    }
  }
  __syncthreads();
  const int64_t rb = range_s[0], re = range_s[1];
  if (rb >= re) {
    if (a.lds_window > 0) {
      float* dst = a.partial + (int64_t)blockIdx.x * a.lds_window;
      for (int64_t c = tid; c < a.lds_window; c += kBlock) dst[c] = 0.0f;
    }
    return;
  }
  const float* ysrc = YLDS ? y_s : a.y;

  // Loads for the tile whose rows start at r and whose entries start at `first_entry`;
  // every load is unconditional (clamped address), entries past the arrays read as zero.
  // Only used when nnz >= 4 (the vector loads then never leave the arrays).
  const int64_t nnz_full = nnz & ~(int64_t)3;  // entries in whole aligned quads
  auto issue_rows = [&](int64_t r, TileRegs<K>& g) {
    g.rp = a.row_ptr[min(r + tid, re)];
    g.rp1 = a.row_ptr[min(r + tid + 1, re)];
    g.v = HAS_V ? a.v[min(r + tid, re - 1)] : 1.0f;
  };
  auto issue = [&](int64_t r, int64_t first_entry, TileRegs<K>& g) {
    issue_rows(r, g);
    const int64_t e0 = (first_entry & ~(int64_t)3) + (int64_t)tid * K;
    // the last partial quad (nnz % 4 entries), read by every lane and used by the one lane whose
    // quad starts at nnz_full
    float tv[3];
    int32_t tc[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int64_t p = min(nnz_full + q, nnz - 1);
      tv[q] = a.values[p];
      tc[q] = a.col_idx[p];
    }
#pragma unroll
    for (int k = 0; k < K; k += 4) {
      const int64_t e = e0 + k;
      const int64_t ec = min(e, nnz_full - 4);
      float xv[4];
      int32_t xc[4];
      if constexpr (ALIGNED) {
        const f4 vv = *reinterpret_cast<const f4*>(a.values + ec);
        const i4 cc = *reinterpret_cast<const i4*>(a.col_idx + ec);
        xv[0] = vv.x; xv[1] = vv.y; xv[2] = vv.z; xv[3] = vv.w;
        xc[0] = cc.x; xc[1] = cc.y; xc[2] = cc.z; xc[3] = cc.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xv[q] = a.values[ec + q];
          xc[q] = a.col_idx[ec + q];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool full = e < nnz_full;
        const bool tail = (e == nnz_full) && (e + q < nnz);
        g.val[k + q] = full ? xv[q] : (tail && q < 3 ? tv[q < 3 ? q : 0] : 0.0f);
        g.col[k + q] = full ? xc[q] : (tail && q < 3 ? tc[q < 3 ? q : 0] : 0);
      }
    }
  };
  // Small matrices (nnz < 4): element loads, guarded.
  auto issue_small = [&](int64_t r, int64_t first_entry, TileRegs<K>& g) {
    issue_rows(r, g);
    const int64_t e0 = (first_entry & ~(int64_t)3) + (int64_t)tid * K;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const bool in = e0 + k < nnz;
      g.val[k] = in ? a.values[e0 + k] : 0.0f;
      g.col[k] = in ? a.col_idx[e0 + k] : 0;
    }
  };
  // Publishes the state of the tile of `cnt` rows whose first entry is `first` into buffer b
  // (row_ptr, v, zeroed dots, row-start marks, the row of each wavefront's first entry) and
  // returns whether this thread's row ends inside the tile's T entry slots; the rows that do
  // form a prefix, so their count is the number of rows of the tile.
  auto stage = [&](int b, int cnt, int64_t first, const TileRegs<K>& g) -> bool {
    const int64_t base = first & ~(int64_t)3;
    u_s[b][tid] = 0.0f;
    bool fits = false;
    if (tid < cnt) {
      if (tid == 0) rp_s[b][0] = g.rp;
      rp_s[b][tid + 1] = g.rp1;
      v_s[b][tid] = g.v;
      const int64_t s = (int64_t)g.rp - base, e = (int64_t)g.rp1 - base;
      if (e > s && s < T) mark_s[b][s] = (uint16_t)(tid + 1);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int64_t pw = max((int64_t)w * 64 * K, first - base);
        if (s <= pw && pw < e) wfirst_s[b][w] = tid;
      }
      fits = e <= T;
    }
    return fits;
  };

  TileRegs<K> ga, gb;
  int buf = 0;
  int64_t ra = rb;
  int cnt = (int)min((int64_t)kTileRows, re - ra);
  int j;
  {
    const int64_t p0 = a.row_ptr[ra];
    if (nnz >= 4) issue(ra, p0, ga); else issue_small(ra, p0, ga);
    j = __syncthreads_count(stage(0, cnt, p0, ga));
  }

  auto step = [&](TileRegs<K>& g, TileRegs<K>& gn) -> bool {
    const int b = buf;
    const int32_t pa = rp_s[b][0];
    const int64_t base = (int64_t)pa & ~(int64_t)3;
    const bool long_row = (j == 0);  // row ra alone holds more entries than a tile
    const int32_t pb = long_row ? rp_s[b][1] : rp_s[b][j];
    const int64_t ra_next = ra + (long_row ? 1 : j);
    const bool more = ra_next < re;
    const int cnt_next = more ? (int)min((int64_t)kTileRows, re - ra_next) : 0;
    const int64_t e0 = base + (int64_t)tid * K;

    // (a) gathers of y for this tile's entries, before anything of the next tile is issued
    float yv[K];
    if (!long_row) {
#pragma unroll
      for (int k = 0; k < K; ++k) yv[k] = ysrc[g.col[k]];
    }
    // (b) the next tile's row_ptr, v and entries (they start where this tile ends)
    if (nnz >= 4) issue(min(ra_next, re - 1), pb, gn); else issue_small(min(ra_next, re - 1), pb, gn);

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
      // the whole workgroup sweeps the row twice: dot, then scatter
      float s = 0.0f;
      for (int64_t p = pa + tid; p < pb; p += kBlock) s = fmaf(a.values[p], ysrc[a.col_idx[p]], s);
      s = group_sum(s, 64);
      if (lane == 0) lred[wave] = s;
      __syncthreads();
      float t = lred[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) t += lred[w];
      const float u = v_s[b][0] * t;
      for (int64_t p = pa + tid; p < pb; p += kBlock) scatter(a, out_s, a.col_idx[p], u * a.values[p]);
    } else {
      // (c) the row of each entry: the latest row-start mark at or before it, within the thread,
      // then across the wavefront, then the row that holds the wavefront's first entry
      bool ok[K];
      int rk[K];
      int run_max = -1;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        ok[k] = (e0 + k >= pa) && (e0 + k < pb);
        run_max = max(run_max, mk[k]);
        mk[k] = run_max;
      }
      const int wf = wfirst_s[b][wave];
      const int before = max(wf, dpp_int<dpp::kWaveShr1>(-1, wave_max_scan(run_max)));
#pragma unroll
      for (int k = 0; k < K; ++k) rk[k] = max(before, mk[k]);  // in [0, kTileRows)

      // (d) per-row dots. Runs of one row inside the thread are summed in registers; a row
      // strictly inside the thread is complete and stored; the first run (head) and the last
      // (tail) may continue in neighbouring threads and are finished below.
      int r0 = -1, r1 = -1;
      float head = 0.0f, run = 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (ok[k]) {
          const float p = g.val[k] * yv[k];
          if (rk[k] != r1) {
            if (r1 >= 0) {
              if (r1 == r0) head = run;
              else u_s[b][r1] = v_s[b][r1] * run;
            }
            if (r0 < 0) r0 = rk[k];
            r1 = rk[k];
            run = p;
          } else {
            run += p;
          }
        }
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
      // (e) scatter
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (ok[k]) scatter(a, out_s, g.col[k], u_s[b][rk[k]] * g.val[k]);
    }
    if (!more) return false;
    const bool fits = stage(b ^ 1, cnt_next, pb, gn);
    ra = ra_next;
    buf = b ^ 1;
    cnt = cnt_next;
    j = __syncthreads_count(fits);  // the next tile's state is published
    return true;
  };

  while (step(ga, gb) && step(gb, ga)) {
  }

  if (a.lds_window > 0) {
    __syncthreads();
    float* dst = a.partial + (int64_t)blockIdx.x * a.lds_window;
    for (int64_t c = tid; c < a.lds_window; c += kBlock) dst[c] = out_s[c];
  }
}

template <int K, bool YLDS, bool HAS_V, bool ALIGNED>
hipError_t launch_k(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  const size_t lds = ((size_t)a.lds_window + (YLDS ? (size_t)a.n : 0)) * sizeof(float);
  const void* fn = reinterpret_cast<const void*>(&csr_fused<K, YLDS, HAS_V, ALIGNED>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((csr_fused<K, YLDS, HAS_V, ALIGNED>), dim3((unsigned)p.grid), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

template <int K>
hipError_t launch_kk(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  const bool yl = p.y_in_lds != 0, hv = a.v != nullptr, al = a.aligned;
  if (yl) {
    if (hv) return al ? launch_k<K, true, true, true>(a, p, s) : launch_k<K, true, true, false>(a, p, s);
    return al ? launch_k<K, true, false, true>(a, p, s) : launch_k<K, true, false, false>(a, p, s);
  }
  if (hv) return al ? launch_k<K, false, true, true>(a, p, s) : launch_k<K, false, true, false>(a, p, s);
  return al ? launch_k<K, false, false, true>(a, p, s) : launch_k<K, false, false, false>(a, p, s);
}

}  // namespace

hipError_t launch_csr(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if (p.block_threads != kBlock || p.grid <= 0 || p.grid > INT32_MAX || p.kernel != XTVXY_CSR_TILES)
    return hipErrorInvalidValue;
  switch (p.entries_per_thread) {
    case 4: return launch_kk<4>(a, p, s);
    case 8: return launch_kk<8>(a, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace xtvxy
