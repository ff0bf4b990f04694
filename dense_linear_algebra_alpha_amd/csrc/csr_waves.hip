// Fused CSR kernel with independent wavefronts, for out = alpha * X^T (v .* (X y)) + beta * z.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract): one
// fused kernel for sparse X; each stored entry is loaded once and used for both
// the row dot product and the transposed scatter, and partial outputs are
// aggregated hierarchically.
//
// The tiled kernel (csr.hip) has all wavefronts of a workgroup take each tile
// together, which costs two or three workgroup barriers per tile; with gathers
// and scatters whose latency varies from lane to lane, every barrier waits for
// the slowest wavefront. Here each wavefront walks rows of its own and the
// workgroup meets only twice, at the start (LDS window zeroed) and at the end
// (window written out):
//   - wavefront g of G = grid * BLK / 64 owns the rows whose first entry lies in
//     [g q, (g + 1) q), q = ceil(nnz / G), found by a 64-way search of row_ptr;
//   - it takes them in tiles of whole rows, at most 64 rows and 64 K entry slots:
//     lane l holds the K consecutive entries from base + K l (base = the tile's
//     first entry rounded down to 4), loaded as vectors of 4 (values fp32, or
//     bf16 widened exactly as they are loaded);
//   - the row of each entry comes from row-start marks in the wavefront's own LDS
//     bytes (a running maximum within the lane, then across the wavefront); per-row
//     dots are summed in registers and finished by a segmented sum across the
//     wavefront; every row of a tile lies inside the tile, so each row's value
//     u_row = v_row * dot is written exactly once, to the wavefront's LDS;
//   - scatter of u_row * value: columns below the window W go to the workgroup's
//     LDS copy of the output (shared by its wavefronts, compare-and-swap adds),
//     the others to the wavefront's own bins (the chunk pool and bin passes of
//     csr_bins.hip), or to global atomics;
//   - a row with more entries than a tile is taken by its wavefront alone in
//     slices of 64 K entries, twice (dot, then scatter).
// The next tile's row_ptr, v and entries load while the current tile is
// processed, and its y gathers are issued at the end of the step, as in the
// tiled kernel (no branch around loads issued ahead: the vector-memory counter
// completes in order).
#include "csr_common.h"
#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

typedef int32_t i4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// The loads of one tile, held in registers while the previous tile is processed.
template <int K>
struct WaveTile {
  float val[K];
  int32_t col[K];
  float yv[K];
  int32_t rp;   // row_ptr[r + lane]: first entry of this lane's row of the tile
  int32_t rp1;  // row_ptr[r + lane + 1]: its end
  float v;      // v[r + lane]
};

// What the kernel computes: the whole pattern (partials of X^T (v .* (X y))), its first half
// alone (t = alpha v .* (X y) + beta t0 per row, no scatter) or its second half alone (partials
// of X^T u, u given in place of v, no y and no dots).
enum WaveMode { kWaveFused = 0, kWaveRowdot = 1, kWaveTmv = 2 };

template <class VT, int BLK, int K, int YMODE, bool HAS_V, bool ALIGNED, int COLD, int MODE>
__global__ __launch_bounds__(BLK) void csr_waves(CsrArgs a) {
  static_assert(BLK == 256 || BLK == 512 || BLK == 1024, "workgroups of 256, 512 or 1024 threads");
  static_assert(K == 8, "eight entries per lane: two vectors of 4, one 8-byte word of marks");
  constexpr int NW = BLK / 64;  // wavefronts of the workgroup
  constexpr int TW = 64 * K;    // entry slots of a wavefront's tile
  constexpr bool BINNED = COLD == kColdBinned;
  constexpr bool kGathers = MODE != kWaveTmv;     // the second half alone reads no y
  constexpr bool kScatter = MODE != kWaveRowdot;  // the first half alone writes rows, not columns
  static_assert(kScatter || COLD == kColdNone, "the first half alone has no window and no bins");
  constexpr uint32_t S = kBinChunkItems;
  __shared__ __align__(16) uint8_t mark_s[NW][TW];  // 1 + tile row whose first entry sits at slot q, else 0
  __shared__ float u_s[NW][64];                     // the dots of the tile's rows, then u_row = v_row * dot
  __shared__ float sink_s[BLK];                     // a private LDS word per thread for masked-off adds
  extern __shared__ __align__(16) float dyn[];
  float* out_s = dyn;                 // [lds_window], shared by the wavefronts
  float* y_s = dyn + a.lds_window;    // [y_window]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t nnz = (uint32_t)a.nnz;
  const uint32_t nnz_full = nnz & ~3u;
  const int32_t window = (int32_t)a.lds_window;
  const int32_t y_window = YMODE == kYGlobal ? 0 : (int32_t)a.y_window;

  for (int32_t j = tid; j < window; j += BLK) out_s[j] = 0.0f;
  for (int32_t j = tid; j < y_window; j += BLK) y_s[j] = a.y[j];
  {
    u2* mw = reinterpret_cast<u2*>(&mark_s[wave][lane * K]);
    *mw = u2{0u, 0u};
  }
  sink_s[tid] = 0.0f;
  // This wavefront's bins (columns >= window): per bin the ranks handed out in the current
  // batch, the current chunk and its fill, and for the batch's writers the chunk and fill the
  // batch started from and the first of the new chunks it took.
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
    const float fast = y_s[min(col, y_window - 1)];
    const float slow = a.y[col < y_window ? 0 : col];
    return col < y_window ? fast : slow;
  };
  // K entries from base + K lane with no branch around the loads: quads at or past the last
  // whole quad read the last whole quad (the launch guarantees nnz >= 4 for vector loads), element
  // loads are clamped to nnz - 1. Slots outside the tile or slice hold entries of other positions;
  // every use masks them. The up to three entries after the whole quads are patched in by
  // patch_tail before first use (a branch the whole wavefront takes, for the last slices only).
  const uint32_t last_quad = ALIGNED ? nnz_full - 4u : 0u;
  auto load_clamped = [&](uint32_t base, float (&val)[K], int32_t (&col)[K]) {
    const uint32_t e0 = base + (uint32_t)lane * K;
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
  auto patch_tail = [&](uint32_t base, float (&val)[K], int32_t (&col)[K]) {
    if constexpr (ALIGNED) {
      if (nnz != nnz_full && base + TW > nnz_full) {
        const uint32_t e0 = base + (uint32_t)lane * K;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const uint32_t p = e0 + k;
          if (p >= nnz_full && p < nnz) {
            val[k] = csr_value<VT>(a.values, p);
            col[k] = a.col_idx[p];
          }
        }
      }
    }
  };
  auto load_slice = [&](uint32_t base, float (&val)[K], int32_t (&col)[K]) {
    load_clamped(base, val, col);
    patch_tail(base, val, col);
  };

  // Scatter of K products c[k] to columns col[k] where on[k] (wavefront-uniform control flow).
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
      // ranks within the wavefront's batch of each bin
      uint32_t rank[K];
      bool cold[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        cold[k] = on[k] && col[k] >= window;
        const int bin = cold[k] ? (col[k] - window) >> a.bin_shift : 0;
        rank[k] = cold[k] ? __hip_atomic_fetch_add((lds_uint*)(cnt_w + bin), 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WAVEFRONT)
                          : 0u;
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
      for (int k = 0; k < K; ++k) {
        const bool hot = on[k] && !cold[k];
        lds_add_f32(hot ? out_s + col[k] : sink_s + tid, hot ? c[k] : 0.0f);
      }
      wave_lds_sync();
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (cold[k]) {
          const int bin = (col[k] - window) >> a.bin_shift;
          const int32_t oc = oc_w[bin];
          const uint32_t of = of_w[bin];
          const uint32_t room = oc >= 0 ? S - of : 0u;
          const uint64_t pos = rank[k] < room ? (uint64_t)oc * S + of + rank[k]
                                              : (uint64_t)first_w[bin] * S + (rank[k] - room);
          if (pos < pool_items) a.pool[pos] = make_int2(col[k], __float_as_int(c[k]));
        }
      }
    }
  };

  // This wavefront's rows.
  const int64_t G = (int64_t)gridDim.x * NW;
  const int64_t gw = (int64_t)blockIdx.x * NW + wave;
  const int64_t q = (a.nnz + G - 1) / G;
  int64_t rb64, re64;
  wave_lower_bound_pair(a.row_ptr, a.m, gw * q, (gw + 1) * q, rb64, re64);
  const int32_t rb = (int32_t)rb64;
  const int32_t re = (gw + 1 == G) ? (int32_t)a.m : (int32_t)re64;

  auto issue = [&](int32_t r, int32_t re_, uint32_t first_entry, WaveTile<K>& g) {
    g.rp = a.row_ptr[min(r + lane, re_)];
    g.rp1 = a.row_ptr[min(r + lane + 1, re_)];
    g.v = HAS_V ? a.v[min(r + lane, re_ - 1)] : 1.0f;
    load_clamped(first_entry & ~3u, g.val, g.col);
  };
  constexpr bool kGatherAhead = kGathers && YMODE != kYLds;

  int32_t r = rb;
  auto step = [&](WaveTile<K>& g, WaveTile<K>& gn) -> bool {
    const uint32_t pa = (uint32_t)__builtin_amdgcn_readfirstlane(g.rp);
    const uint32_t base = pa & ~3u;
    const bool valid = r + lane < re;
    const bool fits = valid && ((uint32_t)g.rp1 - base <= (uint32_t)TW);
    const int R = __popcll(__ballot(fits));  // fits holds for a prefix of the lanes
    const bool long_row = R == 0;            // row r alone holds more entries than a tile
    const uint32_t pb = (uint32_t)__shfl(g.rp1, long_row ? 0 : R - 1, 64);
    const int32_t r_next = r + (long_row ? 1 : R);
    const bool more = r_next < re;
    const uint32_t e0 = base + (uint32_t)lane * K;
    const uint32_t len = pb - pa;
    // the next tile's row_ptr, v and entries (they start where this tile ends); after the last
    // tile the same loads read this tile's entries again (cached) instead of the next
    // wavefront's, with no branch around them
    issue(min(r_next, re - 1), re, more ? pb : pa, gn);
    if constexpr (kGathers && !kGatherAhead) {
#pragma unroll
      for (int k = 0; k < K; ++k) g.yv[k] = gather_y(g.col[k]);
    }

    bool ok[K];
#pragma unroll
    for (int k = 0; k < K; ++k) ok[k] = e0 + k - pa < len;  // unsigned: positions before pa wrap

    if (long_row) {
      // The wavefront takes the row in slices of TW entries, twice (the dot, then the scatter);
      // the first slice is in registers for the dot, and each later slice is requested while
      // the one before is used.
      float hv[K], nv[K];
      int32_t hc[K], nc[K];
      uint32_t sb;
      float u = __shfl(g.v, 0, 64);  // v of the row; the given u when the second half runs alone
      if constexpr (kGathers) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) s += ok[k] ? g.val[k] * g.yv[k] : 0.0f;
        sb = base + TW;  // < pb: the row does not fit one tile
        load_slice(sb, hv, hc);
        while (true) {
          float yy[K];
#pragma unroll
          for (int k = 0; k < K; ++k) yy[k] = gather_y(hc[k]);
          const uint32_t nb = sb + TW;
          load_slice(nb, nv, nc);
          const uint32_t h0 = sb + (uint32_t)lane * K;
#pragma unroll
          for (int k = 0; k < K; ++k) s += (h0 + k < pb) ? hv[k] * yy[k] : 0.0f;
          if (nb >= pb) break;
          sb = nb;
#pragma unroll
          for (int k = 0; k < K; ++k) {
            hv[k] = nv[k];
            hc[k] = nc[k];
          }
        }
        u *= group_sum(s, 64);
      }
      if constexpr (MODE == kWaveRowdot) {
        if (lane == 0) a.t_out[r] = a.alpha * u + (a.beta != 0.0f ? a.beta * a.t0[r] : 0.0f);
      } else {
        // the scatter reloads the first slice too, so that its registers are free in the loops
        sb = base;
        load_slice(sb, hv, hc);
        while (true) {
          const uint32_t nb = sb + TW;
          load_slice(nb, nv, nc);
          const uint32_t h0 = sb + (uint32_t)lane * K;
          float c[K];
          bool on[K];
#pragma unroll
          for (int k = 0; k < K; ++k) {
            on[k] = h0 + k - pa < len;  // unsigned: positions before pa wrap
            c[k] = u * hv[k];
          }
          scatter_k(c, hc, on);
          if (nb >= pb) break;
          sb = nb;
#pragma unroll
          for (int k = 0; k < K; ++k) {
            hv[k] = nv[k];
            hc[k] = nc[k];
          }
        }
      }
    } else {
      // row-start marks of the tile's nonempty rows
      if (lane < R && g.rp1 > g.rp) mark_s[wave][(uint32_t)g.rp - base] = (uint8_t)(lane + 1);
      wave_lds_sync();
      int mk[K];
      {
        u2* mw = reinterpret_cast<u2*>(&mark_s[wave][lane * K]);
        const u2 w = *mw;
        *mw = u2{0u, 0u};  // cleared for the next tile
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          mk[k] = (int)((w.x >> (8 * k)) & 0xffu) - 1;
          mk[4 + k] = (int)((w.y >> (8 * k)) & 0xffu) - 1;
        }
      }
      // the row of each entry: the latest mark at or before it, within the lane, then across
      // the wavefront (slots before the tile's first entry read row 0 and are masked)
      int rk[K];
      int run_max = -1;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        run_max = max(run_max, mk[k]);
        mk[k] = run_max;
      }
      const int before = max(0, dpp_int<dpp::kWaveShr1>(-1, wave_max_scan(run_max)));
#pragma unroll
      for (int k = 0; k < K; ++k) rk[k] = max(before, mk[k]);  // in [0, R)
      // per-row dots: runs of one row inside the lane summed in registers; a row strictly
      // inside the lane is stored; the first and last runs are finished by a segmented sum
      // across the wavefront. Every row ends inside the tile, so each gets one write. Slots
      // outside the tile belong to its first row (before it) or its last nonempty row (after
      // it) and add a zero product there, so the row logic needs no mask. Lane j then scales
      // the dot of the tile's row j by that row's v, which it holds.
      if constexpr (MODE == kWaveTmv) {
        u_s[wave][lane] = g.v;  // the given u of the tile's rows
      } else {
      float pk[K];
#pragma unroll
      for (int k = 0; k < K; ++k) pk[k] = ok[k] ? g.val[k] * g.yv[k] : 0.0f;
      const int r0 = rk[0], r1 = rk[K - 1];
      float head = 0.0f, run = pk[0];
#pragma unroll
      for (int k = 1; k < K; ++k) {
        const bool fresh = rk[k] != rk[k - 1];
        if (fresh && rk[k - 1] != r0) u_s[wave][rk[k - 1]] = run;
        head = (fresh && rk[k - 1] == r0) ? run : head;
        run = fresh ? pk[k] : run + pk[k];
      }
      const float tails = wave_segmented_sum(run, r1);
      const float prev_tails = dpp_float<dpp::kWaveShr1>(0.0f, tails);
      const int prev_key = dpp_int<dpp::kWaveShr1>(-1, r1);
      const int next_r0 = dpp_int<dpp::kWaveShl1>(-1, r0);
      if (r0 != r1) u_s[wave][r0] = head + (prev_key == r0 ? prev_tails : 0.0f);
      if (next_r0 != r1) u_s[wave][r1] = tails;
      }
      wave_lds_sync();
      if constexpr (MODE == kWaveRowdot) {
        if (lane < R) {
          const float u = g.rp1 > g.rp ? g.v * u_s[wave][lane] : 0.0f;  // an empty row's dot is 0, whatever v
          a.t_out[r + lane] = a.alpha * u + (a.beta != 0.0f ? a.beta * a.t0[r + lane] : 0.0f);
        }
      } else {
        if constexpr (MODE == kWaveFused && HAS_V) {
          if (lane < R) u_s[wave][lane] *= g.v;
          wave_lds_sync();
        }
        float c[K];
#pragma unroll
        for (int k = 0; k < K; ++k) c[k] = u_s[wave][rk[k]] * g.val[k];
        scatter_k(c, g.col, ok);
      }
    }
    if (!more) return false;
    // the next tile's y gathers, a step ahead
    patch_tail(pb & ~3u, gn.val, gn.col);
    if constexpr (kGatherAhead) {
#pragma unroll
      for (int k = 0; k < K; ++k) gn.yv[k] = gather_y(gn.col[k]);
    }
    r = r_next;
    wave_lds_sync();  // this tile's LDS reads come before the next tile's writes
    return true;
  };

  if (rb < re) {
    WaveTile<K> ga, gb;
    const uint32_t p0 = (uint32_t)a.row_ptr[rb];
    issue(rb, re, p0, ga);
    patch_tail(p0 & ~3u, ga.val, ga.col);
    if constexpr (kGatherAhead) {
#pragma unroll
      for (int k = 0; k < K; ++k) ga.yv[k] = gather_y(ga.col[k]);
    }
    while (step(ga, gb) && step(gb, ga)) {
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

template <class VT, int BLK, int K, int YMODE, bool HAS_V, bool ALIGNED, int COLD, int MODE>
hipError_t launch_w(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  const size_t lds = csr_waves_dynamic_lds(a.lds_window, YMODE == kYGlobal ? 0 : a.y_window, a.bins, BLK);
  const void* fn = reinterpret_cast<const void*>(&csr_waves<VT, BLK, K, YMODE, HAS_V, ALIGNED, COLD, MODE>);
  hipError_t e = allow_dynamic_lds(fn);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((csr_waves<VT, BLK, K, YMODE, HAS_V, ALIGNED, COLD, MODE>), dim3((unsigned)p.grid), dim3(BLK), lds,
                     s, a);
  return hipGetLastError();
}

template <class VT, int BLK, int K, int YMODE, int COLD, int MODE>
hipError_t launch_wv(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  const bool al = a.aligned && a.nnz >= 4;  // vector loads need one whole quad of entries
  if (MODE == kWaveTmv || a.v != nullptr)   // u is always given to the second half
    return al ? launch_w<VT, BLK, K, YMODE, true, true, COLD, MODE>(a, p, s)
              : launch_w<VT, BLK, K, YMODE, true, false, COLD, MODE>(a, p, s);
  if constexpr (MODE != kWaveTmv)
    return al ? launch_w<VT, BLK, K, YMODE, false, true, COLD, MODE>(a, p, s)
              : launch_w<VT, BLK, K, YMODE, false, false, COLD, MODE>(a, p, s);
  return hipErrorInvalidValue;
}

template <class VT, int BLK, int K, int COLD, int MODE>
hipError_t launch_wy(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if constexpr (MODE == kWaveTmv) {
    return launch_wv<VT, BLK, K, kYGlobal, COLD, MODE>(a, p, s);  // no y
  } else {
    if (a.y_window >= a.n) return launch_wv<VT, BLK, K, kYLds, COLD, MODE>(a, p, s);
    if (a.y_window > 0) return launch_wv<VT, BLK, K, kYSplit, COLD, MODE>(a, p, s);
    return launch_wv<VT, BLK, K, kYGlobal, COLD, MODE>(a, p, s);
  }
}

template <class VT, int BLK, int K, int MODE>
hipError_t launch_wc(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if constexpr (MODE == kWaveRowdot) {
    return launch_wy<VT, BLK, K, kColdNone, MODE>(a, p, s);  // no scatter
  } else {
    if (a.bins > 0) return launch_wy<VT, BLK, K, kColdBinned, MODE>(a, p, s);
    if (a.lds_window < a.n) return launch_wy<VT, BLK, K, kColdAtomic, MODE>(a, p, s);
    return launch_wy<VT, BLK, K, kColdNone, MODE>(a, p, s);
  }
}

template <int MODE, class VT = float>
hipError_t launch_wb(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s) {
  if (p.block_threads == 256) return launch_wc<VT, 256, 8, MODE>(a, p, s);
  if (p.block_threads == 512) return launch_wc<VT, 512, 8, MODE>(a, p, s);
  if (p.block_threads == 1024) return launch_wc<VT, 1024, 8, MODE>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_csr_waves(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s, int mode) {
  if (p.grid <= 0 || p.grid > INT32_MAX || p.kernel != XTVXY_CSR_WAVES || p.entries_per_thread != 8)
    return hipErrorInvalidValue;
  if (a.nnz <= 0 || a.nnz > INT32_MAX || a.m <= 0 || a.m > INT32_MAX - 1024 || a.lds_window < 0 ||
      a.lds_window > a.n || a.y_window < 0 || a.y_window > a.n)
    return hipErrorInvalidValue;
  const bool binned = a.bins > 0;
  if (binned && (a.pool == nullptr || a.pool_next == nullptr || a.chunk_bin == nullptr || a.chunk_fill == nullptr ||
                 a.bins > kMaxBins || a.acc != nullptr))
    return hipErrorInvalidValue;
  if (a.value_bytes != 4 && a.value_bytes != 2) return hipErrorInvalidValue;
  const bool b16 = a.value_bytes == 2;  // bf16 values
  if (mode == kCsrRowdot) {
    // the first half alone: no output window and no scatter; t_out (and t0 when beta != 0)
    if (a.lds_window != 0 || binned || a.t_out == nullptr || (a.beta != 0.0f && a.t0 == nullptr))
      return hipErrorInvalidValue;
    return b16 ? launch_wb<kWaveRowdot, bf16_t>(a, p, s) : launch_wb<kWaveRowdot>(a, p, s);
  }
  if (!binned && a.lds_window < a.n && a.acc == nullptr) return hipErrorInvalidValue;
  if (mode == kCsrTmv) {
    if (a.v == nullptr) return hipErrorInvalidValue;  // u
    return b16 ? launch_wb<kWaveTmv, bf16_t>(a, p, s) : launch_wb<kWaveTmv>(a, p, s);
  }
  if (mode != kCsrFused) return hipErrorInvalidValue;
  return b16 ? launch_wb<kWaveFused, bf16_t>(a, p, s) : launch_wb<kWaveFused>(a, p, s);
}

}  // namespace xtvxy
