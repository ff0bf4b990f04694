// Analytical launch-parameter model.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract): an
// analytical model takes the characteristics of the input and the resources of
// the GPU and estimates near-optimal kernel launch parameters. The page gives
// no formula; this model is the plainest one for a kernel bound by HBM
// bandwidth:
//
//   time(plan) = bytes(X, v, y, z, out) / bandwidth(plan)
//              + bytes(partials written and read back) / bandwidth
//              + launches * launch_cost
//   bandwidth(plan) = min(sustained_fraction * peak,
//                         compute_units * bytes_in_flight_per_cu / latency)
//
// where bytes_in_flight_per_cu follows from the row layout (rows kept in
// flight per workgroup times their bytes) and the workgroups resident per CU.
// The row layout itself is fixed by n (the smallest layout that covers a row),
// so the model chooses the number of workgroups per CU, hence the grid and the
// coarsening factor rows_per_unit = ceil(m / units). More workgroups hide
// more latency but write more partial n-vectors; the model trades the two, and
// never asks for more workgroups per CU than the chosen kernel can keep resident
// (a grid beyond that runs as a second, thinly populated round).
// The constants are calibrated on MI355X: a plain streaming read sustains
// about 0.88 of the 8 TB/s peak; the CSR and group-row kernels reach it once
// about 128 KiB of loads are in flight per CU (about 4.5 us of latency under
// load), the dense wave- and block-row kernels with about 2 us worth.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "internal.h"

namespace xtvxy {
namespace {

constexpr double kSustained = 0.88;     // sustained fraction of peak HBM bandwidth (streaming read)
constexpr double kLatency = 4.5e-6;     // seconds of loaded-memory latency that loads in flight must cover
// The dense wave- and block-row kernels need no barrier between their rows' loads and reach the
// sustained rate with about 2 us worth of loads in flight (one 32 KiB workgroup per CU streams
// ~6.7 TB/s); the group-row kernels wait for the other members every two rows and keep kLatency.
constexpr double kLatencyDenseRows = 2.0e-6;
constexpr double kLaunch = 3.0e-6;      // seconds per dependent kernel launch
constexpr int kMaxWgPerCu = 8;          // 256-thread workgroups per CU (32 wavefronts)
constexpr double kAtomicRate = 2.0e10;  // global fp32 atomics per second on distinct addresses (measured)
constexpr int64_t kCsrLdsBudget = 64 * 1024;  // CSR: LDS bytes for the output and y windows
constexpr int kCsrThreadsPerCuLarge = 1024;  // CSR: threads per CU the windows leave room for when n is large
constexpr int64_t kWaveRowsMaxMean = 128;     // CSR: mean entries per row up to which the wavefront kernel is used
constexpr int kMaxThreadsPerCu = 2048;       // 32 wavefronts

int next_pow2(int64_t x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

double bandwidth(const xtvxy_device_info& d, double inflight_per_cu, double latency = kLatency) {
  const double bw_latency = d.compute_units * inflight_per_cu / latency;
  return std::min(kSustained * d.hbm_bytes_per_s, bw_latency);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Wave-row layout: rows a wavefront keeps in flight per row group and column chunks.
int wave_unroll(int chunks) { return 8 / chunks; }

}  // namespace

DenseWorkspace dense_workspace(int64_t n, const xtvxy_launch_params& p, int elem_bytes) {
  DenseWorkspace w{};
  if (p.kernel == XTVXY_DENSE_GROUP_ROWS) {
    const int64_t groups = p.grid / std::max<int32_t>(p.group, 1);
    w.partial_rows = (size_t)groups;
    w.partial_off = 0;
    w.xchg_off = align_up(w.partial_off + (size_t)groups * n * sizeof(float));
    w.error_off =
        align_up(w.xchg_off + (size_t)groups * 2 * p.group * group_rows_per_step(p.chunks, p.vec, elem_bytes) *
                                  sizeof(uint64_t));
    w.total = align_up(w.error_off + sizeof(uint32_t));
  } else {
    w.partial_rows = (size_t)p.grid;
    w.partial_off = 0;
    w.total = align_up((size_t)p.grid * n * sizeof(float));
  }
  return w;
}

CsrWorkspace csr_workspace(int64_t m, int64_t n, int64_t nnz, const xtvxy_launch_params& p, int64_t binned) {
  (void)m;
  CsrWorkspace w{};
  w.partial_off = 0;
  w.partial_rows = (size_t)p.grid;
  size_t off = align_up((size_t)p.grid * (size_t)p.lds_window * sizeof(float));
  if (p.lds_window >= n) {
    w.total = off;
    return w;
  }
  if (p.bin_columns <= 0) {
    w.acc_off = off;
    w.total = align_up(off + (size_t)n * sizeof(float));
    return w;
  }
  // binning: every (workgroup, bin) pair (the wavefront kernel: every (wavefront, bin) pair)
  // leaves at most one chunk partly filled, so ceil(items / S) + owners * B chunks always suffice,
  // items being the binned entries (all nnz when their number is not known)
  int shift = 0;
  while ((1 << shift) < p.bin_columns) ++shift;
  w.bin_shift = shift;
  w.bins = (int32_t)ceil_div(n - p.lds_window, (int64_t)p.bin_columns);
  const int64_t owners = p.kernel == XTVXY_CSR_WAVES || p.kernel == XTVXY_CSR_ROWS
                             ? p.grid * (int64_t)(p.block_threads / 64)
                             : p.grid;
  const int64_t items = binned >= 0 ? std::min(binned, nnz) : nnz;
  w.pool_chunks = ceil_div(std::max<int64_t>(items, 1), kBinChunkItems) + owners * (int64_t)w.bins;
  w.max_units = ceil_div(w.pool_chunks, kBinUnitChunks) + w.bins;
  w.counter_off = off;
  off = align_up(off + sizeof(uint32_t));
  w.pool_off = off;
  off = align_up(off + (size_t)w.pool_chunks * kBinChunkItems * 2 * sizeof(int32_t));
  w.chunk_bin_off = off;
  off = align_up(off + (size_t)w.pool_chunks * sizeof(int32_t));
  w.chunk_fill_off = off;
  off = align_up(off + (size_t)w.pool_chunks * sizeof(int32_t));
  w.order_off = off;
  off = align_up(off + (size_t)w.pool_chunks * sizeof(int32_t));
  w.counts_off = off;
  off = align_up(off + (size_t)w.bins * kBinSortGroups * sizeof(int32_t));
  w.bin_start_off = off;
  off = align_up(off + (size_t)(w.bins + 1) * sizeof(int32_t));
  w.unit_start_off = off;
  off = align_up(off + (size_t)(w.bins + 1) * sizeof(int32_t));
  w.partial2_off = off;
  off = align_up(off + (size_t)w.max_units * (size_t)p.bin_columns * sizeof(float));
  w.total = off;
  return w;
}

xtvxy_status complete_dense(int64_t m, int64_t n, int64_t ldx, const xtvxy_device_info& d,
                            xtvxy_launch_params* p, int elem_bytes) {
  (void)ldx;
  if (elem_bytes != 4 && elem_bytes != 2) return XTVXY_ERROR_INVALID_VALUE;
  const int wide = 16 / elem_bytes;  // elements per 16-byte load: 4 fp32 or 8 bf16
  if (p->block_threads != kBlock || (p->vec != 1 && p->vec != wide) || p->grid <= 0 || p->grid > INT32_MAX)
    return XTVXY_ERROR_INVALID_VALUE;
  if (p->vec == wide && n % wide != 0) return XTVXY_ERROR_INVALID_VALUE;  // chunks never straddle the row end
  switch (p->kernel) {
    case XTVXY_DENSE_WAVE_ROWS: {
      const int lpr = p->lanes_per_row;
      if (lpr < 1 || lpr > 64 || (lpr & (lpr - 1)) != 0) return XTVXY_ERROR_INVALID_VALUE;
      if (p->chunks != 1 && p->chunks != 2 && p->chunks != 4) return XTVXY_ERROR_INVALID_VALUE;
      if ((int64_t)lpr * p->vec * p->chunks < n) return XTVXY_ERROR_INVALID_VALUE;
      p->group = 1;
      break;
    }
    case XTVXY_DENSE_BLOCK_ROWS:
    case XTVXY_DENSE_GROUP_ROWS: {
      if (p->chunks != 1 && p->chunks != 2 && p->chunks != 4 && p->chunks != 8) return XTVXY_ERROR_INVALID_VALUE;
      if (elem_bytes == 2 && p->vec == 8 && p->chunks == 8) return XTVXY_ERROR_INVALID_VALUE;  // registers
      const int64_t slice = (int64_t)kBlock * p->vec * p->chunks;
      if (p->kernel == XTVXY_DENSE_BLOCK_ROWS) {
        p->group = 1;
        if (slice < n) return XTVXY_ERROR_INVALID_VALUE;
      } else {
        if (p->group < 1 || p->group > kGroupMaxMembers || (int64_t)p->group * slice < n ||
            p->grid % p->group != 0)
          return XTVXY_ERROR_INVALID_VALUE;
      }
      p->lanes_per_row = kBlock;
      break;
    }
    default:
      return XTVXY_ERROR_INVALID_VALUE;
  }
  const int64_t units = p->grid / p->group;
  if (p->rows_per_unit <= 0) p->rows_per_unit = std::max<int64_t>(1, ceil_div(m, units));
  if (p->rows_per_unit * units < m) return XTVXY_ERROR_INVALID_VALUE;
  p->workspace_bytes = (int64_t)dense_workspace(n, *p, elem_bytes).total;
  (void)d;
  return XTVXY_SUCCESS;
}

xtvxy_status model_dense(int64_t m, int64_t n, int64_t ldx, bool aligned16, const xtvxy_device_info& d,
                         xtvxy_launch_params* p, int elem_bytes, int max_wg_per_cu) {
  std::memset(p, 0, sizeof(*p));
  if (elem_bytes != 4 && elem_bytes != 2) return XTVXY_ERROR_INVALID_VALUE;
  p->block_threads = kBlock;
  const int wide = 16 / elem_bytes;  // elements per 16-byte load
  p->vec = (aligned16 && ldx % wide == 0 && n % wide == 0) ? wide : 1;
  const int vec = p->vec;
  const int max_chunks = (elem_bytes == 2 && vec == 8) ? 4 : 8;  // block/group rows
  double inflight_per_wg;  // bytes of X a workgroup has requested before it needs the first of them
  int64_t rows_per_step;   // rows a workgroup (or group) consumes per step
  if (n <= 64 * vec * 4) {
    p->kernel = XTVXY_DENSE_WAVE_ROWS;
    p->chunks = (n <= 64 * vec) ? 1 : (n <= 128 * vec) ? 2 : 4;
    p->lanes_per_row = next_pow2(std::max<int64_t>(1, ceil_div(n, (int64_t)vec * p->chunks)));
    p->group = 1;
    rows_per_step = (int64_t)kWaves * (64 / p->lanes_per_row) * wave_unroll(p->chunks);
    inflight_per_wg = (double)rows_per_step * n * elem_bytes;
  } else if (n <= (int64_t)kBlock * vec * max_chunks) {
    p->kernel = XTVXY_DENSE_BLOCK_ROWS;
    const int64_t per = (int64_t)kBlock * vec;
    p->chunks = (n <= per) ? 1 : (n <= 2 * per) ? 2 : (n <= 4 * per) ? 4 : 8;
    p->group = 1;
    p->lanes_per_row = kBlock;
    rows_per_step = block_rows_per_step(p->chunks, vec, elem_bytes);
    inflight_per_wg = (double)rows_per_step * n * elem_bytes;
  } else {
    p->kernel = XTVXY_DENSE_GROUP_ROWS;
    const int64_t per = (int64_t)kBlock * vec;
    p->group = (int32_t)ceil_div(n, per * max_chunks);
    const int64_t slice = ceil_div(n, p->group);
    p->chunks = (slice <= per) ? 1 : (slice <= 2 * per) ? 2 : (slice <= 4 * per) ? 4 : 8;
    p->lanes_per_row = kBlock;
    rows_per_step = group_rows_per_step(p->chunks, p->vec, elem_bytes);
    inflight_per_wg = (double)rows_per_step * slice * elem_bytes;
  }

  const double io_bytes = (double)elem_bytes * m * n + 4.0 * ((double)m + 3.0 * n);
  // workgroups per CU: at most what the kernel's registers and LDS let reside at once, when known
  int max_per_cu = (p->kernel == XTVXY_DENSE_GROUP_ROWS) ? 2 : kMaxWgPerCu;
  if (max_wg_per_cu > 0) max_per_cu = std::min(max_per_cu, max_wg_per_cu);
  double best = 1e300;
  int64_t best_grid = 1;
  for (int k = 1; k <= max_per_cu; k *= 2) {
    int64_t grid = (int64_t)d.compute_units * k;
    const int64_t units_needed = std::max<int64_t>(1, ceil_div(m, rows_per_step));  // no idle units
    if (p->kernel == XTVXY_DENSE_GROUP_ROWS) {
      grid = grid / p->group * p->group;
      if (grid < p->group) grid = p->group;
      grid = std::min<int64_t>(grid, units_needed * p->group);
    } else {
      grid = std::min<int64_t>(grid, units_needed);
    }
    const double resident_per_cu = std::min<double>(k, (double)grid / d.compute_units);
    const double latency = p->kernel == XTVXY_DENSE_GROUP_ROWS ? kLatency : kLatencyDenseRows;
    const double bw = bandwidth(d, std::max(resident_per_cu, 1.0 / d.compute_units) * inflight_per_wg, latency);
    const double partial_bytes = 2.0 * (double)(grid / p->group) * n * sizeof(float);
    const double t = io_bytes / bw + partial_bytes / (kSustained * d.hbm_bytes_per_s) + 2 * kLaunch;
    // The group-row kernel takes as many workgroups per CU as reside (at most two), whatever the
    // cost says: its members wait for each other's dots with nothing in flight, which the cost
    // does not see, and a second workgroup streams meanwhile (8192 x 65536: one per CU 40% slower).
    const bool group_more = p->kernel == XTVXY_DENSE_GROUP_ROWS;
    if (t < best * 0.999 || group_more) {
      best = t;
      best_grid = grid;
    }
  }
  p->grid = best_grid;
  p->rows_per_unit = 0;
  p->predicted_seconds = best;
  return complete_dense(m, n, ldx, d, p, elem_bytes);
}

int64_t csr_fused_lds(int64_t n, const xtvxy_launch_params& p, int32_t bins) {
  (void)n;
  if (p.kernel == XTVXY_CSR_WAVES)
    return (int64_t)(csr_waves_dynamic_lds(p.lds_window, p.y_window, bins, p.block_threads) +
                     csr_waves_static_lds(p.block_threads));
  if (p.kernel == XTVXY_CSR_ROWS)
    return (int64_t)csr_rows_dynamic_lds(p.lds_window, p.y_window, bins, p.block_threads);
  int64_t lds = ((int64_t)p.lds_window + (int64_t)p.y_window) * (int64_t)sizeof(float);
  if (bins > 0) lds = ((lds + 7) & ~(int64_t)7) + (int64_t)bins * (int64_t)kCsrBinStateBytes;
  return lds + (int64_t)csr_static_lds(p.entries_per_thread, p.block_threads);
}

xtvxy_status complete_csr(int64_t m, int64_t n, int64_t nnz, const xtvxy_device_info& d,
                          xtvxy_launch_params* p) {
  if ((p->kernel != XTVXY_CSR_TILES && p->kernel != XTVXY_CSR_WAVES && p->kernel != XTVXY_CSR_ROWS) ||
      p->grid <= 0 || p->grid > INT32_MAX)
    return XTVXY_ERROR_INVALID_VALUE;
  // (threads, entries per thread): tiles 256 x 4, 256 x 8 or 512 x 8; wavefronts 256, 512 or 1024 x 8;
  // row classes 256, 512 or 1024 x 16
  const bool any_blk = p->block_threads == 256 || p->block_threads == 512 || p->block_threads == 1024;
  const bool shape_ok =
      p->kernel == XTVXY_CSR_TILES
          ? (p->block_threads == 256 && (p->entries_per_thread == 4 || p->entries_per_thread == 8)) ||
                (p->block_threads == 512 && p->entries_per_thread == 8)
          : any_blk && p->entries_per_thread == (p->kernel == XTVXY_CSR_ROWS ? kRowsSlots : 8);
  if (!shape_ok) return XTVXY_ERROR_INVALID_VALUE;
  if (p->lds_window < 0 || p->lds_window > n || p->y_window < 0 || p->y_window > n)
    return XTVXY_ERROR_INVALID_VALUE;
  const int32_t bc = p->bin_columns;
  if (bc != 0 && (bc < 1024 || bc > 32768 || (bc & (bc - 1)) != 0)) return XTVXY_ERROR_INVALID_VALUE;
  if (p->lds_window >= n) p->bin_columns = 0;  // nothing outside the window
  const int32_t bins = p->bin_columns > 0 ? (int32_t)ceil_div(n - p->lds_window, p->bin_columns) : 0;
  if (bins > kMaxBins) return XTVXY_ERROR_INVALID_VALUE;
  if (csr_fused_lds(n, *p, bins) > d.lds_bytes) return XTVXY_ERROR_INVALID_VALUE;
  if (bins > 0 && (int64_t)p->bin_columns * (int64_t)sizeof(float) > d.lds_bytes) return XTVXY_ERROR_INVALID_VALUE;
  p->group = 1;
  const CsrWorkspace w = csr_workspace(m, n, nnz, *p);
  if (bins > 0 && (w.pool_chunks > INT32_MAX || (uint64_t)w.pool_chunks * kBinChunkItems > UINT32_MAX * 4ull ||
                   w.max_units > INT32_MAX))
    return XTVXY_ERROR_UNSUPPORTED;
  p->workspace_bytes = (int64_t)w.total;
  return XTVXY_SUCCESS;
}

xtvxy_status model_csr(int64_t m, int64_t n, int64_t nnz, const xtvxy_device_info& d, xtvxy_launch_params* p,
                       bool fused) {
  std::memset(p, 0, sizeof(*p));
  p->kernel = XTVXY_CSR_TILES;
  p->block_threads = 256;
  p->vec = 1;
  p->chunks = 1;
  p->group = 1;
  p->entries_per_thread = 8;
  // Both windows (the output columns accumulated in LDS, and the part of y gathered from
  // LDS) cover all of n when they fit a budget that leaves room for several workgroups per
  // CU. Otherwise latency hiding matters more than window size (measured on a Zipf-skewed
  // 10^6-column matrix): workgroups of 512 threads (tiles of 4096 entries, half the barriers
  // per entry), sized so that two fit on a CU, and the windows share the LDS that leaves,
  // three parts for the output and one for y. The columns outside the output window are binned when
  // the bins fit (bins of 16384 columns, or 32768 when there would be too many), else sent to
  // global atomics. Binning costs a write and a read of 8 bytes per cold product and two more
  // launches; atomics run at about kAtomicRate.
  int32_t bins = 0;
  if ((int64_t)n * 8 <= kCsrLdsBudget) {
    p->lds_window = (int32_t)n;
    p->y_window = (int32_t)n;
  } else {
    p->lds_window = (int32_t)std::min<int64_t>(n, kCsrLdsBudget / 8);
    p->y_window = p->lds_window;
    p->block_threads = 512;
    for (int32_t bc = 16384; bc <= 32768; bc *= 2) {
      const int64_t b = ceil_div(n, bc);  // at least as many bins as any window leaves
      if (b > kMaxBins) continue;
      const int64_t avail = d.lds_bytes / (kCsrThreadsPerCuLarge / p->block_threads) - 512 -
                            (int64_t)csr_static_lds(p->entries_per_thread, p->block_threads) -
                            8 - b * (int64_t)kCsrBinStateBytes;
      const int64_t cols = std::max<int64_t>(avail, 0) / 4;
      bins = (int32_t)ceil_div(n - std::min<int64_t>(n, cols * 3 / 4), bc);
      p->bin_columns = bc;
      p->lds_window = (int32_t)std::min<int64_t>(n, cols * 3 / 4);
      p->y_window = (int32_t)std::min<int64_t>(n, cols - p->lds_window);
      break;
    }
  }
  const int64_t wg_lds = csr_fused_lds(n, *p, bins);
  const int max_per_cu =
      (int)std::max<int64_t>(1, std::min<int64_t>(kMaxThreadsPerCu / p->block_threads, d.lds_bytes / wg_lds));
  const double io_bytes = 8.0 * nnz + 4.0 * (m + 1) + 4.0 * m + 12.0 * n;
  const int64_t tile = (int64_t)p->block_threads * p->entries_per_thread;
  // the model knows nothing of the column distribution: it prices the columns outside
  // the window as uniformly hit
  const double cold = n > 0 ? (double)(n - p->lds_window) / n * nnz : 0.0;
  double cold_cost = cold / kAtomicRate;
  if (bins > 0) {
    const double binned = 16.0 * cold / (kSustained * d.hbm_bytes_per_s) +
                          (cold / ((double)kBinChunkItems * kBinUnitChunks) + bins) * p->bin_columns * 8.0 /
                              (kSustained * d.hbm_bytes_per_s) +
                          2 * kLaunch + 5e-6;
    if (binned < cold_cost) {
      cold_cost = binned;
    } else {
      p->bin_columns = 0;
    }
  }
  double best = 1e300;
  int64_t best_grid = 1;
  for (int k = 1; k <= max_per_cu; k *= 2) {
    int64_t grid = (int64_t)d.compute_units * k;
    grid = std::max<int64_t>(1, std::min<int64_t>(grid, ceil_div(std::max<int64_t>(nnz, 1), tile)));
    const double resident = std::min<double>(k, (double)grid / d.compute_units);
    const double bw = bandwidth(d, std::max(resident, 1.0 / d.compute_units) * tile * 8.0);
    const double partial_bytes = 2.0 * grid * p->lds_window * sizeof(float);
    const double t = io_bytes / bw + partial_bytes / (kSustained * d.hbm_bytes_per_s) + cold_cost +
                     3 * kLaunch;
    if (t < best * 0.999) {
      best = t;
      best_grid = grid;
    }
  }
  p->grid = best_grid;
  p->predicted_seconds = best;
  xtvxy_status st = complete_csr(m, n, nnz, d, p);
  if (st != XTVXY_SUCCESS || !fused) return st;
  // Narrow matrices (both windows hold all of n) with at most kWaveRowsMaxMean entries per row on
  // average: the wavefront kernel on the same grid. Its tiles of 512 entries are one wavefront's,
  // so it needs no workgroup barrier per tile. Measured on narrow matrices of 500 to 8192 columns
  // (uniform rows of 3 to 100 entries, and Zipf rows of mean 19 and 40 with rows of up to 600 and
  // 2726 entries) it ran 7-26% faster than the workgroup tiles at their best grid; rows longer
  // than a tile take two sweeps, so much longer mean rows keep the workgroup tiles. The halves
  // alone keep them too:
  // without a scatter (rowdot) or without gathers (tmv) the tiles' barriers cost little, and the
  // wavefront kernel measured no faster (rowdot) or 6% slower (tmv) there.
  if (p->lds_window == n && p->y_window == n && p->block_threads == 256 && p->entries_per_thread == 8 &&
      nnz <= kWaveRowsMaxMean * m) {
    xtvxy_launch_params q = *p;
    q.kernel = XTVXY_CSR_WAVES;
    if (complete_csr(m, n, nnz, d, &q) == XTVXY_SUCCESS) *p = q;
  }
  return XTVXY_SUCCESS;
}

bool refine_waves_grid(int64_t m, int64_t n, int64_t nnz, int64_t longest_row, const xtvxy_device_info& d,
                       xtvxy_launch_params* p) {
  // When every row fits a 512-slot tile (a row of len entries spans len + 3 slots from its quad)
  // and rows hold 8 or more entries on average, the wavefront kernel's tiles are full, and three
  // 256-thread workgroups per CU ran fastest (uniform rows of 10-100 entries: 7-8% faster than
  // four). Shorter rows (tiles capped at 64 rows) or rows longer than a tile (two sweeps) ran
  // faster with four or more, the model's choice.
  if (p->kernel != XTVXY_CSR_WAVES || p->block_threads != 256 || longest_row + 3 > 512 || nnz < 8 * m ||
      p->grid <= 3 * (int64_t)d.compute_units)
    return false;
  xtvxy_launch_params q = *p;
  q.grid = 3 * (int64_t)d.compute_units;
  if (complete_csr(m, n, nnz, d, &q) != XTVXY_SUCCESS) return false;
  *p = q;
  return true;
}

}  // namespace xtvxy
