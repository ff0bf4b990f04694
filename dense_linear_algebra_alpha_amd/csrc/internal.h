// Internal declarations shared by the host layer (api.cpp, model.cpp) and the
// kernels (*.hip) of the xtvxy library. Not installed; the public ABI is
// include/xtvxy.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "xtvxy.h"

namespace xtvxy {

constexpr int kBlock = 256;          // threads per workgroup of every fused kernel
constexpr int kWaves = kBlock / 64;  // wavefronts per workgroup
constexpr int kBlockRowsInFlight = 2;  // rows a block-row workgroup loads per step (but see below)
// Rows a group-row workgroup loads per step, i.e. per exchange of partial dots between the
// members. Each thread's column sums live in LDS, so a step's rows may take 128 registers: fp32
// 4 rows of 8 chunks of 4 floats (at most 16 rows); 16-bit elements stay packed (two to a
// register, widened at each use), so 8 rows of 4 chunks of 8, or 16 rows of 1 or 2 chunks, and
// 2 rows of 8 chunks (their y takes 64 registers). Fewer chunks per thread (wider groups) buy
// more rows per exchange.
// Members of a group-row group at most: 128 x 8192 = 1,048,576 columns with 16-byte loads.
constexpr int kGroupMaxMembers = 128;
constexpr int group_rows_per_step(int chunks, int vec, int elem_bytes) {
  if (chunks < 1 || chunks > 16) return 1;
  if (elem_bytes == 2) return chunks <= 2 ? 16 : chunks == 4 ? 8 : 16 / chunks;
  const int words = chunks * (vec > 0 ? vec : 1);  // fp32: one register per element
  return words >= 128 ? 1 : (128 / words > 16 ? 16 : 128 / words);
}
// fp32 block rows of 8 chunks of 4 (too many registers for the next step's rows to be requested
// early) keep their column sums in LDS like the group rows and take as many rows per step
// (4 instead of 2); every other block-row layout takes kBlockRowsInFlight rows and its prefetch.
constexpr bool block_sums_in_lds(int chunks, int vec, int elem_bytes) {
  return elem_bytes == 4 && vec == 4 && chunks == 8;
}
constexpr int block_rows_per_step(int chunks, int vec, int elem_bytes) {
  return block_sums_in_lds(chunks, vec, elem_bytes) ? group_rows_per_step(chunks, vec, elem_bytes)
                                                     : kBlockRowsInFlight;
}
// CSR kernel: LDS besides the output and y windows, for workgroups of `blk` threads holding
// `ept` entries each: row_ptr, v and dots of two tiles, a sink word per thread and small
// scalars (29 blk + 64 bytes), plus two tiles of 16-bit row-start marks (4 blk ept bytes)
constexpr size_t csr_static_lds(int ept, int blk) { return 29 * (size_t)blk + 256 + 4 * (size_t)blk * ept; }
constexpr size_t kAlign = 256;       // alignment of every workspace region
// CSR binning of the columns outside the LDS window
constexpr int kBinChunkItems = 512;  // (column, product) items per workspace chunk (4 KiB)
constexpr int kMaxBins = 512;        // column bins of one call
constexpr int kBinUnitChunks = 128;  // chunks one workgroup of the bin pass accumulates
constexpr int kBinSortGroups = 256;  // workgroups of the counting sort of chunks by bin
// LDS of the fused CSR kernel for the per-bin state (count, current chunk, fill, room, two
// positions) when binning
constexpr size_t kCsrBinStateBytes = 32;
// Wavefront CSR kernel (csr_waves.hip): static LDS per workgroup of `blk` threads (row-start
// marks of 512 entry slots, u of 64 rows per wavefront, a sink word per thread), and the
// dynamic LDS: output and y windows, then each wavefront's bin state (6 words per bin).
constexpr size_t kCsrWaveBinStateBytes = 24;
constexpr size_t csr_waves_static_lds(int blk) { return (size_t)(blk / 64) * (512 + 256) + 4 * (size_t)blk; }
constexpr size_t csr_waves_dynamic_lds(int64_t window, int64_t y_window, int32_t bins, int blk) {
  return (((size_t)(window + y_window) * 4 + 7) & ~(size_t)7) +
         (bins > 0 ? (size_t)bins * kCsrWaveBinStateBytes * (size_t)(blk / 64) : 0);
}
// Row-class CSR kernel (csr_rows.hip): no static LDS; the dynamic LDS holds the output and y
// windows, a sink word per thread, then each wavefront's bin state (6 words per bin).
constexpr int kRowsSlots = 8;       // entry slots per lane and batch (two 16-byte quads)
constexpr int kRowsVeryLong = 7;    // class of the rows longer than a wavefront's 64 * 8 slots
constexpr size_t csr_rows_dynamic_lds(int64_t window, int64_t y_window, int32_t bins, int blk) {
  return (size_t)(window + y_window + blk) * 4 +
         (bins > 0 ? (size_t)bins * kCsrWaveBinStateBytes * (size_t)(blk / 64) : 0);
}
// Class of a nonempty row of `len` entries: the smallest c with len + 3 <= 8 * 2^c (a group of 2^c
// lanes covers the row's quads, whatever the row's first entry mod 4), kRowsVeryLong beyond c = 6.
constexpr int csr_row_class(int64_t len) {
  return len + 3 <= 8 ? 0 : len + 3 <= 16 ? 1 : len + 3 <= 32 ? 2 : len + 3 <= 64 ? 3
       : len + 3 <= 128 ? 4 : len + 3 <= 256 ? 5 : len + 3 <= 512 ? 6 : kRowsVeryLong;
}

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Arguments of the dense fused kernels.
struct DenseArgs {
  int64_t m, n, ldx;
  const void* X;      // fp32 or 16-bit elements (elem_bytes 4 or 2)
  int32_t elem_bytes;
  int32_t f16;        // 16-bit elements are fp16 (1) or bf16 (0)
  const float* v;     // nullptr: v = 1
  const float* y;
  float* partial;     // [rows of partials][n] fp32
  int64_t rows_per_unit;
  int32_t lanes_per_row;
  int32_t group;      // group-row path: workgroups per row
  void* xchg;         // group-row path: [groups][2][group][rows per step] 64-bit tagged slots (zeroed)
  uint32_t* error;    // group-row path: set when a wait for the other members gives up
  uint32_t wait_polls;     // group-row path: polls before a wait gives up (0: the kernel's own bound)
  uint32_t wait_tag_skew;  // group-row path: 0; nonzero only under the failure-path test hook (the
                           // waits then look for a step tag nobody publishes and always give up)
};

// Arguments of the CSR fused kernels.
struct CsrArgs {
  int64_t m, n, nnz;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const void* values;     // fp32, or bf16 bit patterns when value_bytes == 2
  int32_t value_bytes;    // 4 or 2
  const float* v;
  const float* y;
  float* partial;     // [grid][lds_window] per-workgroup partial sums of output columns [0, lds_window)
  float* acc;         // [n] global accumulator of columns >= lds_window (zeroed before launch), or null
  int64_t lds_window;
  int64_t y_window;   // y[0, y_window) is gathered from an LDS copy, the rest from global memory
  bool aligned;       // col_idx 16-byte and values 16-byte (fp32) or 8-byte (bf16) aligned:
                      // entries load as vectors
  // the first half of the pattern alone (launch mode kCsrRowdot): t_out = alpha v .* (X y) + beta t0
  float alpha, beta;
  const float* t0;    // read only when beta != 0 (may equal t_out)
  float* t_out;
  // binning of the columns >= lds_window (bins > 0; acc is then null)
  int32_t bins;            // B = ceil((n - lds_window) / 2^bin_shift)
  int32_t bin_shift;       // log2 of the columns per bin
  int64_t pool_chunks;     // P: chunks in the pool (never exceeded: ceil(nnz / S) + grid * B)
  uint32_t* pool_next;     // chunks handed out (zeroed before launch)
  int2* pool;              // [P][kBinChunkItems] items {column, product bits}
  int32_t* chunk_bin;      // [P] bin of each handed-out chunk
  int32_t* chunk_fill;     // [P] items in each handed-out chunk
  // row-class kernel (csr_rows.hip): the analysis's nonempty rows grouped by class (index, and
  // entry bounds {s, e} per position) and its batches {first position, class * 256 + rows}, with
  // batch_prefix[k] = entries before batch k
  const int32_t* rows;
  const int32_t* bounds;        // [positions][2]
  const int32_t* batches;       // [batches_count][2]
  const int32_t* batch_prefix;  // [batches_count + 1]
  int32_t batches_count;
};

// Arguments of the bin passes (csr_bins.hip) that follow a binned fused launch.
struct CsrBinArgs {
  int64_t lds_window;
  int32_t bins, bin_shift;
  int64_t pool_chunks, max_units;
  const uint32_t* pool_next;
  const int2* pool;
  const int32_t* chunk_bin;
  const int32_t* chunk_fill;
  int32_t* order;          // [P] chunk ids grouped by bin
  int32_t* counts;         // [B][kBinSortGroups] chunks per bin and sorting workgroup, then their offsets
  int32_t* bin_start;      // [B + 1] first position in `order` of each bin
  int32_t* unit_start;     // [B + 1] first unit of each bin (unit_start[B] = units in all)
  float* partial2;         // [max_units][2^bin_shift] per-unit sums of the bin's columns
};

// Lets kernel `fn` take as dynamic LDS all of the device's LDS that its static LDS leaves. The
// attribute is set once per (device, kernel) for the process; later calls only look it up (api.cpp).
hipError_t allow_dynamic_lds(const void* fn);

// Kernel launchers (dense.hip, csr.hip, aggregate.hip). Each returns the first
// HIP error it meets.
hipError_t launch_dense(const DenseArgs& a, const xtvxy_launch_params& p, hipStream_t s);
// What a CSR launch computes: the whole pattern's partials, the first half alone (row values
// written to t_out; no window, no partials) or the second half alone (X^T u partials, u passed
// as v, no y).
enum CsrLaunchMode { kCsrFused = 0, kCsrRowdot = 1, kCsrTmv = 2 };
hipError_t launch_csr(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s, int mode = kCsrFused);
// The same launches by the wavefront kernel (plan kernel XTVXY_CSR_WAVES).
hipError_t launch_csr_waves(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s, int mode = kCsrFused);
// The row-class kernel (plan kernel XTVXY_CSR_ROWS; the fused pattern only).
hipError_t launch_csr_rows(const CsrArgs& a, const xtvxy_launch_params& p, hipStream_t s);
// Structure analysis kernels (csr_rows.hip): counts[col] += 1 for every stored entry (counts
// zeroed by the caller); out[p] = slot[col_idx[p]]; yp[s] = y[perm[s]].
hipError_t launch_col_count(const int32_t* col_idx, int64_t nnz, uint32_t* counts, hipStream_t s);
hipError_t launch_relabel(const int32_t* col_idx, int64_t nnz, const int32_t* slot, int32_t* out, hipStream_t s);
hipError_t launch_permute(const float* y, const int32_t* perm, int64_t n, float* yp, hipStream_t s);
// Bin passes: group the handed-out chunks by bin, then accumulate every unit of a bin in LDS.
hipError_t launch_csr_bins(const CsrBinArgs& a, hipStream_t s);
// Per-bin partial sums for the aggregation (null: no binning).
struct BinPartials {
  const float* partial2;
  const int32_t* unit_start;
  int64_t first_col;  // the first binned column (the LDS window)
  int32_t bin_shift;
};
// out[j] = alpha * (sum_{r < rows} partial[r * ldp + j] [j < ldp] + acc[j] [acc != null]
//                   + sum over the units u of j's bin of partial2[u][j - bin start] [binned j])
//          + (beta != 0 ? beta * z[j] : 0),
// in fp64, the partial rows summed in ascending order, rounded once.
// When `error` is given and the word it points to is nonzero when the kernel runs (a group-row
// wait gave up), every out[j] is NaN instead. With `out_perm` (columns relabelled by a CSR
// analysis) the sums are those of relabelled column j, and the result goes to
// out[out_perm[j]] with z[out_perm[j]].
hipError_t launch_aggregate(const float* partial, int64_t rows, int64_t ldp, const float* acc, int64_t n,
                            float alpha, float beta, const float* z, float* out, hipStream_t s,
                            const BinPartials* bins = nullptr, const uint32_t* error = nullptr,
                            const int32_t* out_perm = nullptr);
// out[j] = (beta != 0) ? beta * z[j] : 0
hipError_t launch_beta_only(int64_t n, float beta, const float* z, float* out, hipStream_t s);
// p[i] = 0 for i < count (a kernel, so that the call stays graph-capturable)
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
// t[i] *= v[i]
hipError_t launch_scale(int64_t m, const float* v, float* t, hipStream_t s);
hipError_t launch_csr_check(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr,
                            const int32_t* col_idx, int32_t* flag, hipStream_t s);

// Largest co-resident grid of the dense group-row kernel for a plan (0 on error).
int64_t dense_group_max_resident(const xtvxy_launch_params& p, int elem_bytes = 4);
// Workgroups of a dense plan's kernel that fit on one CU at once (registers, LDS); 0 if unknown.
int dense_resident_per_cu(const xtvxy_launch_params& p, int elem_bytes = 4);

// Analytical launch model (model.cpp).
xtvxy_status model_dense(int64_t m, int64_t n, int64_t ldx, bool aligned16, const xtvxy_device_info& d,
                         xtvxy_launch_params* p, int elem_bytes = 4, int max_wg_per_cu = 0);
xtvxy_status complete_dense(int64_t m, int64_t n, int64_t ldx, const xtvxy_device_info& d,
                            xtvxy_launch_params* p, int elem_bytes = 4);
// fused: the plan is for the whole pattern (the wavefront kernel is a candidate); else for one
// of its halves alone (workgroup tiles).
xtvxy_status model_csr(int64_t m, int64_t n, int64_t nnz, const xtvxy_device_info& d,
                       xtvxy_launch_params* p, bool fused = true);
xtvxy_status complete_csr(int64_t m, int64_t n, int64_t nnz, const xtvxy_device_info& d,
                          xtvxy_launch_params* p);
// The wavefront kernel's grid for a matrix whose longest row is known (a structure analysis, the
// solver's row scan): three 256-thread workgroups per CU when every row fits a tile and rows hold
// 8 or more entries on average, completed; false (plan unchanged) otherwise.
bool refine_waves_grid(int64_t m, int64_t n, int64_t nnz, int64_t longest_row, const xtvxy_device_info& d,
                       xtvxy_launch_params* p);

// Argument checks shared by the fused entry points and the comparator (api.cpp). On
// success *quick tells that only out = beta z (or nothing, when n == 0) remains to do.
xtvxy_status check_dense_args(int64_t m, int64_t n, float alpha, const void* X, int64_t ldx, const float* v,
                              const float* y, float beta, const float* z, const float* out, bool* quick, int elem_bytes = 4);
xtvxy_status check_csr_args(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                            const int32_t* col_idx, const float* values, const float* v, const float* y,
                            float beta, const float* z, const float* out, bool* quick, int value_bytes = 4);

// What an analysed CSR call adds to a fused CSR launch: the row-class work list (for the
// XTVXY_CSR_ROWS kernel) and the permutation of the relabelled output columns.
struct CsrExtras {
  const int32_t* rows;
  const int32_t* bounds;
  const int32_t* batches;
  const int32_t* batch_prefix;
  int32_t batches_count;
  const int32_t* out_perm;  // sums of relabelled column j go to out[out_perm[j]]
  int64_t binned_items;     // entries outside the plan's output window (sizes the bin pool), or -1
};
// The fused CSR path for checked arguments (api.cpp): the plan (`force`, completed here; the model's
// when null), the main kernel, the bin passes and the aggregation, on `stream`.
// Values are fp32 (value_bytes 4) or bf16 bit patterns (2).
xtvxy_status csr_run_fused(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                           const int32_t* col_idx, const void* values, const float* v, const float* y, float beta,
                           const float* z, float* out, void* ws, size_t ws_bytes, hipStream_t stream,
                           const xtvxy_launch_params* force, const CsrExtras* extras, int value_bytes = 4);
// The device description of the current device (cached).
xtvxy_status current_device_info(xtvxy_device_info* d);
// Records the measurement hook's events around a main kernel (api.cpp).
hipError_t mark_before_main(hipStream_t s);
hipError_t mark_after_main(hipStream_t s);

// Halves of the pattern through the rocSPARSE comparator's plan (unfused.cpp).
xtvxy_status unfused_rowdot(xtvxy_csr_unfused_plan p, const float* y, float* t, hipStream_t stream);
xtvxy_status unfused_tmv(xtvxy_csr_unfused_plan p, float alpha, const float* u, float beta, const float* z,
                         float* out, hipStream_t stream);
void unfused_plan_shape(xtvxy_csr_unfused_plan p, int64_t* m, int64_t* n, int64_t* nnz, const int32_t** row_ptr,
                        const int32_t** col_idx, const float** values);

// Newton-CG logistic-regression solver (logreg.hip kernels, logreg.cpp driver).
struct LrScalars {  // device-side scalars of the solver, in its workspace
  double f, gg, ww;        // objective, g.g and w.w at the current iterate
  double gs, ws, ss;       // g.s, w.s, s.s for the line search
  double df;               // f(w + a s) - f(w) at the last trial step
  double rr, kappa, alpha, beta;  // CG: r.r, d.Hd and the two step coefficients
  int32_t neg;             // CG met a direction of non-positive curvature (later iterations do nothing)
  int32_t done;            // CG's residual vanished exactly (later iterations do nothing)
  int32_t iters;           // CG iterations performed (the one that met neg included)
  uint32_t max_row;        // entries of the longest row (set once per solve by launch_lr_max_row)
};
constexpr int kLrMaxParts = 2048;     // partial sums per reduction row (workgroups of a streaming kernel)
constexpr int kLrRows = 4;            // reduction rows
constexpr int64_t kLrSmallCg = 16384; // n up to which one workgroup runs a whole CG update
enum LrFinish { kLrObjective = 0, kLrLine = 1, kLrTrial = 2, kLrCgAlpha = 3, kLrCgBeta = 4 };
// Workgroups of a streaming kernel over `count` elements (256 threads, at least 4 elements each).
inline int lr_grid(int64_t count) {
  if (count <= 0) return 0;
  const int64_t g = (count + 1023) / 1024;
  return (int)(g < kLrMaxParts ? g : kLrMaxParts);
}
// *longest = the largest row_ptr[i + 1] - row_ptr[i] (zeroed here, then an atomic maximum per wavefront).
hipError_t launch_lr_max_row(int64_t m, const int32_t* row_ptr, uint32_t* longest, hipStream_t s);
hipError_t launch_lr_link(int64_t m, float* t, const float* xs, float step, const float* c, float* u, float* v,
                          double* part, hipStream_t s);
hipError_t launch_lr_trial(int64_t m, const float* t, const float* xs, double a, const float* c, double* part,
                           hipStream_t s);
hipError_t launch_lr_dots(int64_t n, int k, const float* const* x, const float* const* y, int row0, double* part,
                          hipStream_t s);
hipError_t launch_lr_finish(int op, const double* part, int64_t m, int64_t n, LrScalars* S, double a, double lam,
                            hipStream_t s);
hipError_t launch_lr_cg_init(int64_t n, const float* g, float* z, float* r, float* d, LrScalars* S, hipStream_t s);
hipError_t launch_lr_cg_step(int64_t n, const float* q, float* d, float* z, float* r, LrScalars* S, bool first,
                             double* part, hipStream_t s);
hipError_t launch_lr_axpy(int64_t n, float a, const float* x, float* y, hipStream_t s);

// Workspace layout of a dense plan.
struct DenseWorkspace {
  size_t partial_off, partial_rows;  // partial sums [partial_rows][n]
  size_t xchg_off, error_off;  // group-row path only
  size_t total;
};
DenseWorkspace dense_workspace(int64_t n, const xtvxy_launch_params& p, int elem_bytes);

struct CsrWorkspace {
  size_t partial_off, partial_rows;  // [grid][lds_window]
  size_t acc_off;                    // [n] accumulator when lds_window < n and no binning
  // binning (bins > 0)
  int32_t bins, bin_shift;
  int64_t pool_chunks, max_units;
  size_t counter_off, pool_off, chunk_bin_off, chunk_fill_off, order_off, counts_off, bin_start_off,
      unit_start_off, partial2_off;
  size_t total;
};
// `binned` is the number of entries whose column lies outside the output window when known (a
// structure analysis counts them), negative when not: every entry is then assumed binned.
CsrWorkspace csr_workspace(int64_t m, int64_t n, int64_t nnz, const xtvxy_launch_params& p, int64_t binned = -1);

}  // namespace xtvxy
