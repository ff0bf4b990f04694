/*
 * xtvxy: fused evaluation of out = alpha * X^T (v .* (X y)) + beta * z on AMD gfx950.
 *
 * The operation is the generic pattern of "On optimizing machine learning
 * workloads via kernel fusion" (abstract): alpha * X^T (v * (X * y)) + beta * z,
 * computed by one fused kernel over dense or sparse X instead of a chain of
 * operator-level library calls. Shapes (the only well-typed reading):
 *     X  m x n,  y, z, out  n-vectors,  v  m-vector,  alpha, beta  scalars,
 *     X y is the matrix-vector product, v .* (X y) the elementwise product.
 * Special cases follow BLAS: n == 0 is a no-op; alpha == 0 or m == 0 (or
 * nnz == 0) gives out = beta * z without reading X, v or y; beta == 0 gives
 * out = alpha * X^T(...) without reading z (z may then be NULL). v == NULL
 * means v = 1 (the normal-equations instance X^T X y). Rows with v_i == 0 are
 * not skipped: NaN and Inf propagate as the formula says.
 *
 * Conventions of every entry point:
 *   - All array pointers are DEVICE pointers on the current HIP device; the
 *     caller owns every buffer. The library keeps no pointer after a call returns
 *     and the fused entry points allocate no device memory: partial results live
 *     in the caller's workspace (size from the *_workspace_size query).
 *   - Calls are asynchronous on `stream` (0 = the null stream). The inputs and
 *     the workspace must stay valid and unmodified until the stream passes the
 *     call. Concurrent calls need distinct workspaces.
 *   - The return value is the only error channel. Argument errors are detected
 *     on the host before anything is enqueued and leave `out` untouched.
 *     XTVXY_ERROR_LAUNCH reports a HIP error from an enqueue (possibly after an
 *     earlier kernel of the same call was enqueued).
 *   - fp32 storage and arithmetic; cross-workgroup sums of partial results are
 *     taken in fp64 in a fixed order, so dense results are bitwise reproducible
 *     for a given device and launch plan. The CSR path accumulates with LDS and
 *     global atomics and is reproducible only up to rounding.
 */
#ifndef XTVXY_H_
#define XTVXY_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define XTVXY_VERSION_MAJOR 0
#define XTVXY_VERSION_MINOR 1

typedef enum xtvxy_status {
  XTVXY_SUCCESS = 0,
  XTVXY_ERROR_INVALID_VALUE = 1, /* negative size, ldx < max(1, n), byte size overflow, bad plan field */
  XTVXY_ERROR_NULL_POINTER = 2,  /* a required pointer is NULL (see each entry point) */
  XTVXY_ERROR_ALIASING = 3,      /* out overlaps an input other than z (out == z is allowed) */
  XTVXY_ERROR_WORKSPACE = 4,     /* workspace NULL or smaller than the query returned */
  XTVXY_ERROR_UNSUPPORTED = 5,   /* beyond int32 indexing: CSR nnz or n above 2^31 - 1, m above 2^31 - 1025;
                                    the comparator: m, n or ldx above 2^31 - 1 */
  XTVXY_ERROR_LAUNCH = 6,        /* a HIP call failed (no device, launch failure, ...) */
  XTVXY_ERROR_LIBRARY = 7        /* rocBLAS / rocSPARSE failed (comparator entry points only) */
} xtvxy_status;

/* Human-readable name of a status code (static storage). */
const char *xtvxy_status_string(xtvxy_status status);

/* ------------------------------------------------------------------------ */
/* Device description and launch plans                                     */
/* ------------------------------------------------------------------------ */

/* The GPU resources the launch model reads (the pages' model maps input
 * characteristics and available GPU resources to launch parameters). */
typedef struct xtvxy_device_info {
  int32_t compute_units;     /* CUs (256 on MI355X) */
  int32_t lds_bytes;         /* LDS bytes one workgroup may allocate (163840) */
  int32_t l2_bytes;          /* L2 bytes of one XCD (4 MiB) */
  int32_t xcds;              /* XCDs sharing the grid (8) */
  double hbm_bytes_per_s;    /* peak HBM bandwidth (8.0e12) */
} xtvxy_device_info;

/* Resources of HIP device `device` (-1 = current device). */
xtvxy_status xtvxy_get_device_info(int device, xtvxy_device_info *info);

/* Dense kernel variants. */
enum {
  XTVXY_DENSE_WAVE_ROWS = 1,  /* rows of <= 1024 columns: lane groups within a wavefront own a row */
  XTVXY_DENSE_BLOCK_ROWS = 2, /* rows of <= 8192 columns: one workgroup owns a row */
  XTVXY_DENSE_GROUP_ROWS = 3  /* wider rows: `group` workgroups split a row by columns */
};
/* CSR kernel: tiles of whole rows; output columns [0, lds_window) accumulate in
 * LDS. The other ("cold") columns either go to a global fp32 accumulator with
 * hardware float atomics (bin_columns == 0), or are binned: the fused kernel
 * appends each cold product to workspace chunks of its bin of bin_columns
 * columns, and a second pass accumulates every bin in LDS (bin_columns > 0). */
enum {
  XTVXY_CSR_TILES = 11,
  /* the same scatter (LDS window, then atomics or bins), but every wavefront walks
   * tiles of whole rows of its own (at most 64 rows and 512 entries), so the
   * workgroup never waits at a barrier per tile; block_threads 256, 512 or 1024,
   * entries_per_thread 8 */
  XTVXY_CSR_WAVES = 12,
  /* rows by length class (needs a structure analysis, xtvxy_csr_f32_analyse; forced plans only,
   * the model never picks it): a group of 2^c lanes takes each row of class c (rows of up to
   * 8 * 2^c - 3 entries) with 8 entry slots per lane, a wavefront takes each row longer than 509
   * entries in slices of 512; every wavefront works alone, the scatter is the others' (LDS window,
   * then atomics or bins); block_threads 256, 512 or 1024, entries_per_thread 8 */
  XTVXY_CSR_ROWS = 13
};

/* Launch parameters chosen by the analytical model (the *_plan queries) or
 * forced by the caller (the *_ex entry points). */
typedef struct xtvxy_launch_params {
  int32_t kernel;          /* one of the XTVXY_DENSE_* / XTVXY_CSR_* values above */
  int32_t vec;             /* 4: 16-byte loads of X (needs ldx % 4 == 0 and 16-byte aligned X), 1: 4-byte */
  int32_t block_threads;   /* threads per workgroup (256) */
  int32_t lanes_per_row;   /* dense wave path: lanes sharing one row (1..64, power of two) */
  int32_t chunks;          /* dense: column chunks of `vec` floats per lane and row */
  int32_t group;           /* dense group path: workgroups per row (column slices); 1 otherwise */
  int64_t grid;            /* workgroups launched */
  int64_t rows_per_unit;   /* dense: rows per workgroup (wave/block paths) or per group */
  int32_t entries_per_thread; /* csr: nonzeros each thread holds per tile (4 or 8; 8 for the wavefront and
                                 row-class kernels) */
  int32_t lds_window;      /* csr: output columns [0, lds_window) accumulated in LDS (0..n) */
  int32_t y_window;        /* csr: y[0, y_window) is copied into each workgroup's LDS and gathered from
                              there, columns >= y_window from global memory (0..n) */
  int32_t bin_columns;     /* csr: 0 = cold columns by global atomics; else columns per bin (power of
                              two, 1024..32768; at most 512 bins, i.e. n - lds_window <= 512 bin_columns) */
  int64_t workspace_bytes; /* workspace the plan needs (filled in by the plan queries); with binning it
                              grows with nnz: about 8 bytes per stored entry plus per-bin partial sums
                              (analysed calls: 8 bytes per entry outside the output window) */
  double predicted_seconds;/* the model's estimate for this plan */
} xtvxy_launch_params;

/* Model-chosen plan for a dense problem; `dev` NULL = the current device.
 * X_aligned16 states whether X is 16-byte aligned (pointer % 16 == 0): the plan
 * depends on it (16-byte loads need an aligned X) and on the device's resources,
 * which `dev` may describe so that plans can be made without a GPU. */
xtvxy_status xtvxy_dense_f32_plan(int64_t m, int64_t n, int64_t ldx, int X_aligned16,
                                  const xtvxy_device_info *dev, xtvxy_launch_params *plan);

/* Model-chosen plan for a CSR problem; `dev` NULL = the current device. */
xtvxy_status xtvxy_csr_f32_plan(int64_t m, int64_t n, int64_t nnz, const xtvxy_device_info *dev,
                                xtvxy_launch_params *plan);

/* The same plan for a caller who knows the matrix's longest row (entries): the launch parameters
 * follow the input's characteristics ("On optimizing machine learning workloads via kernel
 * fusion", abstract), and the row lengths are one the shape does not give. When the model takes
 * the wavefront kernel (XTVXY_CSR_WAVES, 256 threads), every row fits its 512-slot tiles
 * (longest_row + 3 <= 512) and rows hold 8 or more entries on average, the plan runs three
 * workgroups per CU instead of the model's four (full tiles need fewer wavefronts to hide their
 * latency); otherwise it is xtvxy_csr_f32_plan's. Completed (workspace_bytes filled in); pass it
 * to xtvxy_csr_f32_ex. XTVXY_ERROR_INVALID_VALUE when longest_row is negative or above nnz. The
 * structure analysis and the Newton-CG solver apply the same rule. */
xtvxy_status xtvxy_csr_f32_plan_rows(int64_t m, int64_t n, int64_t nnz, int64_t longest_row,
                                     const xtvxy_device_info *dev, xtvxy_launch_params *plan);

/* ------------------------------------------------------------------------ */
/* Fused entry points                                                       */
/* ------------------------------------------------------------------------ */

/* Workspace bytes xtvxy_dense_f32 needs for this shape on the current device
 * (assuming a 16-byte aligned X; an unaligned X never needs more). */
xtvxy_status xtvxy_dense_f32_workspace_size(int64_t m, int64_t n, int64_t ldx, size_t *bytes);

/* out = alpha * X^T (v .* (X y)) + beta * z for dense row-major X: element
 * (i, k) at X[i * ldx + k], ldx >= max(1, n), at least (m-1)*ldx + n floats.
 * Pointers: y and out required when n > 0; X required when alpha != 0, m > 0
 * and n > 0; v optional (NULL = 1); z required iff beta != 0; workspace may be
 * NULL iff the query returned 0. `out` may equal `z` but may not otherwise
 * overlap X, v, y or z. */
xtvxy_status xtvxy_dense_f32(int64_t m, int64_t n, float alpha, const float *X, int64_t ldx,
                             const float *v, const float *y, float beta, const float *z, float *out,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);
/* (Plans of the group-row kernel: its grid never exceeds what the device holds at once, and its
 * launches on one device run one after another whatever their streams (each waits for the
 * previous one; not under graph capture), so every member of a group gets a slot. If a member's
 * bounded wait for the others still gives up, every element of out is NaN; see
 * xtvxy_test_group_wait.) */

/* As xtvxy_dense_f32 with the launch parameters forced (NULL = model). The
 * workspace must hold force->workspace_bytes as returned by xtvxy_dense_f32_plan
 * after the caller's edits (call the plan query with the edited plan to refresh
 * it via xtvxy_dense_f32_plan_complete). */
xtvxy_status xtvxy_dense_f32_ex(int64_t m, int64_t n, float alpha, const float *X, int64_t ldx,
                                const float *v, const float *y, float beta, const float *z,
                                float *out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream, const xtvxy_launch_params *force);

/* Checks a caller-edited dense plan against the shape and fills in grid-derived
 * fields (rows_per_unit when 0, workspace_bytes). */
xtvxy_status xtvxy_dense_f32_plan_complete(int64_t m, int64_t n, int64_t ldx,
                                           const xtvxy_device_info *dev, xtvxy_launch_params *plan);

/* For callers that cannot allocate device memory or provide a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): xtvxy_dense_f32 with the same
 * arguments minus the workspace, which is instead a fixed array of the library in device memory
 * (xtvxy_dense_f32_noalloc_max_workspace bytes, 32 MiB, held by every device the library runs on
 * until the process ends; its address is looked up on the first call on each device). Calls no
 * allocating routine. Shapes whose workspace (xtvxy_dense_f32_workspace_size) exceeds the array
 * return XTVXY_ERROR_WORKSPACE before anything is enqueued; other errors as xtvxy_dense_f32, and
 * the same result bit for bit (same launch plan). All calls on one device share the array:
 * calls that overlap in time on one device (concurrent streams or threads) race and give
 * undefined results; calls ordered on one stream are safe (the array keeps the last call's
 * contents, and each call clears what must start at zero). */
xtvxy_status xtvxy_dense_f32_noalloc_max_workspace(size_t *bytes);
xtvxy_status xtvxy_dense_f32_noalloc(int64_t m, int64_t n, float alpha, const float *X, int64_t ldx,
                                     const float *v, const float *y, float beta, const float *z, float *out,
                                     hipStream_t stream);

/* Reduced-precision storage of dense X: the same pattern with X held as bf16 (bfloat16 bit
 * patterns, uint16_t; an element is the upper 16 bits of an fp32 and widens to it exactly).
 * v, y, z and out stay fp32 and every operation is fp32 as in xtvxy_dense_f32, so the result is
 * that of xtvxy_dense_f32 on the widened matrix up to rounding order; X takes half the bytes.
 * The pages describe the pattern in fp32 only ("On optimizing machine learning workloads via
 * kernel fusion", abstract); bf16 storage is this library's extension. Same arguments, rules and
 * error codes as the fp32 entry points; a plan's vec is 8 (16-byte loads of 8 elements: X 16-byte
 * aligned, ldx % 8 == 0 and n % 8 == 0) or 1, and block/group-row plans with vec 8 take at most 4
 * chunks. */
xtvxy_status xtvxy_dense_bf16_workspace_size(int64_t m, int64_t n, int64_t ldx, size_t *bytes);
xtvxy_status xtvxy_dense_bf16_plan(int64_t m, int64_t n, int64_t ldx, int X_aligned16, const xtvxy_device_info *dev,
                                   xtvxy_launch_params *plan);
xtvxy_status xtvxy_dense_bf16_plan_complete(int64_t m, int64_t n, int64_t ldx, const xtvxy_device_info *dev,
                                            xtvxy_launch_params *plan);
xtvxy_status xtvxy_dense_bf16(int64_t m, int64_t n, float alpha, const uint16_t *X, int64_t ldx, const float *v,
                              const float *y, float beta, const float *z, float *out, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);
xtvxy_status xtvxy_dense_bf16_ex(int64_t m, int64_t n, float alpha, const uint16_t *X, int64_t ldx, const float *v,
                                 const float *y, float beta, const float *z, float *out, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream, const xtvxy_launch_params *force);
/* The same with X held as IEEE fp16 (binary16 bit patterns, uint16_t; every fp16 value widens to
 * fp32 exactly, subnormals, infinities and NaN included): all arithmetic fp32, the result that of
 * xtvxy_dense_f32 on the widened matrix up to rounding order. Plans, workspace sizes and every rule
 * are those of the bf16 entry points (the same 2 bytes per element): use
 * xtvxy_dense_bf16_plan, _plan_complete and _workspace_size. */
xtvxy_status xtvxy_dense_f16(int64_t m, int64_t n, float alpha, const uint16_t *X, int64_t ldx, const float *v,
                             const float *y, float beta, const float *z, float *out, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);
xtvxy_status xtvxy_dense_f16_ex(int64_t m, int64_t n, float alpha, const uint16_t *X, int64_t ldx, const float *v,
                                const float *y, float beta, const float *z, float *out, void *workspace,
                                size_t workspace_bytes, hipStream_t stream, const xtvxy_launch_params *force);

/* Workspace bytes xtvxy_csr_f32 needs for this shape on the current device. */
xtvxy_status xtvxy_csr_f32_workspace_size(int64_t m, int64_t n, int64_t nnz, size_t *bytes);

/* The same pattern for CSR X: zero-based int32 row_ptr[m + 1] (row_ptr[0] == 0,
 * non-decreasing, row_ptr[m] == nnz), int32 col_idx[nnz] in [0, n), fp32
 * values[nnz]. Columns may be unsorted within a row; a column stored twice in
 * a row contributes twice; empty rows are allowed. A malformed structure is
 * undefined behaviour (check it with xtvxy_csr_check). Pointer rules as for the
 * dense entry point, with row_ptr, col_idx and values in place of X (col_idx
 * and values may be NULL when nnz == 0). */
xtvxy_status xtvxy_csr_f32(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                           const int32_t *col_idx, const float *values, const float *v,
                           const float *y, float beta, const float *z, float *out, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

xtvxy_status xtvxy_csr_f32_ex(int64_t m, int64_t n, int64_t nnz, float alpha,
                              const int32_t *row_ptr, const int32_t *col_idx, const float *values,
                              const float *v, const float *y, float beta, const float *z,
                              float *out, void *workspace, size_t workspace_bytes,
                              hipStream_t stream, const xtvxy_launch_params *force);

xtvxy_status xtvxy_csr_f32_plan_complete(int64_t m, int64_t n, int64_t nnz,
                                         const xtvxy_device_info *dev, xtvxy_launch_params *plan);

/* The CSR pattern with the values stored as bf16: reduced-precision storage of X (its values; the
 * structure stays int32), all arithmetic fp32 ("On optimizing machine learning workloads via
 * kernel fusion", abstract: the fused path reads X once, so its bytes set the time; a bf16 value
 * halves the 8 bytes of a stored entry's value and column to 6). values[nnz] are bf16 bit
 * patterns (the upper 16 bits of an fp32, widened exactly as they are loaded), so the result is
 * that of xtvxy_csr_f32 on the widened values, up to the order of fp32 additions. Everything else
 * as xtvxy_csr_f32: the same plans, the same workspace (xtvxy_csr_f32_workspace_size), the same
 * conventions, pointer, aliasing (out against 2 nnz bytes of values) and error rules; vector loads
 * when col_idx is 16-byte and values 8-byte aligned. The tile and wavefront kernels take bf16
 * values; a forced XTVXY_CSR_ROWS plan gives XTVXY_ERROR_INVALID_VALUE. */
xtvxy_status xtvxy_csr_bf16(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                            const int32_t *col_idx, const uint16_t *values, const float *v, const float *y,
                            float beta, const float *z, float *out, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);
xtvxy_status xtvxy_csr_bf16_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                               const int32_t *col_idx, const uint16_t *values, const float *v, const float *y,
                               float beta, const float *z, float *out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream, const xtvxy_launch_params *force);

/* Structure analysis of a CSR matrix, made once and used by any number of calls whose values
 * change ("On optimizing machine learning workloads via kernel fusion", abstract: the launch
 * parameters come from the input's characteristics; here they are read from the structure):
 *   - the columns are relabelled by how many entries they hold, most first (ties by column), so
 *     that the output and y windows kept in LDS hold the hottest columns whatever their indices;
 *     the analysis keeps the relabelled column indices (4 nnz bytes of device memory) and the
 *     permutation (4 n bytes); each call gathers y into that order (n floats of its workspace)
 *     and writes every output column back to its own index, so results are those of
 *     xtvxy_csr_f32 on the caller's matrix (up to the order of fp32 additions);
 *   - the nonempty rows are grouped by length class for the row-class kernel (XTVXY_CSR_ROWS: the
 *     rows with their entry bounds, 12 bytes per nonempty row, in batches of one class);
 *   - the model's plan for the relabelled matrix (the tiled or wavefront kernel; its windows
 *     [0, W) and [0, Wy) now hold the most frequent columns), and the number of entries outside
 *     any output window, so the bin pool of each call holds exactly the binned entries.
 * xtvxy_csr_f32_analyse is a set-up call: it allocates device memory, synchronises `stream` and
 * reads back row_ptr and the column counts. It keeps row_ptr and values pointers of no call:
 * row_ptr (device) must stay valid and unchanged while the analysis is used (each call reads it);
 * col_idx is read only here. The same CSR conventions and errors as xtvxy_csr_f32 (a malformed
 * structure is undefined behaviour). A matrix with no rows, columns or entries gives an analysis
 * whose calls compute out = beta * z. Destroy it before freeing row_ptr; not thread-safe per
 * analysis; used on the device current when it was made (XTVXY_ERROR_INVALID_VALUE otherwise). */
typedef struct xtvxy_csr_analysis_s *xtvxy_csr_analysis;
xtvxy_status xtvxy_csr_f32_analyse(int64_t m, int64_t n, int64_t nnz, const int32_t *row_ptr,
                                   const int32_t *col_idx, hipStream_t stream, xtvxy_csr_analysis *analysis);
xtvxy_status xtvxy_csr_f32_analysis_destroy(xtvxy_csr_analysis analysis);
/* The model's plan for the analysed matrix (workspace_bytes included). */
xtvxy_status xtvxy_csr_f32_analysed_plan(xtvxy_csr_analysis analysis, xtvxy_launch_params *plan);
/* Checks a caller-edited plan for the analysed matrix and fills in its workspace_bytes. Any CSR
 * kernel on the relabelled columns: XTVXY_CSR_TILES or XTVXY_CSR_WAVES (the model's choices), or
 * XTVXY_CSR_ROWS (forced plans only). */
xtvxy_status xtvxy_csr_f32_analysed_plan_complete(xtvxy_csr_analysis analysis, xtvxy_launch_params *plan);
/* Workspace bytes of xtvxy_csr_f32_analysed (the model's plan). */
xtvxy_status xtvxy_csr_f32_analysed_workspace_size(xtvxy_csr_analysis analysis, size_t *bytes);
/* out = alpha * X^T (v .* (X y)) + beta * z for the analysed matrix with these values (nnz fp32 in
 * the caller's storage order). Pointer rules, aliasing rules (out against values, v, y and row_ptr;
 * out == z allowed) and errors as xtvxy_csr_f32; the workspace is the caller's. Asynchronous on
 * `stream`. The _ex form takes a plan completed by xtvxy_csr_f32_analysed_plan_complete. */
xtvxy_status xtvxy_csr_f32_analysed(xtvxy_csr_analysis analysis, float alpha, const float *values, const float *v,
                                    const float *y, float beta, const float *z, float *out, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);
xtvxy_status xtvxy_csr_f32_analysed_ex(xtvxy_csr_analysis analysis, float alpha, const float *values,
                                       const float *v, const float *y, float beta, const float *z, float *out,
                                       void *workspace, size_t workspace_bytes, hipStream_t stream,
                                       const xtvxy_launch_params *force);
/* The analysed call with bf16 values (nnz bf16 bit patterns in the caller's storage order), as
 * xtvxy_csr_bf16 is to xtvxy_csr_f32: same analysis, plans and workspace as the fp32 call; a forced
 * XTVXY_CSR_ROWS plan gives XTVXY_ERROR_INVALID_VALUE. */
xtvxy_status xtvxy_csr_bf16_analysed(xtvxy_csr_analysis analysis, float alpha, const uint16_t *values,
                                     const float *v, const float *y, float beta, const float *z, float *out,
                                     void *workspace, size_t workspace_bytes, hipStream_t stream);
xtvxy_status xtvxy_csr_bf16_analysed_ex(xtvxy_csr_analysis analysis, float alpha, const uint16_t *values,
                                        const float *v, const float *y, float beta, const float *z, float *out,
                                        void *workspace, size_t workspace_bytes, hipStream_t stream,
                                        const xtvxy_launch_params *force);

/* The two halves of the pattern on their own, for CSR X ("On optimizing machine learning
 * workloads via kernel fusion", abstract: the pattern chains X y and X^T (.); iterative solvers
 * such as Newton-CG for logistic regression also need each product by itself: the margins X w
 * and the gradient X^T r):
 *   xtvxy_csr_f32_rowdot:  t = alpha * v .* (X y) + beta * t0     (m-vector, one kernel)
 *   xtvxy_csr_f32_tmv:     out = alpha * X^T u + beta * z          (n-vector)
 * Same CSR conventions, limits and error codes as xtvxy_csr_f32. rowdot: v optional (NULL = 1);
 * t0 read only when beta != 0 and may equal t (in place); y, v and t0 read only when alpha != 0;
 * no workspace. tmv: u required when alpha != 0 and m, nnz > 0; z read only when beta != 0 and
 * may equal out; the workspace of xtvxy_csr_f32_workspace_size(m, n, nnz) suffices (with _ex:
 * force->workspace_bytes after xtvxy_csr_f32_plan_complete). The _ex forms take a launch plan
 * (entries_per_thread must be 8; rowdot ignores lds_window and bin_columns, tmv y_window; either
 * CSR kernel; without a plan the workgroup-tile kernel runs). Asynchronous on `stream`. */
xtvxy_status xtvxy_csr_f32_rowdot(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                                  const int32_t *col_idx, const float *values, const float *v, const float *y,
                                  float beta, const float *t0, float *t, hipStream_t stream);
xtvxy_status xtvxy_csr_f32_rowdot_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                                     const int32_t *col_idx, const float *values, const float *v, const float *y,
                                     float beta, const float *t0, float *t, hipStream_t stream,
                                     const xtvxy_launch_params *force);
xtvxy_status xtvxy_csr_f32_tmv(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                               const int32_t *col_idx, const float *values, const float *u, float beta,
                               const float *z, float *out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);
xtvxy_status xtvxy_csr_f32_tmv_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                                  const int32_t *col_idx, const float *values, const float *u, float beta,
                                  const float *z, float *out, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream, const xtvxy_launch_params *force);
/* The two halves with the values stored as bf16 (as xtvxy_csr_bf16 is to xtvxy_csr_f32): the same
 * rules, plans and workspace as the fp32 halves; values[nnz] are bf16 bit patterns widened exactly
 * as they are loaded. */
xtvxy_status xtvxy_csr_bf16_rowdot(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                                   const int32_t *col_idx, const uint16_t *values, const float *v, const float *y,
                                   float beta, const float *t0, float *t, hipStream_t stream);
xtvxy_status xtvxy_csr_bf16_rowdot_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                                      const int32_t *col_idx, const uint16_t *values, const float *v, const float *y,
                                      float beta, const float *t0, float *t, hipStream_t stream,
                                      const xtvxy_launch_params *force);
xtvxy_status xtvxy_csr_bf16_tmv(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                                const int32_t *col_idx, const uint16_t *values, const float *u, float beta,
                                const float *z, float *out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);
xtvxy_status xtvxy_csr_bf16_tmv_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                                   const int32_t *col_idx, const uint16_t *values, const float *u, float beta,
                                   const float *z, float *out, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream, const xtvxy_launch_params *force);

/* Device-side structure check of a CSR matrix. Writes to *d_flag (a device
 * int32) 0 when row_ptr[0] == 0, row_ptr is non-decreasing, row_ptr[m] == nnz
 * and every column index lies in [0, n); otherwise a positive code (1: row_ptr
 * ends, 2: row_ptr decreases, 3: column out of range). Asynchronous. */
xtvxy_status xtvxy_csr_check(int64_t m, int64_t n, int64_t nnz, const int32_t *row_ptr,
                             const int32_t *col_idx, int32_t *d_flag, hipStream_t stream);

/* Timing hook for measurements, per calling thread. While both events are
 * non-NULL, every fused call made by the thread that set them records
 * `before_main` on its stream just before its main fused kernel and
 * `after_main` just after it (before the aggregation kernel), so that
 * hipEventElapsedTime gives that kernel's time; calls from other threads are
 * not bracketed. NULL, NULL switches the hook off for the thread. The events
 * are the caller's. */
xtvxy_status xtvxy_set_kernel_timing_events(hipEvent_t before_main, hipEvent_t after_main);

/* Test hook of the dense group-row kernel's failure path, per calling thread. The members of a
 * group (XTVXY_DENSE_GROUP_ROWS) wait for each other's partial dot products with a bounded wait;
 * when a wait gives up (which does not happen in normal operation), the call
 * completes and every element of `out` is NaN. With `polls` > 0 each wait gives up after that
 * many polls; with `unanswered` nonzero the waits look for a step tag no member publishes, so
 * every wait gives up and the result must be all NaN (0, 0 restores normal operation). For tests
 * of that path only; XTVXY_ERROR_INVALID_VALUE for polls < 0. */
xtvxy_status xtvxy_test_group_wait(int32_t polls, int32_t unanswered);

/* Measurement helper, not part of the pattern: one kernel that reads `bytes` (a multiple of 16)
 * from the 16-byte aligned device buffer with 16-byte non-temporal loads over `grid` workgroups
 * of 256 threads, each taking one contiguous stretch, and writes nothing (the device float
 * `sink` is written only if the data sum to a value a zeroed buffer never gives). Its time gives
 * the GPU's streaming-read ceiling, the practical bound of the HBM-bound fused kernels.
 * Asynchronous on `stream`. */
xtvxy_status xtvxy_read_probe(const void *buffer, size_t bytes, int64_t grid, float *sink, hipStream_t stream);

/* Measurement helper, not part of the pattern: the access pattern of the wavefront CSR kernel
 * alone. Reads `entries` 4-byte elements from each of the two 16-byte aligned device arrays
 * (column indices and values in the kernel) over `grid` workgroups of 4 wavefronts, in tiles of
 * 512 entries per wavefront (8 per lane, two 16-byte loads per array), the next tile requested
 * before the current one is used; with `interleave` 0 each wavefront reads one contiguous
 * stretch (the kernel's layout), with 1 the 4 wavefronts of a workgroup take alternate tiles of
 * the workgroup's stretch. `entries` must be a positive multiple of grid * 2048
 * (XTVXY_ERROR_INVALID_VALUE otherwise). Writes nothing but `sink` (only for data a zeroed pair of
 * arrays never holds). Asynchronous on `stream`. */
xtvxy_status xtvxy_tile_stream_probe(const void *indices, const void *values, int64_t entries, int64_t grid,
                                     int32_t interleave, float *sink, hipStream_t stream);

/* What xtvxy_scatter_probe measures. */
typedef enum {
  XTVXY_PROBE_ATOMIC_PER_XCD = 0, /* fp32 atomic add of 1 into the copy of the XCD the wavefront runs on
                                     (8 copies of n floats), workgroup scope */
  XTVXY_PROBE_ATOMIC_DEVICE = 1,  /* fp32 atomic add of 1 into one copy of n floats, device scope */
  XTVXY_PROBE_ITEM_STORES = 2,    /* an 8-byte store {k, 1} to item slot c of n slots */
  XTVXY_PROBE_GATHERS = 3         /* a 4-byte load of float c of n */
} xtvxy_probe_kind;

/* Measurement helper, not part of the pattern: the rates of the primitives a scatter of products
 * to columns outside an LDS window could use. "On optimizing machine learning workloads via
 * kernel fusion" (abstract) aggregates partial results hierarchically; for the columns outside
 * the window the library bins products instead of adding them with global atomics, and this
 * probe measures that choice. One kernel of `grid` workgroups of 256 threads performs `items`
 * updates of kind `kind`; update k targets column c = hash(k) mod n (skew 0), or n u^3 with u a
 * uniform of the hash (skew 1: a quarter of the updates on the first 1.6% of the columns).
 * `buffer` (16-byte aligned device memory of `bytes` bytes) must hold 8 n floats for
 * XTVXY_PROBE_ATOMIC_PER_XCD, n 8-byte items for XTVXY_PROBE_ITEM_STORES and n floats otherwise
 * (else XTVXY_ERROR_WORKSPACE); the atomics add to its contents, the stores overwrite it, the
 * gathers only read it (the device float `sink` is written only if the gathered values sum to a
 * value a zeroed buffer never gives). XTVXY_ERROR_INVALID_VALUE for an unknown kind, n == 0, a
 * skew other than 0 or 1 or grid outside [1, 2^31). Asynchronous on `stream`. */
xtvxy_status xtvxy_scatter_probe(int kind, void *buffer, size_t bytes, uint32_t n, uint32_t items, int skew,
                                 int64_t grid, float *sink, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Unfused comparator: the same result from operator-level library calls    */
/* (the pages' baseline of several library kernel launches)               */
/* ------------------------------------------------------------------------ */

/* Workspace bytes of the dense comparator: the m-vector t = X y. */
xtvxy_status xtvxy_dense_f32_unfused_reference_workspace_size(int64_t m, int64_t n, size_t *bytes);

/* rocBLAS sgemv (t = X y), an elementwise kernel (t = v .* t, skipped when v
 * is NULL), a copy of z into out when beta != 0 and out != z, and rocBLAS
 * sgemv (out = alpha X^T t + beta out). Same arguments and rules as
 * xtvxy_dense_f32. Not thread-safe (one rocBLAS handle per device). */
xtvxy_status xtvxy_dense_f32_unfused_reference(int64_t m, int64_t n, float alpha, const float *X,
                                               int64_t ldx, const float *v, const float *y,
                                               float beta, const float *z, float *out,
                                               void *workspace, size_t workspace_bytes,
                                               hipStream_t stream);

/* The stronger dense comparator. rocBLAS's sgemv without transpose on the column-major view of a
 * row-major X (the comparator's last step, X^T t) is slow when X has few columns and many rows
 * (about 55 GB/s at 10^6 x 256). Given a copy of X^T, both steps are transposed sgemvs, each
 * reading its matrix along its rows, as the CSR comparator's explicit-transpose plan does for
 * SpMV.
 *   xtvxy_dense_f32_transpose: Xt (n x m, row-major, leading dimension ldxt >= m) = X^T, by
 *     rocBLAS sgeam; a set-up call for the comparator, kept out of timed regions. X and Xt must
 *     not overlap (XTVXY_ERROR_ALIASING). XTVXY_ERROR_INVALID_VALUE for negative sizes,
 *     ldx < n or ldxt < m; XTVXY_ERROR_UNSUPPORTED beyond 2^31 - 1; nothing to do when m or n
 *     is 0. Asynchronous on `stream`.
 *   xtvxy_dense_f32_unfused_reference_explicit: the comparator above with X^T t computed from Xt
 *     (n x m, ldxt >= m, made from the same X; the caller keeps the two consistent). Otherwise
 *     the same arguments, rules and workspace as xtvxy_dense_f32_unfused_reference; Xt is read
 *     only when X is, and out must not overlap it. */
xtvxy_status xtvxy_dense_f32_transpose(int64_t m, int64_t n, const float *X, int64_t ldx, float *Xt, int64_t ldxt,
                                       hipStream_t stream);
xtvxy_status xtvxy_dense_f32_unfused_reference_explicit(int64_t m, int64_t n, float alpha, const float *X,
                                                        int64_t ldx, const float *Xt, int64_t ldxt, const float *v,
                                                        const float *y, float beta, const float *z, float *out,
                                                        void *workspace, size_t workspace_bytes,
                                                        hipStream_t stream);

/* The CSR comparator keeps rocSPARSE descriptors and the result of the
 * structure analysis in a plan, made once per matrix (blocking, allocates).
 * Unlike the dense comparator it does not take xtvxy_csr_f32's argument list
 * with a caller workspace: rocSPARSE's SpMV needs a structure analysis of the
 * matrix and an opaque buffer whose size and contents are rocSPARSE's, made
 * once per matrix, and a fair comparison keeps that set-up out of the timed
 * calls (as the fused path needs no set-up at all). So the plan owns those
 * buffers (there is no separate workspace query), the per-call entry point
 * takes the plan in place of the matrix arrays, and the other arguments
 * (alpha, v, y, beta, z, out, stream) keep xtvxy_csr_f32's meaning and rules. */
typedef struct xtvxy_csr_unfused_plan_s *xtvxy_csr_unfused_plan;

xtvxy_status xtvxy_csr_f32_unfused_plan_create(int64_t m, int64_t n, int64_t nnz,
                                               const int32_t *row_ptr, const int32_t *col_idx,
                                               const float *values, hipStream_t stream,
                                               xtvxy_csr_unfused_plan *plan);
xtvxy_status xtvxy_csr_f32_unfused_plan_destroy(xtvxy_csr_unfused_plan plan);

/* Plan options. XTVXY_UNFUSED_TRANSPOSE_OP: X^T t is rocSPARSE's SpMV with the transpose
 * operation on X (the plain operator-level chain). XTVXY_UNFUSED_EXPLICIT_TRANSPOSE: the plan
 * also builds X^T as a second CSR matrix once (rocSPARSE csr2csc; 8 nnz + 4 (n + 1) more bytes
 * of device memory, made at plan creation, blocking) and X^T t becomes a forward SpMV with it:
 * the stronger comparator wherever the library's transposed SpMV is slow (it serialises on
 * shared output columns). The plan must be destroyed before X's buffers are freed; the copy
 * holds X's values as of plan creation. */
enum { XTVXY_UNFUSED_TRANSPOSE_OP = 0, XTVXY_UNFUSED_EXPLICIT_TRANSPOSE = 1 };
xtvxy_status xtvxy_csr_f32_unfused_plan_create_ex(int64_t m, int64_t n, int64_t nnz, const int32_t *row_ptr,
                                                  const int32_t *col_idx, const float *values, int32_t options,
                                                  hipStream_t stream, xtvxy_csr_unfused_plan *plan);

/* rocSPARSE SpMV (t = X y), the elementwise kernel, and rocSPARSE SpMV with
 * the transposed matrix (out = alpha X^T t + beta out; with the explicit
 * transpose, a forward SpMV with the plan's X^T). Uses the plan's buffers;
 * not thread-safe per plan. */
xtvxy_status xtvxy_csr_f32_unfused_reference(xtvxy_csr_unfused_plan plan, float alpha,
                                             const float *v, const float *y, float beta,
                                             const float *z, float *out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Empirical tuning beside the analytical model                            */
/* ------------------------------------------------------------------------ */

/* The pages' analytical model picks launch parameters from the input's characteristics and the
 * GPU's resources and calls the choice near-optimal ("On optimizing machine learning workloads via
 * kernel fusion", abstract). The tuner checks that on the actual input: it times the fused call
 * under every candidate plan the kernels accept for the shape (row layouts, chunks, group sizes and
 * grid sizes for dense X; tile shapes, output and y windows, atomics or bins and grid sizes for
 * CSR; the model's plan among them), re-times the fastest few with the model's plan, and reports
 * both. The model's regret is model_seconds / best_seconds - 1.
 *
 * A set-up call, not a fused entry point: it allocates its own workspace (the largest any
 * candidate needs, e.g. about 2 GB for binned plans of a 2e8-entry matrix), synchronises `stream`,
 * runs the full computation many times and leaves in `out` the result of the last call timed.
 * Arguments as for xtvxy_dense_f32 / xtvxy_csr_f32, plus `repeats` (1..10000) timed calls per
 * candidate (the finalists take 3x). A call whose only work is out = beta z has nothing to tune
 * and returns XTVXY_ERROR_INVALID_VALUE. Results are cached per (device, kind, m, n, ldx or nnz,
 * 16-byte alignment of X) for the life of the process; a cached shape returns at once with
 * from_cache = 1. Pass report.best to the _ex entry points to use the tuned plan (their
 * workspace is report.best.workspace_bytes). */
typedef struct xtvxy_tune_report {
  xtvxy_launch_params model;  /* the analytical model's plan */
  xtvxy_launch_params best;   /* the fastest plan measured */
  double model_seconds;       /* mean seconds per call with the model's plan (final round) */
  double best_seconds;        /* mean seconds per call with the best plan (final round) */
  int32_t candidates;         /* plans timed */
  int32_t from_cache;         /* 1: answered from the cache */
} xtvxy_tune_report;

xtvxy_status xtvxy_dense_f32_tune(int64_t m, int64_t n, float alpha, const float *X, int64_t ldx, const float *v,
                                  const float *y, float beta, const float *z, float *out, int32_t repeats,
                                  hipStream_t stream, xtvxy_tune_report *report);
xtvxy_status xtvxy_dense_bf16_tune(int64_t m, int64_t n, float alpha, const uint16_t *X, int64_t ldx,
                                   const float *v, const float *y, float beta, const float *z, float *out,
                                   int32_t repeats, hipStream_t stream, xtvxy_tune_report *report);
xtvxy_status xtvxy_csr_f32_tune(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                                const int32_t *col_idx, const float *values, const float *v, const float *y,
                                float beta, const float *z, float *out, int32_t repeats, hipStream_t stream,
                                xtvxy_tune_report *report);
/* The same for fp16 X (the candidates of bf16 X, timed with the fp16 kernels) and for bf16 CSR
 * values (the tile and wavefront candidates; the row-class kernel takes fp32 values only). */
xtvxy_status xtvxy_dense_f16_tune(int64_t m, int64_t n, float alpha, const uint16_t *X, int64_t ldx,
                                  const float *v, const float *y, float beta, const float *z, float *out,
                                  int32_t repeats, hipStream_t stream, xtvxy_tune_report *report);
xtvxy_status xtvxy_csr_bf16_tune(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t *row_ptr,
                                 const int32_t *col_idx, const uint16_t *values, const float *v, const float *y,
                                 float beta, const float *z, float *out, int32_t repeats, hipStream_t stream,
                                 xtvxy_tune_report *report);
/* Cache access: kind 0 = dense fp32 X, 2 = dense bf16 X and 3 = dense fp16 X (k = ldx, aligned =
 * X % 16 == 0), 1 = CSR with fp32 values and 4 = CSR with bf16 values (k = nnz, aligned = values
 * and col_idx 16-byte aligned); *found = 0 when the shape was not tuned on the current device.
 * save/load use a text file (one line per entry); load merges, and takes nothing from a file with
 * a malformed line (XTVXY_ERROR_INVALID_VALUE). Plans read from a file are checked again by the
 * _ex entry points that use them. */
xtvxy_status xtvxy_tune_cache_lookup(int32_t kind, int64_t m, int64_t n, int64_t k, int32_t aligned,
                                     xtvxy_tune_report *report, int32_t *found);
xtvxy_status xtvxy_tune_cache_clear(void);
xtvxy_status xtvxy_tune_cache_save(const char *path);
xtvxy_status xtvxy_tune_cache_load(const char *path);

/* ------------------------------------------------------------------------ */
/* An ML algorithm on the pattern: Newton-CG for logistic regression        */
/* ------------------------------------------------------------------------ */

/* "On optimizing machine learning workloads via kernel fusion" (abstract) finds the pattern
 * inside ML algorithms and closes with a whole algorithm run on the fused kernel; it names no
 * algorithm. This solver is the textbook one whose inner step is the pattern: L2-regularised
 * logistic regression,
 *     minimise f(w) = sum_i [log(1 + exp(t_i)) - c_i t_i] + (lambda / 2) |w|^2,   t = X w,
 * by line search Newton-CG (Nocedal and Wright, "Numerical Optimization", Algorithm 7.1, with
 * the backtracking of Algorithm 3.1). With p = sigmoid(t), the gradient is X^T (p - c) + lambda w
 * and every Hessian-vector product H d = X^T (p(1 - p) .* (X d)) + lambda d is the pattern with
 * alpha = 1, v = p(1 - p), y = z = d, beta = lambda.
 *
 * One Newton step k, all on `stream`:
 *   link     t += a_{k-1} X s_{k-1}; u = p - c; v = p(1 - p); loss terms (one m-length kernel)
 *   gradient g = X^T u + lambda w                        (the pattern's second half)
 *   stop     when |g_k| <= grad_tol |g_0|, or k == max_newton
 *   CG       s ~ -H^{-1} g: each iteration one Hessian-vector product and one vector-update
 *            kernel; stops at |r| < min(cg_forcing, sqrt|g_k|) |g_k| (unless fixed_cg), at
 *            max_cg iterations, or at a direction of non-positive curvature (then s = -g if
 *            that happens at once, else the current s)
 *   margins  X s                                         (the pattern's first half)
 *   step     a = 1, 1/2, 1/4, ... until f(w + a s) - f(w) <= 1e-4 a g.s, where the change of f
 *            is summed row by row in fp64 (one m-length kernel per trial); w += a s.
 * The host reads a few scalars back to take the decisions (one synchronisation per Newton
 * step, per line-search trial, and per CG iteration, or once per CG solve with fixed_cg, whose
 * stops on curvature or a vanished residual are taken on the device), so the call is
 * synchronous. Vectors are fp32; reductions (dot products, loss sums) are fp64 in a fixed
 * order.
 *
 * Engines: XTVXY_LOGREG_FUSED runs the three products with this library's kernels
 * (xtvxy_csr_f32, xtvxy_csr_f32_tmv, xtvxy_csr_f32_rowdot); XTVXY_LOGREG_UNFUSED runs them with
 * the rocSPARSE comparator of `unfused` (a plan made for the same matrix), everything else
 * being the same kernels, so the two differ only in how X is multiplied. */
enum { XTVXY_LOGREG_FUSED = 0, XTVXY_LOGREG_UNFUSED = 1 };
enum { XTVXY_LOGREG_CONVERGED = 0, XTVXY_LOGREG_ITERATION_LIMIT = 1, XTVXY_LOGREG_LINE_SEARCH_FAILED = 2 };

typedef struct xtvxy_logreg_options {
  float lambda;            /* L2 weight, finite and >= 0 */
  int32_t max_newton;      /* Newton steps, >= 0 */
  int32_t max_cg;          /* CG iterations per step, >= 1 */
  int32_t max_backtracks;  /* step lengths tried per step (1, 1/2, ...), >= 1 */
  double grad_tol;         /* stop at |g_k| <= grad_tol |g_0|; finite, >= 0 */
  double cg_forcing;       /* CG forcing cap, in (0, 1] (0.5 in the textbook) */
  int32_t fixed_cg;        /* nonzero: no early CG stop on the residual (fixed work per step) */
  int32_t engine;          /* XTVXY_LOGREG_FUSED or XTVXY_LOGREG_UNFUSED */
} xtvxy_logreg_options;

typedef struct xtvxy_logreg_report {
  int32_t status;              /* XTVXY_LOGREG_CONVERGED, _ITERATION_LIMIT or _LINE_SEARCH_FAILED */
  int32_t newton_iterations;   /* steps taken */
  int32_t cg_iterations;       /* Hessian-vector products, all steps */
  int32_t line_search_trials;  /* objective changes evaluated, all steps */
  double loss0, loss;          /* f at the start and at the returned w */
  double grad_norm0, grad_norm;/* |g| at the start and at the returned w */
  double seconds;              /* host wall time from the first enqueue to the last synchronisation */
} xtvxy_logreg_report;

/* Workspace bytes of xtvxy_logreg_newton_cg_f32 for this shape on the current device (4 m-vectors,
 * 5 n-vectors, reduction partials, and the workspace of xtvxy_csr_f32_workspace_size). */
xtvxy_status xtvxy_logreg_newton_cg_f32_workspace_size(int64_t m, int64_t n, int64_t nnz, size_t *bytes);

/* Runs the solver from the caller's w (device, n floats; overwritten with the result).
 * X is CSR as for xtvxy_csr_f32; labels (device, m floats) are the c_i, normally in {0, 1}
 * (any value in [0, 1] is a valid soft label). `unfused` must be a plan of the same m, n, nnz
 * and matrix pointers when opt->engine is XTVXY_LOGREG_UNFUSED and is ignored otherwise.
 * `report` (host) may be NULL. `history` (host, may be NULL) receives up to history_rows rows of
 * 6 doubles per iterate k = 0, 1, ...: f_k, |g_k|, CG iterations of step k, g_k.s_k, the accepted
 * step a_k, line-search trials of step k (the last four are NaN for the final iterate).
 * Returns argument errors before anything is enqueued; after a HIP or library error, w holds an
 * unspecified iterate. Not thread-safe for one workspace; the workspace and the inputs must stay
 * valid for the call (it synchronises `stream` before returning). */
xtvxy_status xtvxy_logreg_newton_cg_f32(int64_t m, int64_t n, int64_t nnz, const int32_t *row_ptr,
                                        const int32_t *col_idx, const float *values, const float *labels,
                                        float *w, const xtvxy_logreg_options *opt, xtvxy_csr_unfused_plan unfused,
                                        void *workspace, size_t workspace_bytes, hipStream_t stream,
                                        xtvxy_logreg_report *report, double *history, int64_t history_rows);

/* The same solver with X's values stored as bf16 bit patterns (nnz uint16_t, device), each
 * widened exactly to fp32 where it is read, as in xtvxy_csr_bf16; labels, w and every vector
 * and reduction are as above. Only the fused engine takes bf16 values: opt->engine must be
 * XTVXY_LOGREG_FUSED (else XTVXY_ERROR_INVALID_VALUE), and the workspace is the one of
 * xtvxy_logreg_newton_cg_f32_workspace_size. The products are xtvxy_csr_bf16, _bf16_tmv and
 * _bf16_rowdot; the iterates equal those of the fp32 solver run on the widened values, up to
 * the rounding of the products' sums. */
xtvxy_status xtvxy_logreg_newton_cg_bf16(int64_t m, int64_t n, int64_t nnz, const int32_t *row_ptr,
                                         const int32_t *col_idx, const uint16_t *values, const float *labels,
                                         float *w, const xtvxy_logreg_options *opt, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream, xtvxy_logreg_report *report,
                                         double *history, int64_t history_rows);

#ifdef __cplusplus
}
#endif

#endif /* XTVXY_H_ */
