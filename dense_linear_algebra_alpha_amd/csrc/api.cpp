// C ABI of the xtvxy library: argument checks, BLAS-style quick returns, launch
// plans and kernel dispatch for the fused entry points declared in xtvxy.h.
// Every argument error is detected here, on the host, before anything is
// enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <set>
#include <utility>

#include "internal.h"

using namespace xtvxy;

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_info_mutex;
bool g_info_valid[kMaxDevices];
xtvxy_device_info g_info[kMaxDevices];

xtvxy_status device_info(int device, xtvxy_device_info* out) {
  if (device < 0) {
    if (hipGetDevice(&device) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  }
  if (device >= kMaxDevices) return XTVXY_ERROR_INVALID_VALUE;
  std::lock_guard<std::mutex> lock(g_info_mutex);
  if (!g_info_valid[device]) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return XTVXY_ERROR_LAUNCH;
    xtvxy_device_info d{};
    d.compute_units = prop.multiProcessorCount;
    d.lds_bytes = (int32_t)prop.sharedMemPerBlock;
    d.l2_bytes = prop.l2CacheSize;
    // gfx94x/gfx95x parts group 32 (or 38/40) CUs per XCD; the count only steers tile placement
    d.xcds = prop.multiProcessorCount >= 64 ? prop.multiProcessorCount / 32 : 1;
    // memoryClockRate is in kHz; HBM3/HBM3E parts transfer 4 bits per pin per reported clock
    // (MI300X: 1.3 GHz x 4 x 1024 B = 5.3 TB/s; MI355X: 2.0 GHz x 4 x 1024 B = 8.2 TB/s)
    d.hbm_bytes_per_s = 4.0 * prop.memoryClockRate * 1e3 * (prop.memoryBusWidth / 8.0);
    if (d.hbm_bytes_per_s <= 0) d.hbm_bytes_per_s = 8.0e12;
    g_info[device] = d;
    g_info_valid[device] = true;
  }
  *out = g_info[device];
  return XTVXY_SUCCESS;
}

// [a, a + an) and [b, b + bn) (in bytes) overlap
bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

bool mul_overflows(int64_t a, int64_t b) { return a != 0 && b > INT64_MAX / a; }

xtvxy_status launch_status(hipError_t e) { return e == hipSuccess ? XTVXY_SUCCESS : XTVXY_ERROR_LAUNCH; }

// Measurement hook: events recorded around the main fused kernel of each call made by the thread
// that set them (per thread, so that calls from other threads are never bracketed by them).
thread_local hipEvent_t g_before_main = nullptr, g_after_main = nullptr;

// Failure-path test hook of the group-row kernel (per thread): polls per wait, and whether the
// waits look for a tag that no member publishes.
thread_local uint32_t g_wait_polls = 0, g_wait_unanswered = 0;

// (device, kernel) pairs whose dynamic-LDS limit has been raised to the device's LDS.
std::mutex g_lds_mutex;
std::set<std::pair<int, const void*>> g_lds_done;

hipError_t mark(hipEvent_t e, hipStream_t s) { return e ? hipEventRecord(e, s) : hipSuccess; }

// Checks shared by the dense fused entry point and its comparator. Returns SUCCESS with
// *quick set when nothing beyond out = beta z (or nothing at all) has to be computed.
xtvxy_status check_dense(int64_t m, int64_t n, float alpha, const void* X, int64_t ldx, const float* v,
                         const float* y, float beta, const float* z, const float* out, bool* quick,
                         int elem_bytes = 4) {
  *quick = false;
  if (m < 0 || n < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (ldx < (n > 1 ? n : 1)) return XTVXY_ERROR_INVALID_VALUE;
  if (mul_overflows(m, ldx) || m * ldx > INT64_MAX / 8) return XTVXY_ERROR_INVALID_VALUE;
  if (n == 0) {
    *quick = true;
    return XTVXY_SUCCESS;
  }
  if (!out || !y) return XTVXY_ERROR_NULL_POINTER;
  if (beta != 0.0f && !z) return XTVXY_ERROR_NULL_POINTER;
  const bool reads_x = alpha != 0.0f && m > 0;
  if (reads_x && !X) return XTVXY_ERROR_NULL_POINTER;
  const size_t nb = (size_t)n * sizeof(float);
  if (reads_x) {
    const size_t xb = ((size_t)(m - 1) * ldx + n) * (size_t)elem_bytes;
    if (overlap(out, nb, X, xb) || overlap(out, nb, y, nb) || (v && overlap(out, nb, v, (size_t)m * sizeof(float))))
      return XTVXY_ERROR_ALIASING;
  }
  if (beta != 0.0f && z != out && overlap(out, nb, z, nb)) return XTVXY_ERROR_ALIASING;
  if (!reads_x) *quick = true;
  return XTVXY_SUCCESS;
}

xtvxy_status check_csr(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                       const int32_t* col_idx, const void* values, const float* v, const float* y, float beta,
                       const float* z, const float* out, bool* quick, int value_bytes = 4) {
  *quick = false;
  if (m < 0 || n < 0 || nnz < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (nnz > INT32_MAX || m > INT32_MAX - 1024 || n > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  if (n == 0) {
    *quick = true;
    return XTVXY_SUCCESS;
  }
  if (!out || !y) return XTVXY_ERROR_NULL_POINTER;
  if (beta != 0.0f && !z) return XTVXY_ERROR_NULL_POINTER;
  const bool reads_x = alpha != 0.0f && m > 0 && nnz > 0;
  if (reads_x && (!row_ptr || !col_idx || !values)) return XTVXY_ERROR_NULL_POINTER;
  const size_t nb = (size_t)n * sizeof(float);
  if (reads_x) {
    if (overlap(out, nb, row_ptr, (size_t)(m + 1) * 4) || overlap(out, nb, col_idx, (size_t)nnz * 4) ||
        overlap(out, nb, values, (size_t)nnz * (size_t)value_bytes) || overlap(out, nb, y, nb) ||
        (v && overlap(out, nb, v, (size_t)m * sizeof(float))))
      return XTVXY_ERROR_ALIASING;
  }
  if (beta != 0.0f && z != out && overlap(out, nb, z, nb)) return XTVXY_ERROR_ALIASING;
  if (!reads_x) *quick = true;
  return XTVXY_SUCCESS;
}

xtvxy_status dense_plan_query(int64_t m, int64_t n, int64_t ldx, int X_aligned16, const xtvxy_device_info* dev,
                              xtvxy_launch_params* plan, int elem_bytes);

xtvxy_status dense_plan_for(int64_t m, int64_t n, int64_t ldx, bool aligned, const xtvxy_device_info& d,
                            const xtvxy_launch_params* force, xtvxy_launch_params* plan, int elem_bytes = 4) {
  if (force) {
    *plan = *force;
    xtvxy_status st = complete_dense(m, n, ldx, d, plan, elem_bytes);
    if (st != XTVXY_SUCCESS) return st;
    const int wide = 16 / elem_bytes;  // a 16-byte load per chunk needs an aligned X and ldx
    if (plan->vec == wide && (!aligned || ldx % wide != 0)) return XTVXY_ERROR_INVALID_VALUE;
    return XTVXY_SUCCESS;
  }
  return dense_plan_query(m, n, ldx, aligned ? 1 : 0, nullptr, plan, elem_bytes);
}

xtvxy_status csr_plan_for(int64_t m, int64_t n, int64_t nnz, const xtvxy_device_info& d,
                          const xtvxy_launch_params* force, xtvxy_launch_params* plan, bool fused) {
  if (force) {
    *plan = *force;
    return complete_csr(m, n, nnz, d, plan);
  }
  return model_csr(m, n, nnz, d, plan, fused);
}

// The group-row kernel's grid stays within what the device runs at once (whole groups), so
// that every member finds a slot while the others wait for it (its launches are also ordered
// per device). That limit is only known on the device: shrink the model's grid to it and
// recompute the coarsening; a forced grid beyond it is refused.
xtvxy_status fit_group_grid(int64_t m, int64_t n, int64_t ldx, const xtvxy_device_info& d,
                            xtvxy_launch_params* plan, bool forced, int elem_bytes = 4) {
  if (plan->kernel != XTVXY_DENSE_GROUP_ROWS) return XTVXY_SUCCESS;
  const int64_t cap = dense_group_max_resident(*plan, elem_bytes) / plan->group * plan->group;
  if (cap < plan->group) return XTVXY_ERROR_LAUNCH;
  if (plan->grid > cap) {
    if (forced) return XTVXY_ERROR_INVALID_VALUE;
    plan->grid = cap;
    plan->rows_per_unit = 0;
    return complete_dense(m, n, ldx, d, plan, elem_bytes);
  }
  return XTVXY_SUCCESS;
}

xtvxy_status dense_plan_query(int64_t m, int64_t n, int64_t ldx, int X_aligned16, const xtvxy_device_info* dev,
                              xtvxy_launch_params* plan, int elem_bytes) {
  if (!plan) return XTVXY_ERROR_NULL_POINTER;
  if (m < 0 || n < 0 || ldx < (n > 1 ? n : 1)) return XTVXY_ERROR_INVALID_VALUE;
  xtvxy_device_info d;
  if (dev) {
    d = *dev;
  } else {
    xtvxy_status st = device_info(-1, &d);
    if (st != XTVXY_SUCCESS) return st;
  }
  if (d.compute_units <= 0 || d.hbm_bytes_per_s <= 0) return XTVXY_ERROR_INVALID_VALUE;
  xtvxy_status st = model_dense(m, n, ldx, X_aligned16 != 0, d, plan, elem_bytes);
  if (st == XTVXY_SUCCESS && !dev) {
    // on the current device the kernel's residency is known: cap the workgroups per CU by it
    const int resident = dense_resident_per_cu(*plan, elem_bytes);
    int cap = 1;
    while (cap * 2 <= resident) cap *= 2;
    if (resident > 0 && plan->grid > (int64_t)d.compute_units * cap)
      st = model_dense(m, n, ldx, X_aligned16 != 0, d, plan, elem_bytes, cap);
    if (st == XTVXY_SUCCESS) st = fit_group_grid(m, n, ldx, d, plan, false, elem_bytes);
  }
  return st;
}

xtvxy_status dense_complete_query(int64_t m, int64_t n, int64_t ldx, const xtvxy_device_info* dev,
                                  xtvxy_launch_params* plan, int elem_bytes) {
  if (!plan) return XTVXY_ERROR_NULL_POINTER;
  if (m < 0 || n < 0 || ldx < (n > 1 ? n : 1)) return XTVXY_ERROR_INVALID_VALUE;
  xtvxy_device_info d;
  if (dev) {
    d = *dev;
  } else {
    xtvxy_status st = device_info(-1, &d);
    if (st != XTVXY_SUCCESS) return st;
  }
  return complete_dense(m, n, ldx, d, plan, elem_bytes);
}

xtvxy_status dense_workspace_query(int64_t m, int64_t n, int64_t ldx, size_t* bytes, int elem_bytes) {
  if (!bytes) return XTVXY_ERROR_NULL_POINTER;
  if (m < 0 || n < 0 || ldx < (n > 1 ? n : 1)) return XTVXY_ERROR_INVALID_VALUE;
  *bytes = 0;
  if (m == 0 || n == 0) return XTVXY_SUCCESS;
  // the larger of the two plans (X 16-byte aligned or not); a width that only an aligned X
  // supports (4-byte loads cover fewer columns per group) takes the aligned plan's size
  size_t best = 0;
  xtvxy_status first_error = XTVXY_SUCCESS;
  int planned = 0;
  for (int aligned = 0; aligned < 2; ++aligned) {
    xtvxy_launch_params p;
    xtvxy_status st = dense_plan_query(m, n, ldx, aligned, nullptr, &p, elem_bytes);
    if (st != XTVXY_SUCCESS) {
      if (first_error == XTVXY_SUCCESS) first_error = st;
      continue;
    }
    ++planned;
    if ((size_t)p.workspace_bytes > best) best = (size_t)p.workspace_bytes;
  }
  if (planned == 0) return first_error;
  *bytes = best;
  return XTVXY_SUCCESS;
}

xtvxy_status dense_impl(int64_t m, int64_t n, float alpha, const void* X, int64_t ldx, const float* v,
                        const float* y, float beta, const float* z, float* out, void* ws, size_t ws_bytes,
                        hipStream_t stream, const xtvxy_launch_params* force, int elem_bytes = 4,
                        bool f16 = false) {
  bool quick = false;
  xtvxy_status st = check_dense(m, n, alpha, X, ldx, v, y, beta, z, out, &quick, elem_bytes);
  if (st != XTVXY_SUCCESS) return st;
  if (quick) return n == 0 ? XTVXY_SUCCESS : launch_status(launch_beta_only(n, beta, z, out, stream));
  xtvxy_device_info d;
  st = device_info(-1, &d);
  if (st != XTVXY_SUCCESS) return st;
  const bool aligned = (reinterpret_cast<uintptr_t>(X) % 16) == 0;
  xtvxy_launch_params plan;
  st = dense_plan_for(m, n, ldx, aligned, d, force, &plan, elem_bytes);
  if (st != XTVXY_SUCCESS) return st;
  st = fit_group_grid(m, n, ldx, d, &plan, force != nullptr, elem_bytes);
  if (st != XTVXY_SUCCESS) return st;
  if (plan.workspace_bytes > 0 && (!ws || ws_bytes < (size_t)plan.workspace_bytes)) return XTVXY_ERROR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return XTVXY_ERROR_WORKSPACE;

  const DenseWorkspace w = dense_workspace(n, plan, elem_bytes);
  char* base = static_cast<char*>(ws);
  DenseArgs a{};
  a.m = m;
  a.n = n;
  a.ldx = ldx;
  a.X = X;
  a.elem_bytes = elem_bytes;
  a.f16 = f16 ? 1 : 0;
  a.v = v;
  a.y = y;
  a.partial = reinterpret_cast<float*>(base + w.partial_off);
  a.rows_per_unit = plan.rows_per_unit;
  a.lanes_per_row = plan.lanes_per_row;
  a.group = plan.group;
  if (plan.kernel == XTVXY_DENSE_GROUP_ROWS) {
    a.xchg = base + w.xchg_off;
    a.error = reinterpret_cast<uint32_t*>(base + w.error_off);
    a.wait_polls = g_wait_polls;
    a.wait_tag_skew = g_wait_unanswered ? 0x80000000u : 0u;
    hipError_t e = launch_zero(base + w.xchg_off, w.total - w.xchg_off, stream);
    if (e != hipSuccess) return XTVXY_ERROR_LAUNCH;
  }
  const hipEvent_t before = g_before_main, after = g_after_main;
  if (before && after && mark(before, stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  hipError_t e = launch_dense(a, plan, stream);
  if (e != hipSuccess) return XTVXY_ERROR_LAUNCH;
  if (before && after && mark(after, stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  e = launch_aggregate(a.partial, (int64_t)w.partial_rows, n, nullptr, n, alpha, beta, z, out, stream, nullptr,
                       plan.kernel == XTVXY_DENSE_GROUP_ROWS ? a.error : nullptr);
  return launch_status(e);
}

// The fused kernel (mode kCsrFused, with v and y) or its second half alone (kCsrTmv, with u
// passed as v and no y), then the bin passes and the aggregation, for checked arguments. Values
// are fp32 (value_bytes 4) or, for the fused pattern on the tile and wavefront kernels, bf16 (2).
xtvxy_status csr_run(int mode, int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                     const int32_t* col_idx, const void* values, const float* v, const float* y, float beta,
                     const float* z, float* out, void* ws, size_t ws_bytes, hipStream_t stream,
                     const xtvxy_launch_params* force, const CsrExtras* extras = nullptr, int value_bytes = 4) {
  if (value_bytes != 4 && value_bytes != 2) return XTVXY_ERROR_INVALID_VALUE;
  xtvxy_device_info d;
  xtvxy_status st = device_info(-1, &d);
  if (st != XTVXY_SUCCESS) return st;
  xtvxy_launch_params plan;
  st = csr_plan_for(m, n, nnz, d, force, &plan, mode == kCsrFused);
  if (st != XTVXY_SUCCESS) return st;
  // the row-class kernel runs on an analysis's work list, and on the whole pattern only
  if (plan.kernel == XTVXY_CSR_ROWS &&
      (extras == nullptr || extras->rows == nullptr || mode != kCsrFused || value_bytes != 4))
    return XTVXY_ERROR_INVALID_VALUE;
  if (mode == kCsrTmv && plan.entries_per_thread != 8) return XTVXY_ERROR_INVALID_VALUE;
  if (mode == kCsrTmv && plan.y_window != 0) {  // no y to gather: the plan with no y window
    plan.y_window = 0;
    st = complete_csr(m, n, nnz, d, &plan);
    if (st != XTVXY_SUCCESS) return st;
  }
  const CsrWorkspace w = csr_workspace(m, n, nnz, plan, extras ? extras->binned_items : -1);
  if (w.total > 0 && (!ws || ws_bytes < w.total)) return XTVXY_ERROR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return XTVXY_ERROR_WORKSPACE;
  CsrArgs a{};
  a.m = m;
  a.n = n;
  a.nnz = nnz;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.values = values;
  a.value_bytes = value_bytes;
  a.v = v;
  a.y = y;
  char* base = static_cast<char*>(ws);
  a.partial = reinterpret_cast<float*>(base + w.partial_off);
  a.lds_window = plan.lds_window;
  a.y_window = plan.y_window;
  const bool binned = w.bins > 0;
  a.acc = (plan.lds_window < n && !binned) ? reinterpret_cast<float*>(base + w.acc_off) : nullptr;
  // vector loads of 4 entries: 16 bytes of column indices and 4 * value_bytes of values
  a.aligned = reinterpret_cast<uintptr_t>(values) % (uintptr_t)(4 * value_bytes) == 0 &&
              reinterpret_cast<uintptr_t>(col_idx) % 16 == 0;
  if (extras) {
    a.rows = extras->rows;
    a.bounds = extras->bounds;
    a.batches = extras->batches;
    a.batch_prefix = extras->batch_prefix;
    a.batches_count = extras->batches_count;
  }
  CsrBinArgs bargs{};
  if (binned) {
    a.bins = w.bins;
    a.bin_shift = w.bin_shift;
    a.pool_chunks = w.pool_chunks;
    a.pool_next = reinterpret_cast<uint32_t*>(base + w.counter_off);
    a.pool = reinterpret_cast<int2*>(base + w.pool_off);
    a.chunk_bin = reinterpret_cast<int32_t*>(base + w.chunk_bin_off);
    a.chunk_fill = reinterpret_cast<int32_t*>(base + w.chunk_fill_off);
    bargs.lds_window = plan.lds_window;
    bargs.bins = w.bins;
    bargs.bin_shift = w.bin_shift;
    bargs.pool_chunks = w.pool_chunks;
    bargs.max_units = w.max_units;
    bargs.pool_next = a.pool_next;
    bargs.pool = a.pool;
    bargs.chunk_bin = a.chunk_bin;
    bargs.chunk_fill = a.chunk_fill;
    bargs.order = reinterpret_cast<int32_t*>(base + w.order_off);
    bargs.counts = reinterpret_cast<int32_t*>(base + w.counts_off);
    bargs.bin_start = reinterpret_cast<int32_t*>(base + w.bin_start_off);
    bargs.unit_start = reinterpret_cast<int32_t*>(base + w.unit_start_off);
    bargs.partial2 = reinterpret_cast<float*>(base + w.partial2_off);
  }
  hipError_t e;
  if (a.acc) {
    e = launch_zero(a.acc, (size_t)n * sizeof(float), stream);
    if (e != hipSuccess) return XTVXY_ERROR_LAUNCH;
  }
  if (binned) {
    e = launch_zero(a.pool_next, sizeof(uint32_t), stream);
    if (e != hipSuccess) return XTVXY_ERROR_LAUNCH;
  }
  const hipEvent_t before = g_before_main, after = g_after_main;
  if (before && after && mark(before, stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  e = plan.kernel == XTVXY_CSR_ROWS    ? launch_csr_rows(a, plan, stream)
      : plan.kernel == XTVXY_CSR_WAVES ? launch_csr_waves(a, plan, stream, mode)
                                       : launch_csr(a, plan, stream, mode);
  if (e != hipSuccess) return XTVXY_ERROR_LAUNCH;
  if (before && after && mark(after, stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  BinPartials bp{bargs.partial2, bargs.unit_start, plan.lds_window, w.bin_shift};
  if (binned) {
    e = launch_csr_bins(bargs, stream);
    if (e != hipSuccess) return XTVXY_ERROR_LAUNCH;
  }
  e = launch_aggregate(a.partial, (int64_t)w.partial_rows, plan.lds_window, a.acc, n, alpha, beta, z, out, stream,
                       binned ? &bp : nullptr, nullptr, extras ? extras->out_perm : nullptr);
  return launch_status(e);
}

xtvxy_status csr_impl(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                      const int32_t* col_idx, const void* values, const float* v, const float* y, float beta,
                      const float* z, float* out, void* ws, size_t ws_bytes, hipStream_t stream,
                      const xtvxy_launch_params* force, int value_bytes = 4) {
  bool quick = false;
  xtvxy_status st = check_csr(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, &quick, value_bytes);
  if (st != XTVXY_SUCCESS) return st;
  if (quick) return n == 0 ? XTVXY_SUCCESS : launch_status(launch_beta_only(n, beta, z, out, stream));
  return csr_run(kCsrFused, m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, ws, ws_bytes, stream,
                 force, nullptr, value_bytes);
}

// out = alpha X^T u + beta z (the second half of the pattern alone).
xtvxy_status tmv_impl(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                      const int32_t* col_idx, const void* values, const float* u, float beta, const float* z,
                      float* out, void* ws, size_t ws_bytes, hipStream_t stream, const xtvxy_launch_params* force,
                      int value_bytes = 4) {
  if (m < 0 || n < 0 || nnz < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (nnz > INT32_MAX || m > INT32_MAX - 1024 || n > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  if (n == 0) return XTVXY_SUCCESS;
  if (!out) return XTVXY_ERROR_NULL_POINTER;
  if (beta != 0.0f && !z) return XTVXY_ERROR_NULL_POINTER;
  const bool reads_x = alpha != 0.0f && m > 0 && nnz > 0;
  const size_t nb = (size_t)n * sizeof(float);
  if (reads_x) {
    if (!row_ptr || !col_idx || !values || !u) return XTVXY_ERROR_NULL_POINTER;
    if (overlap(out, nb, row_ptr, (size_t)(m + 1) * 4) || overlap(out, nb, col_idx, (size_t)nnz * 4) ||
        overlap(out, nb, values, (size_t)nnz * (size_t)value_bytes) || overlap(out, nb, u, (size_t)m * sizeof(float)))
      return XTVXY_ERROR_ALIASING;
  }
  if (beta != 0.0f && z != out && overlap(out, nb, z, nb)) return XTVXY_ERROR_ALIASING;
  if (!reads_x) return launch_status(launch_beta_only(n, beta, z, out, stream));
  return csr_run(kCsrTmv, m, n, nnz, alpha, row_ptr, col_idx, values, u, nullptr, beta, z, out, ws, ws_bytes,
                 stream, force, nullptr, value_bytes);
}

// t = alpha v .* (X y) + beta t0 (the first half of the pattern alone); needs no workspace.
xtvxy_status rowdot_impl(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                         const int32_t* col_idx, const void* values, const float* v, const float* y, float beta,
                         const float* t0, float* t, hipStream_t stream, const xtvxy_launch_params* force,
                         int value_bytes = 4) {
  if (m < 0 || n < 0 || nnz < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (nnz > INT32_MAX || m > INT32_MAX - 1024 || n > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  if (m == 0) return XTVXY_SUCCESS;
  if (!t) return XTVXY_ERROR_NULL_POINTER;
  if (beta != 0.0f && !t0) return XTVXY_ERROR_NULL_POINTER;
  const bool reads_x = alpha != 0.0f && n > 0 && nnz > 0;
  const size_t mb = (size_t)m * sizeof(float);
  if (reads_x) {
    if (!row_ptr || !col_idx || !values || !y) return XTVXY_ERROR_NULL_POINTER;
    if (overlap(t, mb, row_ptr, (size_t)(m + 1) * 4) || overlap(t, mb, col_idx, (size_t)nnz * 4) ||
        overlap(t, mb, values, (size_t)nnz * (size_t)value_bytes) || overlap(t, mb, y, (size_t)n * sizeof(float)) ||
        (v && overlap(t, mb, v, mb)))
      return XTVXY_ERROR_ALIASING;
  }
  if (beta != 0.0f && t0 != t && overlap(t, mb, t0, mb)) return XTVXY_ERROR_ALIASING;
  if (!reads_x) return launch_status(launch_beta_only(m, beta, t0, t, stream));
  xtvxy_device_info d;
  xtvxy_status st = device_info(-1, &d);
  if (st != XTVXY_SUCCESS) return st;
  xtvxy_launch_params plan;
  st = csr_plan_for(m, n, nnz, d, force, &plan, false);
  if (st != XTVXY_SUCCESS) return st;
  if (plan.entries_per_thread != 8) return XTVXY_ERROR_INVALID_VALUE;
  // no scatter: no output window, no bins (the LDS left holds the y window)
  plan.lds_window = 0;
  plan.bin_columns = 0;
  st = complete_csr(m, n, nnz, d, &plan);
  if (st != XTVXY_SUCCESS) return st;
  CsrArgs a{};
  a.m = m;
  a.n = n;
  a.nnz = nnz;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.values = values;
  a.value_bytes = value_bytes;
  a.v = v;
  a.y = y;
  a.lds_window = 0;
  a.y_window = plan.y_window;
  a.aligned = reinterpret_cast<uintptr_t>(values) % (uintptr_t)(4 * value_bytes) == 0 &&
              reinterpret_cast<uintptr_t>(col_idx) % 16 == 0;
  a.alpha = alpha;
  a.beta = beta;
  a.t0 = t0;
  a.t_out = t;
  const hipEvent_t before = g_before_main, after = g_after_main;
  if (before && after && mark(before, stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  const hipError_t e = plan.kernel == XTVXY_CSR_WAVES ? launch_csr_waves(a, plan, stream, kCsrRowdot)
                                                      : launch_csr(a, plan, stream, kCsrRowdot);
  if (e != hipSuccess) return XTVXY_ERROR_LAUNCH;
  if (before && after && mark(after, stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  return XTVXY_SUCCESS;
}

}  // namespace

extern "C" {

const char* xtvxy_status_string(xtvxy_status s) {
  switch (s) {
    case XTVXY_SUCCESS: return "XTVXY_SUCCESS";
    case XTVXY_ERROR_INVALID_VALUE: return "XTVXY_ERROR_INVALID_VALUE";
    case XTVXY_ERROR_NULL_POINTER: return "XTVXY_ERROR_NULL_POINTER";
    case XTVXY_ERROR_ALIASING: return "XTVXY_ERROR_ALIASING";
    case XTVXY_ERROR_WORKSPACE: return "XTVXY_ERROR_WORKSPACE";
    case XTVXY_ERROR_UNSUPPORTED: return "XTVXY_ERROR_UNSUPPORTED";
    case XTVXY_ERROR_LAUNCH: return "XTVXY_ERROR_LAUNCH";
    case XTVXY_ERROR_LIBRARY: return "XTVXY_ERROR_LIBRARY";
  }
  return "XTVXY_UNKNOWN_STATUS";
}

xtvxy_status xtvxy_set_kernel_timing_events(hipEvent_t before_main, hipEvent_t after_main) {
  if ((before_main == nullptr) != (after_main == nullptr)) return XTVXY_ERROR_NULL_POINTER;
  g_before_main = before_main;
  g_after_main = after_main;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_test_group_wait(int32_t polls, int32_t unanswered) {
  if (polls < 0) return XTVXY_ERROR_INVALID_VALUE;
  g_wait_polls = (uint32_t)polls;
  g_wait_unanswered = unanswered != 0 ? 1u : 0u;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_get_device_info(int device, xtvxy_device_info* info) {
  if (!info) return XTVXY_ERROR_NULL_POINTER;
  return device_info(device, info);
}



xtvxy_status xtvxy_dense_f32_plan(int64_t m, int64_t n, int64_t ldx, int X_aligned16, const xtvxy_device_info* dev,
                                  xtvxy_launch_params* plan) {
  return dense_plan_query(m, n, ldx, X_aligned16, dev, plan, 4);
}

xtvxy_status xtvxy_dense_f32_plan_complete(int64_t m, int64_t n, int64_t ldx, const xtvxy_device_info* dev,
                                           xtvxy_launch_params* plan) {
  return dense_complete_query(m, n, ldx, dev, plan, 4);
}

xtvxy_status xtvxy_dense_bf16_plan(int64_t m, int64_t n, int64_t ldx, int X_aligned16, const xtvxy_device_info* dev,
                                   xtvxy_launch_params* plan) {
  return dense_plan_query(m, n, ldx, X_aligned16, dev, plan, 2);
}

xtvxy_status xtvxy_dense_bf16_plan_complete(int64_t m, int64_t n, int64_t ldx, const xtvxy_device_info* dev,
                                            xtvxy_launch_params* plan) {
  return dense_complete_query(m, n, ldx, dev, plan, 2);
}

xtvxy_status xtvxy_csr_f32_plan(int64_t m, int64_t n, int64_t nnz, const xtvxy_device_info* dev,
                                xtvxy_launch_params* plan) {
  if (!plan) return XTVXY_ERROR_NULL_POINTER;
  if (m < 0 || n < 0 || nnz < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (nnz > INT32_MAX || m > INT32_MAX - 1024 || n > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  xtvxy_device_info d;
  if (dev) {
    d = *dev;
  } else {
    xtvxy_status st = device_info(-1, &d);
    if (st != XTVXY_SUCCESS) return st;
  }
  if (d.compute_units <= 0 || d.hbm_bytes_per_s <= 0) return XTVXY_ERROR_INVALID_VALUE;
  return model_csr(m, n, nnz, d, plan);
}

xtvxy_status xtvxy_csr_f32_plan_rows(int64_t m, int64_t n, int64_t nnz, int64_t longest_row,
                                     const xtvxy_device_info* dev, xtvxy_launch_params* plan) {
  if (!plan) return XTVXY_ERROR_NULL_POINTER;
  if (longest_row < 0 || longest_row > nnz) return XTVXY_ERROR_INVALID_VALUE;
  xtvxy_status st = xtvxy_csr_f32_plan(m, n, nnz, dev, plan);
  if (st != XTVXY_SUCCESS) return st;
  xtvxy_device_info d;
  if (dev) {
    d = *dev;
  } else if ((st = device_info(-1, &d)) != XTVXY_SUCCESS) {
    return st;
  }
  (void)refine_waves_grid(m, n, nnz, longest_row, d, plan);
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_csr_f32_plan_complete(int64_t m, int64_t n, int64_t nnz, const xtvxy_device_info* dev,
                                         xtvxy_launch_params* plan) {
  if (!plan) return XTVXY_ERROR_NULL_POINTER;
  if (m < 0 || n < 0 || nnz < 0) return XTVXY_ERROR_INVALID_VALUE;
  xtvxy_device_info d;
  if (dev) {
    d = *dev;
  } else {
    xtvxy_status st = device_info(-1, &d);
    if (st != XTVXY_SUCCESS) return st;
  }
  return complete_csr(m, n, nnz, d, plan);
}


xtvxy_status xtvxy_dense_f32_workspace_size(int64_t m, int64_t n, int64_t ldx, size_t* bytes) {
  return dense_workspace_query(m, n, ldx, bytes, 4);
}

xtvxy_status xtvxy_dense_bf16_workspace_size(int64_t m, int64_t n, int64_t ldx, size_t* bytes) {
  return dense_workspace_query(m, n, ldx, bytes, 2);
}

xtvxy_status xtvxy_csr_f32_workspace_size(int64_t m, int64_t n, int64_t nnz, size_t* bytes) {
  if (!bytes) return XTVXY_ERROR_NULL_POINTER;
  *bytes = 0;
  if (m < 0 || n < 0 || nnz < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (m == 0 || n == 0 || nnz == 0) return XTVXY_SUCCESS;
  xtvxy_launch_params p;
  xtvxy_status st = xtvxy_csr_f32_plan(m, n, nnz, nullptr, &p);
  if (st != XTVXY_SUCCESS) return st;
  *bytes = (size_t)p.workspace_bytes;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_dense_f32(int64_t m, int64_t n, float alpha, const float* X, int64_t ldx, const float* v,
                             const float* y, float beta, const float* z, float* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return dense_impl(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream, nullptr);
}

xtvxy_status xtvxy_dense_f32_ex(int64_t m, int64_t n, float alpha, const float* X, int64_t ldx, const float* v,
                                const float* y, float beta, const float* z, float* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, const xtvxy_launch_params* force) {
  return dense_impl(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream, force);
}

xtvxy_status xtvxy_dense_bf16(int64_t m, int64_t n, float alpha, const uint16_t* X, int64_t ldx, const float* v,
                              const float* y, float beta, const float* z, float* out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  return dense_impl(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream, nullptr, 2);
}

xtvxy_status xtvxy_dense_bf16_ex(int64_t m, int64_t n, float alpha, const uint16_t* X, int64_t ldx, const float* v,
                                 const float* y, float beta, const float* z, float* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream, const xtvxy_launch_params* force) {
  return dense_impl(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream, force, 2);
}

xtvxy_status xtvxy_dense_f16(int64_t m, int64_t n, float alpha, const uint16_t* X, int64_t ldx, const float* v,
                             const float* y, float beta, const float* z, float* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return dense_impl(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream, nullptr, 2, true);
}

xtvxy_status xtvxy_dense_f16_ex(int64_t m, int64_t n, float alpha, const uint16_t* X, int64_t ldx, const float* v,
                                const float* y, float beta, const float* z, float* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, const xtvxy_launch_params* force) {
  return dense_impl(m, n, alpha, X, ldx, v, y, beta, z, out, workspace, workspace_bytes, stream, force, 2, true);
}

xtvxy_status xtvxy_csr_f32(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                           const int32_t* col_idx, const float* values, const float* v, const float* y, float beta,
                           const float* z, float* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return csr_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, workspace, workspace_bytes,
                  stream, nullptr);
}

xtvxy_status xtvxy_csr_f32_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                              const int32_t* col_idx, const float* values, const float* v, const float* y,
                              float beta, const float* z, float* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, const xtvxy_launch_params* force) {
  return csr_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, workspace, workspace_bytes,
                  stream, force);
}

xtvxy_status xtvxy_csr_bf16(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                            const int32_t* col_idx, const uint16_t* values, const float* v, const float* y,
                            float beta, const float* z, float* out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return csr_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, workspace, workspace_bytes,
                  stream, nullptr, 2);
}

xtvxy_status xtvxy_csr_bf16_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                               const int32_t* col_idx, const uint16_t* values, const float* v, const float* y,
                               float beta, const float* z, float* out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, const xtvxy_launch_params* force) {
  return csr_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, workspace, workspace_bytes,
                  stream, force, 2);
}

xtvxy_status xtvxy_csr_bf16_rowdot(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                                   const int32_t* col_idx, const uint16_t* values, const float* v, const float* y,
                                   float beta, const float* t0, float* t, hipStream_t stream) {
  return rowdot_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t, stream, nullptr, 2);
}

xtvxy_status xtvxy_csr_bf16_rowdot_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                                      const int32_t* col_idx, const uint16_t* values, const float* v, const float* y,
                                      float beta, const float* t0, float* t, hipStream_t stream,
                                      const xtvxy_launch_params* force) {
  return rowdot_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t, stream, force, 2);
}

xtvxy_status xtvxy_csr_bf16_tmv(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                                const int32_t* col_idx, const uint16_t* values, const float* u, float beta,
                                const float* z, float* out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return tmv_impl(m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out, workspace, workspace_bytes, stream,
                  nullptr, 2);
}

xtvxy_status xtvxy_csr_bf16_tmv_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                                   const int32_t* col_idx, const uint16_t* values, const float* u, float beta,
                                   const float* z, float* out, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream, const xtvxy_launch_params* force) {
  return tmv_impl(m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out, workspace, workspace_bytes, stream,
                  force, 2);
}

xtvxy_status xtvxy_csr_f32_rowdot(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                                  const int32_t* col_idx, const float* values, const float* v, const float* y,
                                  float beta, const float* t0, float* t, hipStream_t stream) {
  return rowdot_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t, stream, nullptr);
}

xtvxy_status xtvxy_csr_f32_rowdot_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                                     const int32_t* col_idx, const float* values, const float* v, const float* y,
                                     float beta, const float* t0, float* t, hipStream_t stream,
                                     const xtvxy_launch_params* force) {
  return rowdot_impl(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, t0, t, stream, force);
}

xtvxy_status xtvxy_csr_f32_tmv(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                               const int32_t* col_idx, const float* values, const float* u, float beta,
                               const float* z, float* out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return tmv_impl(m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out, workspace, workspace_bytes, stream,
                  nullptr);
}

xtvxy_status xtvxy_csr_f32_tmv_ex(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                                  const int32_t* col_idx, const float* values, const float* u, float beta,
                                  const float* z, float* out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, const xtvxy_launch_params* force) {
  return tmv_impl(m, n, nnz, alpha, row_ptr, col_idx, values, u, beta, z, out, workspace, workspace_bytes, stream,
                  force);
}

xtvxy_status xtvxy_csr_check(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                             int32_t* d_flag, hipStream_t stream) {
  if (m < 0 || n < 0 || nnz < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (nnz > INT32_MAX || m >= INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  if (!row_ptr || !d_flag || (nnz > 0 && !col_idx)) return XTVXY_ERROR_NULL_POINTER;
  return launch_status(launch_csr_check(m, n, nnz, row_ptr, col_idx, d_flag, stream));
}

}  // extern "C"

// Shared with unfused.cpp: the dense argument checks.
namespace xtvxy {
xtvxy_status check_dense_args(int64_t m, int64_t n, float alpha, const void* X, int64_t ldx, const float* v,
                              const float* y, float beta, const float* z, const float* out, bool* quick,
                              int elem_bytes) {
  return check_dense(m, n, alpha, X, ldx, v, y, beta, z, out, quick, elem_bytes);
}
xtvxy_status check_csr_args(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                            const int32_t* col_idx, const float* values, const float* v, const float* y,
                            float beta, const float* z, const float* out, bool* quick, int value_bytes) {
  return check_csr(m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, quick, value_bytes);
}
}  // namespace xtvxy

namespace xtvxy {
hipError_t allow_dynamic_lds(const void* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_lds_mutex);
  if (g_lds_done.count({dev, fn})) return hipSuccess;
  int lds = 0;
  e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  hipFuncAttributes attr;
  e = hipFuncGetAttributes(&attr, fn);
  if (e != hipSuccess) return e;
  const int dynamic = lds - (int)attr.sharedSizeBytes;  // the kernel's static LDS comes out of the same budget
  if (dynamic <= 0) return hipErrorInvalidValue;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, dynamic);
  if (e != hipSuccess) return e;
  g_lds_done.insert({dev, fn});
  return hipSuccess;
}
}  // namespace xtvxy

namespace xtvxy {
xtvxy_status csr_run_fused(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                           const int32_t* col_idx, const void* values, const float* v, const float* y, float beta,
                           const float* z, float* out, void* ws, size_t ws_bytes, hipStream_t stream,
                           const xtvxy_launch_params* force, const CsrExtras* extras, int value_bytes) {
  return csr_run(kCsrFused, m, n, nnz, alpha, row_ptr, col_idx, values, v, y, beta, z, out, ws, ws_bytes, stream,
                 force, extras, value_bytes);
}
xtvxy_status current_device_info(xtvxy_device_info* d) { return device_info(-1, d); }
hipError_t mark_before_main(hipStream_t s) {
  return g_before_main && g_after_main ? hipEventRecord(g_before_main, s) : hipSuccess;
}
hipError_t mark_after_main(hipStream_t s) {
  return g_before_main && g_after_main ? hipEventRecord(g_after_main, s) : hipSuccess;
}
}  // namespace xtvxy
