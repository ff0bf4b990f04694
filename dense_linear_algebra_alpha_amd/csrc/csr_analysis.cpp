// Structure analysis of a CSR matrix and the calls that use it (xtvxy.h: xtvxy_csr_f32_analyse,
// xtvxy_csr_f32_analysed). "On optimizing machine learning workloads via kernel fusion" (abstract):
// the launch parameters follow from the input's characteristics; the characteristics read here
// are the matrix's column counts (which columns are hot) and row lengths (which row classes).
//
// Once per matrix (blocking, allocating):
//   1. counts[j] = entries of column j (a counting kernel), read back;
//   2. the columns ordered by count, most first, ties by index: perm[s] = the column of slot s;
//      the relabelled indices col_slot[p] = slot of col_idx[p] (a gather kernel);
//   3. the nonempty rows grouped by class (csr_row_class: very long rows first, then classes
//      6 down to 0, each in row order) with their entry bounds, and cut into batches: 64 / 2^c
//      rows of class c < 7 (a row per group of 2^c lanes), one very long row;
//   4. the model's plan for the relabelled matrix, the wavefront kernel's grid refined by the
//      longest row (refine_waves_grid); the prefix sums of the sorted column counts give the
//      entries outside any output window, so each call's bin pool holds exactly those.
// Per call: yp[s] = y[perm[s]] into the workspace, the fused kernel on (row_ptr, col_slot, values,
// v, yp), the bin passes, and the aggregation writing out[perm[s]].
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

#include "internal.h"

using namespace xtvxy;

struct xtvxy_csr_analysis_s {
  int device = -1;
  int64_t m = 0, n = 0, nnz = 0;
  const int32_t* row_ptr = nullptr;  // the caller's
  int32_t* col_slot = nullptr;       // [nnz] relabelled column indices (owned)
  int32_t* perm = nullptr;           // [n] column of each slot (owned)
  int32_t* rows = nullptr;           // nonempty rows by class (owned)
  int32_t* bounds = nullptr;         // [rows][2] their entry bounds (owned)
  int32_t* batches = nullptr;        // [batches_count][2] (owned)
  int32_t* batch_prefix = nullptr;   // [batches_count + 1] (owned)
  int32_t batches_count = 0;
  int64_t longest_row = 0;           // entries of the longest row
  std::vector<int64_t> covered;      // entries in the k most frequent columns, k = 0..n
  xtvxy_launch_params plan{};        // the model's, workspace_bytes including the gathered y
};

namespace {

void release(xtvxy_csr_analysis a) {
  if (!a) return;
  for (void* p : {(void*)a->col_slot, (void*)a->perm, (void*)a->rows, (void*)a->bounds, (void*)a->batches,
                  (void*)a->batch_prefix})
    if (p) (void)hipFree(p);
  delete a;
}

// Entries whose relabelled column lies outside the plan's output window: those outside the
// lds_window most frequent columns.
int64_t binned_items(const xtvxy_csr_analysis a, const xtvxy_launch_params& p) {
  if (a->covered.empty()) return -1;  // an empty matrix was not analysed
  const int64_t w = std::min<int64_t>(std::max<int64_t>(p.lds_window, 0), a->n);
  return a->nnz - a->covered[(size_t)w];
}

// Bytes of the fused path's workspace for a completed plan (its bin pool sized for the entries
// the plan bins), then the gathered y.
size_t yp_offset(const xtvxy_csr_analysis a, const xtvxy_launch_params& p) {
  return align_up((size_t)csr_workspace(a->m, a->n, a->nnz, p, binned_items(a, p)).total);
}

xtvxy_status complete_for(const xtvxy_csr_analysis a, xtvxy_launch_params* p) {
  xtvxy_device_info d;
  xtvxy_status st = current_device_info(&d);
  if (st != XTVXY_SUCCESS) return st;
  st = complete_csr(a->m, a->n, a->nnz, d, p);
  if (st != XTVXY_SUCCESS) return st;
  p->workspace_bytes = (int64_t)(yp_offset(a, *p) + align_up((size_t)a->n * sizeof(float)));
  return XTVXY_SUCCESS;
}

template <class T>
hipError_t upload(T** dst, const std::vector<T>& src, hipStream_t stream) {
  hipError_t e = hipMalloc(reinterpret_cast<void**>(dst), std::max<size_t>(src.size(), 1) * sizeof(T));
  if (e != hipSuccess) return e;
  if (src.empty()) return hipSuccess;
  return hipMemcpyAsync(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice, stream);
}

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

// Steps 1-3 for a matrix with rows, columns and entries.
xtvxy_status analyse(xtvxy_csr_analysis an, const int32_t* row_ptr, const int32_t* col_idx, hipStream_t stream) {
  const int64_t m = an->m, n = an->n, nnz = an->nnz;
  // 1. column counts
  uint32_t* counts = nullptr;
  if (hipMalloc(&counts, (size_t)n * sizeof(uint32_t)) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  std::vector<uint32_t> h_counts((size_t)n);
  std::vector<int32_t> h_rp((size_t)m + 1);
  hipError_t e = launch_zero(counts, (size_t)n * sizeof(uint32_t), stream);
  if (e == hipSuccess) e = launch_col_count(col_idx, nnz, counts, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h_counts.data(), counts, (size_t)n * sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h_rp.data(), row_ptr, ((size_t)m + 1) * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  (void)hipFree(counts);
  if (e != hipSuccess) return XTVXY_ERROR_LAUNCH;

  // 2. the columns by count, most first; the relabelled indices
  std::vector<int32_t> perm((size_t)n), slot((size_t)n);
  std::iota(perm.begin(), perm.end(), 0);
  std::stable_sort(perm.begin(), perm.end(), [&](int32_t x, int32_t y) { return h_counts[x] > h_counts[y]; });
  an->covered.assign((size_t)n + 1, 0);
  for (int64_t s = 0; s < n; ++s) {
    slot[(size_t)perm[s]] = (int32_t)s;
    an->covered[(size_t)s + 1] = an->covered[(size_t)s] + h_counts[(size_t)perm[s]];
  }
  int32_t* d_slot = nullptr;
  e = upload(&an->perm, perm, stream);
  if (e == hipSuccess) e = upload(&d_slot, slot, stream);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&an->col_slot), (size_t)nnz * sizeof(int32_t));
  if (e == hipSuccess) e = launch_relabel(col_idx, nnz, d_slot, an->col_slot, stream);

  // 3. rows by class with their bounds, batches
  std::vector<std::vector<int32_t>> by_class(kRowsVeryLong + 1);
  for (int64_t i = 0; i < m; ++i) {
    const int64_t len = (int64_t)h_rp[(size_t)i + 1] - h_rp[(size_t)i];
    if (len > 0) by_class[(size_t)csr_row_class(len)].push_back((int32_t)i);
  }
  std::vector<int32_t> rows, bounds, batches, prefix(1, 0);
  rows.reserve((size_t)m);
  bounds.reserve(2 * (size_t)m);
  for (int c = kRowsVeryLong; c >= 0; --c) {
    const std::vector<int32_t>& rc = by_class[(size_t)c];
    const size_t per = c == kRowsVeryLong ? 1 : (size_t)(64 >> c);
    for (size_t i = 0; i < rc.size(); i += per) {
      const size_t end = std::min(rc.size(), i + per);
      batches.push_back((int32_t)rows.size());
      batches.push_back(c * 256 + (int32_t)(end - i));
      int64_t entries = 0;
      for (size_t k = i; k < end; ++k) {
        const int32_t r = rc[k];
        rows.push_back(r);
        bounds.push_back(h_rp[(size_t)r]);
        bounds.push_back(h_rp[(size_t)r + 1]);
        entries += (int64_t)h_rp[(size_t)r + 1] - h_rp[(size_t)r];
      }
      prefix.push_back(prefix.back() + (int32_t)entries);
    }
  }
  an->batches_count = (int32_t)(batches.size() / 2);
  for (int64_t i = 0; i < m; ++i)
    an->longest_row = std::max<int64_t>(an->longest_row, (int64_t)h_rp[(size_t)i + 1] - h_rp[(size_t)i]);
  if (e == hipSuccess) e = upload(&an->rows, rows, stream);
  if (e == hipSuccess) e = upload(&an->bounds, bounds, stream);
  if (e == hipSuccess) e = upload(&an->batches, batches, stream);
  if (e == hipSuccess) e = upload(&an->batch_prefix, prefix, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);  // the host vectors above outlive their copies
  if (d_slot) (void)hipFree(d_slot);
  return e == hipSuccess ? XTVXY_SUCCESS : XTVXY_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

xtvxy_status xtvxy_csr_f32_analyse(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                                   hipStream_t stream, xtvxy_csr_analysis* analysis) {
  if (!analysis) return XTVXY_ERROR_NULL_POINTER;
  *analysis = nullptr;
  if (m < 0 || n < 0 || nnz < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (nnz > INT32_MAX || m > INT32_MAX - 1024 || n > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  const bool empty = m == 0 || n == 0 || nnz == 0;
  if (!empty && (!row_ptr || !col_idx)) return XTVXY_ERROR_NULL_POINTER;
  xtvxy_csr_analysis an = new xtvxy_csr_analysis_s;
  an->m = m;
  an->n = n;
  an->nnz = nnz;
  an->row_ptr = row_ptr;
  if (hipGetDevice(&an->device) != hipSuccess) {
    release(an);
    return XTVXY_ERROR_LAUNCH;
  }
  if (!empty) {
    xtvxy_status st = analyse(an, row_ptr, col_idx, stream);
    if (st == XTVXY_SUCCESS) {
      xtvxy_device_info d;
      st = current_device_info(&d);
      // the model's plan for the relabelled matrix: its output and y windows [0, W) and [0, Wy) now
      // hold the most frequent columns whatever the caller's column order
      if (st == XTVXY_SUCCESS) st = model_csr(m, n, nnz, d, &an->plan);
      // the longest row refines the wavefront kernel's grid
      if (st == XTVXY_SUCCESS) (void)refine_waves_grid(m, n, nnz, an->longest_row, d, &an->plan);
      if (st == XTVXY_SUCCESS) st = complete_for(an, &an->plan);
    }
    if (st != XTVXY_SUCCESS) {
      release(an);
      return st;
    }
  }
  *analysis = an;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_csr_f32_analysis_destroy(xtvxy_csr_analysis analysis) {
  release(analysis);
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_csr_f32_analysed_plan(xtvxy_csr_analysis analysis, xtvxy_launch_params* plan) {
  if (!analysis || !plan) return XTVXY_ERROR_NULL_POINTER;
  *plan = analysis->plan;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_csr_f32_analysed_plan_complete(xtvxy_csr_analysis analysis, xtvxy_launch_params* plan) {
  if (!analysis || !plan) return XTVXY_ERROR_NULL_POINTER;
  if (analysis->nnz == 0 || analysis->m == 0 || analysis->n == 0) {
    plan->workspace_bytes = 0;
    return XTVXY_SUCCESS;
  }
  return complete_for(analysis, plan);
}

xtvxy_status xtvxy_csr_f32_analysed_workspace_size(xtvxy_csr_analysis analysis, size_t* bytes) {
  if (!analysis || !bytes) return XTVXY_ERROR_NULL_POINTER;
  *bytes = (size_t)analysis->plan.workspace_bytes;
  return XTVXY_SUCCESS;
}

}  // extern "C"

namespace {

// An analysed call with fp32 (value_bytes 4) or bf16 (2) values.
xtvxy_status analysed_impl(xtvxy_csr_analysis an, float alpha, const void* values, int value_bytes, const float* v,
                           const float* y, float beta, const float* z, float* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream, const xtvxy_launch_params* force) {
  if (!an) return XTVXY_ERROR_NULL_POINTER;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  if (dev != an->device) return XTVXY_ERROR_INVALID_VALUE;
  const int64_t m = an->m, n = an->n, nnz = an->nnz;
  if (n == 0) return XTVXY_SUCCESS;
  if (!out || !y) return XTVXY_ERROR_NULL_POINTER;
  if (beta != 0.0f && !z) return XTVXY_ERROR_NULL_POINTER;
  const bool reads_x = alpha != 0.0f && m > 0 && nnz > 0;
  if (reads_x && !values) return XTVXY_ERROR_NULL_POINTER;
  const size_t nb = (size_t)n * sizeof(float);
  if (reads_x) {
    if (overlap(out, nb, an->row_ptr, (size_t)(m + 1) * 4) ||
        overlap(out, nb, values, (size_t)nnz * (size_t)value_bytes) ||
        overlap(out, nb, y, nb) || (v && overlap(out, nb, v, (size_t)m * sizeof(float))))
      return XTVXY_ERROR_ALIASING;
  }
  if (beta != 0.0f && z != out && overlap(out, nb, z, nb)) return XTVXY_ERROR_ALIASING;
  if (!reads_x) return launch_beta_only(n, beta, z, out, stream) == hipSuccess ? XTVXY_SUCCESS : XTVXY_ERROR_LAUNCH;
  xtvxy_launch_params plan = force ? *force : an->plan;
  if (force) {
    xtvxy_status st = complete_for(an, &plan);
    if (st != XTVXY_SUCCESS) return st;
  }
  if (value_bytes != 4 && plan.kernel == XTVXY_CSR_ROWS) return XTVXY_ERROR_INVALID_VALUE;  // fp32 values only
  if (!workspace || workspace_bytes < (size_t)plan.workspace_bytes) return XTVXY_ERROR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return XTVXY_ERROR_WORKSPACE;
  const size_t yoff = yp_offset(an, plan);
  float* yp = reinterpret_cast<float*>(static_cast<char*>(workspace) + yoff);
  if (launch_permute(y, an->perm, n, yp, stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  CsrExtras x{an->rows, an->bounds, an->batches, an->batch_prefix, an->batches_count, an->perm,
              binned_items(an, plan)};
  return csr_run_fused(m, n, nnz, alpha, an->row_ptr, an->col_slot, values, v, yp, beta, z, out, workspace, yoff,
                       stream, &plan, &x, value_bytes);
}

}  // namespace

extern "C" {

xtvxy_status xtvxy_csr_f32_analysed_ex(xtvxy_csr_analysis an, float alpha, const float* values, const float* v,
                                       const float* y, float beta, const float* z, float* out, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream, const xtvxy_launch_params* force) {
  return analysed_impl(an, alpha, values, 4, v, y, beta, z, out, workspace, workspace_bytes, stream, force);
}

xtvxy_status xtvxy_csr_f32_analysed(xtvxy_csr_analysis analysis, float alpha, const float* values, const float* v,
                                    const float* y, float beta, const float* z, float* out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  return analysed_impl(analysis, alpha, values, 4, v, y, beta, z, out, workspace, workspace_bytes, stream, nullptr);
}

xtvxy_status xtvxy_csr_bf16_analysed_ex(xtvxy_csr_analysis an, float alpha, const uint16_t* values, const float* v,
                                        const float* y, float beta, const float* z, float* out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream,
                                        const xtvxy_launch_params* force) {
  return analysed_impl(an, alpha, values, 2, v, y, beta, z, out, workspace, workspace_bytes, stream, force);
}

xtvxy_status xtvxy_csr_bf16_analysed(xtvxy_csr_analysis analysis, float alpha, const uint16_t* values,
                                     const float* v, const float* y, float beta, const float* z, float* out,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return analysed_impl(analysis, alpha, values, 2, v, y, beta, z, out, workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"
