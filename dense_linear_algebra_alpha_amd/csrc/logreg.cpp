// Newton-CG for L2-regularised logistic regression on CSR X: the host driver.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract) closes with a whole ML
// algorithm run on the fused kernel. Here that algorithm is line search Newton-CG (Nocedal and
// Wright, "Numerical Optimization", Algorithm 7.1, with the backtracking of Algorithm 3.1), whose
// Hessian-vector product is the pattern (alpha 1, v = p(1 - p), y = z = d, beta = lambda), whose
// gradient is the pattern's second half and whose line search needs the first half (X s).
//
// The driver enqueues kernels on the caller's stream and copies the solver's device scalars
// (LrScalars) to the host only where a decision needs them: after the gradient (stop?), after
// each CG iteration when CG stops on its residual (converged? curvature?) or once after a fixed
// number of them, after each line-search trial (accept?). Everything that touches an m- or
// n-vector runs in the library's kernels.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cmath>
#include <cstdint>
#include <limits>

#include "internal.h"

using namespace xtvxy;

namespace {

constexpr double kArmijo = 1e-4;  // sufficient-decrease constant c1
constexpr double kShrink = 0.5;   // step-length factor between trials
constexpr int kHistoryCols = 6;

struct LrWorkspace {
  size_t product_off, product_bytes;  // workspace of the fused products
  size_t t_off, u_off, v_off, xs_off; // m-vectors
  size_t g_off, s_off, r_off, d_off, q_off;  // n-vectors
  size_t part_off, scalars_off;
  size_t total;
};

LrWorkspace lr_workspace(int64_t m, int64_t n, size_t product_bytes) {
  LrWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  w.product_bytes = product_bytes;
  w.product_off = take(product_bytes);
  const size_t mb = (size_t)m * sizeof(float), nb = (size_t)n * sizeof(float);
  w.t_off = take(mb);
  w.u_off = take(mb);
  w.v_off = take(mb);
  w.xs_off = take(mb);
  w.g_off = take(nb);
  w.s_off = take(nb);
  w.r_off = take(nb);
  w.d_off = take(nb);
  w.q_off = take(nb);
  w.part_off = take((size_t)kLrRows * kLrMaxParts * sizeof(double));
  w.scalars_off = take(sizeof(LrScalars));
  w.total = off;
  return w;
}

bool finite(double x) { return std::isfinite(x); }

xtvxy_status check_options(const xtvxy_logreg_options* o) {
  if (!o) return XTVXY_ERROR_NULL_POINTER;
  if (!finite(o->lambda) || o->lambda < 0.0f) return XTVXY_ERROR_INVALID_VALUE;
  if (o->max_newton < 0 || o->max_cg < 1 || o->max_backtracks < 1) return XTVXY_ERROR_INVALID_VALUE;
  if (!finite(o->grad_tol) || o->grad_tol < 0.0) return XTVXY_ERROR_INVALID_VALUE;
  if (!(o->cg_forcing > 0.0 && o->cg_forcing <= 1.0)) return XTVXY_ERROR_INVALID_VALUE;
  if (o->engine != XTVXY_LOGREG_FUSED && o->engine != XTVXY_LOGREG_UNFUSED) return XTVXY_ERROR_INVALID_VALUE;
  return XTVXY_SUCCESS;
}

// The products of one engine: H d, X^T u + lambda w, X s.
struct Engine {
  int kind;
  int64_t m, n, nnz;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const void* values;       // fp32, or bf16 bit patterns (value_bytes 2; the fused engine only)
  int value_bytes;
  xtvxy_csr_unfused_plan plan;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  const xtvxy_launch_params* hvp_plan;  // the fused H d's plan when the row lengths refine it, else null

  const float* f32() const { return static_cast<const float*>(values); }
  const uint16_t* b16() const { return static_cast<const uint16_t*>(values); }

  xtvxy_status hvp(const float* v, float lam, const float* d, float* q) const {
    if (kind == XTVXY_LOGREG_FUSED && value_bytes == 2)
      return xtvxy_csr_bf16_ex(m, n, nnz, 1.0f, row_ptr, col_idx, b16(), v, d, lam, d, q, ws, ws_bytes, stream,
                               hvp_plan);
    if (kind == XTVXY_LOGREG_FUSED)
      return xtvxy_csr_f32_ex(m, n, nnz, 1.0f, row_ptr, col_idx, f32(), v, d, lam, d, q, ws, ws_bytes, stream,
                              hvp_plan);
    return xtvxy_csr_f32_unfused_reference(plan, 1.0f, v, d, lam, d, q, stream);
  }
  xtvxy_status gradient(const float* u, float lam, const float* w, float* g) const {
    if (kind == XTVXY_LOGREG_FUSED && value_bytes == 2)
      return xtvxy_csr_bf16_tmv(m, n, nnz, 1.0f, row_ptr, col_idx, b16(), u, lam, w, g, ws, ws_bytes, stream);
    if (kind == XTVXY_LOGREG_FUSED)
      return xtvxy_csr_f32_tmv(m, n, nnz, 1.0f, row_ptr, col_idx, f32(), u, lam, w, g, ws, ws_bytes, stream);
    return unfused_tmv(plan, 1.0f, u, lam, w, g, stream);
  }
  xtvxy_status margins(const float* y, float* t) const {
    if (kind == XTVXY_LOGREG_FUSED && value_bytes == 2)
      return xtvxy_csr_bf16_rowdot(m, n, nnz, 1.0f, row_ptr, col_idx, b16(), nullptr, y, 0.0f, nullptr, t, stream);
    if (kind == XTVXY_LOGREG_FUSED)
      return xtvxy_csr_f32_rowdot(m, n, nnz, 1.0f, row_ptr, col_idx, f32(), nullptr, y, 0.0f, nullptr, t, stream);
    return unfused_rowdot(plan, y, t, stream);
  }
};

}  // namespace

extern "C" {

xtvxy_status xtvxy_logreg_newton_cg_f32_workspace_size(int64_t m, int64_t n, int64_t nnz, size_t* bytes) {
  if (!bytes) return XTVXY_ERROR_NULL_POINTER;
  if (m < 0 || n < 0 || nnz < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (nnz > INT32_MAX || m > INT32_MAX - 1024 || n > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  size_t product = 0;
  const xtvxy_status st = xtvxy_csr_f32_workspace_size(m, n, nnz, &product);
  if (st != XTVXY_SUCCESS) return st;
  *bytes = lr_workspace(m, n, product).total;
  return XTVXY_SUCCESS;
}

// The solver with fp32 (value_bytes 4) or bf16 (2; the fused engine only) values.
static xtvxy_status newton_cg(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                              const void* values, int value_bytes, const float* labels, float* w,
                              const xtvxy_logreg_options* opt, xtvxy_csr_unfused_plan unfused, void* workspace,
                              size_t workspace_bytes, hipStream_t stream, xtvxy_logreg_report* report,
                              double* history, int64_t history_rows) {
  // ---- argument checks, before anything touches the device
  if (m < 0 || n < 0 || nnz < 0 || history_rows < 0) return XTVXY_ERROR_INVALID_VALUE;
  if (nnz > INT32_MAX || m > INT32_MAX - 1024 || n > INT32_MAX) return XTVXY_ERROR_UNSUPPORTED;
  xtvxy_status st = check_options(opt);
  if (st != XTVXY_SUCCESS) return st;
  if (value_bytes == 2 && opt->engine != XTVXY_LOGREG_FUSED) return XTVXY_ERROR_INVALID_VALUE;
  if (!row_ptr || (nnz > 0 && (!col_idx || !values)) || (m > 0 && !labels) || (n > 0 && !w))
    return XTVXY_ERROR_NULL_POINTER;
  if (history_rows > 0 && !history) return XTVXY_ERROR_NULL_POINTER;
  if (opt->engine == XTVXY_LOGREG_UNFUSED) {
    if (!unfused) return XTVXY_ERROR_NULL_POINTER;
    int64_t pm, pn, pnnz;
    const int32_t *prp, *pci;
    const float* pv;
    unfused_plan_shape(unfused, &pm, &pn, &pnnz, &prp, &pci, &pv);
    if (pm != m || pn != n || pnnz != nnz || prp != row_ptr || (nnz > 0 && (pci != col_idx || pv != values)))
      return XTVXY_ERROR_INVALID_VALUE;
  }
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return XTVXY_ERROR_WORKSPACE;
  size_t product = 0;
  st = xtvxy_csr_f32_workspace_size(m, n, nnz, &product);
  if (st != XTVXY_SUCCESS) return st;
  const LrWorkspace L = lr_workspace(m, n, product);
  if (workspace_bytes < L.total) return XTVXY_ERROR_WORKSPACE;

  const auto t_start = std::chrono::steady_clock::now();
  char* base = static_cast<char*>(workspace);
  float* t = reinterpret_cast<float*>(base + L.t_off);
  float* u = reinterpret_cast<float*>(base + L.u_off);
  float* v = reinterpret_cast<float*>(base + L.v_off);
  float* xs = reinterpret_cast<float*>(base + L.xs_off);
  float* g = reinterpret_cast<float*>(base + L.g_off);
  float* s = reinterpret_cast<float*>(base + L.s_off);  // the CG iterate, then the Newton step
  float* r = reinterpret_cast<float*>(base + L.r_off);
  float* d = reinterpret_cast<float*>(base + L.d_off);
  float* q = reinterpret_cast<float*>(base + L.q_off);
  double* part = reinterpret_cast<double*>(base + L.part_off);
  LrScalars* S = reinterpret_cast<LrScalars*>(base + L.scalars_off);
  const float lam = opt->lambda;
  LrScalars h{};
  auto launched = [](hipError_t e) { return e == hipSuccess ? XTVXY_SUCCESS : XTVXY_ERROR_LAUNCH; };
  auto read_scalars = [&]() -> xtvxy_status {
    if (hipMemcpyAsync(&h, S, sizeof(LrScalars), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return XTVXY_ERROR_LAUNCH;
    return XTVXY_SUCCESS;
  };
  // The Hessian-vector products are most of a step. Their plan is the model's, except that the
  // longest row (one scan of row_ptr and one read-back per solve) can refine the wavefront
  // kernel's grid, as a structure analysis does (refine_waves_grid).
  xtvxy_launch_params hvp_plan{};
  bool refined = false;
  if (opt->engine == XTVXY_LOGREG_FUSED && m > 0 && nnz > 0 && n > 0) {
    xtvxy_device_info dinfo;
    if ((st = current_device_info(&dinfo)) != XTVXY_SUCCESS) return st;
    if ((st = xtvxy_csr_f32_plan(m, n, nnz, &dinfo, &hvp_plan)) != XTVXY_SUCCESS) return st;
    if (hvp_plan.kernel == XTVXY_CSR_WAVES) {
      if ((st = launched(launch_lr_max_row(m, row_ptr, &S->max_row, stream))) != XTVXY_SUCCESS) return st;
      if ((st = read_scalars()) != XTVXY_SUCCESS) return st;
      refined = refine_waves_grid(m, n, nnz, (int64_t)h.max_row, dinfo, &hvp_plan) &&
                (size_t)hvp_plan.workspace_bytes <= L.product_bytes;
    }
  }
  const Engine E{opt->engine, m, n, nnz, row_ptr, col_idx, values, value_bytes, unfused, base + L.product_off,
                 L.product_bytes, stream, refined ? &hvp_plan : nullptr};
  const double nan = std::numeric_limits<double>::quiet_NaN();
  auto record = [&](int64_t k, int col, double value) {
    if (k < history_rows) history[k * kHistoryCols + col] = value;
  };

  xtvxy_logreg_report rep{};
  rep.status = XTVXY_LOGREG_ITERATION_LIMIT;
  // ---- t = X w and the link quantities of the starting point
  if ((st = E.margins(w, t)) != XTVXY_SUCCESS) return st;
  if ((st = launched(launch_lr_link(m, t, nullptr, 0.0f, labels, u, v, part, stream))) != XTVXY_SUCCESS) return st;
  double g0 = 0.0;
  int64_t k = 0;
  for (;;) {
    // ---- gradient, objective, stop test
    if ((st = E.gradient(u, lam, w, g)) != XTVXY_SUCCESS) return st;
    {
      const float* x[2] = {w, g};
      const float* y[2] = {w, g};
      if ((st = launched(launch_lr_dots(n, 2, x, y, 1, part, stream))) != XTVXY_SUCCESS) return st;
    }
    if ((st = launched(launch_lr_finish(kLrObjective, part, m, n, S, 0.0, lam, stream))) != XTVXY_SUCCESS) return st;
    // CG on H s = -g: with fixed_cg the iterations are enqueued back to back and read once; the
    // stops that do not depend on the residual test (non-positive curvature, an exactly vanished
    // residual) are taken on the device, which then leaves the remaining iterations without
    // effect. Without a gradient tolerance (grad_tol == 0) nothing can stop the solve before the
    // step limit but g == 0, which CG meets as a vanished residual, so the fixed solve is
    // enqueued right behind the gradient and one read-back serves both (the CG kernels leave
    // f, g.g and w.w in the scalars as they are).
    auto enqueue_cg = [&](double eps) -> xtvxy_status {
      xtvxy_status e;
      if ((e = launched(launch_lr_cg_init(n, g, s, r, d, S, stream))) != XTVXY_SUCCESS) return e;
      for (int j = 0; j < opt->max_cg; ++j) {
        if ((e = E.hvp(v, lam, d, q)) != XTVXY_SUCCESS) return e;
        if ((e = launched(launch_lr_cg_step(n, q, d, s, r, S, j == 0, part, stream))) != XTVXY_SUCCESS) return e;
        if (opt->fixed_cg) continue;
        if ((e = read_scalars()) != XTVXY_SUCCESS) return e;
        if (h.neg || h.done || std::sqrt(h.rr) < eps) break;
      }
      return XTVXY_SUCCESS;
    };
    const bool cg_ahead = opt->fixed_cg && opt->grad_tol == 0.0 && k < opt->max_newton;
    if (cg_ahead && (st = enqueue_cg(0.0)) != XTVXY_SUCCESS) return st;
    if ((st = read_scalars()) != XTVXY_SUCCESS) return st;
    const double f = h.f, gnorm = std::sqrt(h.gg);
    if (k == 0) {
      g0 = gnorm;
      rep.loss0 = f;
      rep.grad_norm0 = gnorm;
    }
    rep.loss = f;
    rep.grad_norm = gnorm;
    record(k, 0, f);
    record(k, 1, gnorm);
    for (int col = 2; col < kHistoryCols; ++col) record(k, col, nan);
    if (gnorm <= opt->grad_tol * g0) {
      rep.status = XTVXY_LOGREG_CONVERGED;
      break;
    }
    if (k == opt->max_newton) break;
    if (!cg_ahead) {
      const double eps = std::fmin(opt->cg_forcing, std::sqrt(gnorm)) * gnorm;
      if ((st = enqueue_cg(eps)) != XTVXY_SUCCESS) return st;
      if (opt->fixed_cg && (st = read_scalars()) != XTVXY_SUCCESS) return st;
    }
    const int used = h.iters;
    rep.cg_iterations += used;
    record(k, 2, used);
    // ---- line search along s: X s, slopes, then trials of the objective change
    if ((st = E.margins(s, xs)) != XTVXY_SUCCESS) return st;
    {
      const float* x[3] = {g, w, s};
      const float* y[3] = {s, s, s};
      if ((st = launched(launch_lr_dots(n, 3, x, y, 1, part, stream))) != XTVXY_SUCCESS) return st;
    }
    if ((st = launched(launch_lr_finish(kLrLine, part, m, n, S, 0.0, lam, stream))) != XTVXY_SUCCESS) return st;
    double a = 1.0;
    bool accepted = false;
    int tried = 0;
    for (int b = 0; b < opt->max_backtracks; ++b) {
      if ((st = launched(launch_lr_trial(m, t, xs, a, labels, part, stream))) != XTVXY_SUCCESS) return st;
      if ((st = launched(launch_lr_finish(kLrTrial, part, m, n, S, a, lam, stream))) != XTVXY_SUCCESS) return st;
      if ((st = read_scalars()) != XTVXY_SUCCESS) return st;
      tried = b + 1;
      if (h.df <= kArmijo * a * h.gs) {
        accepted = true;
        break;
      }
      a *= kShrink;
    }
    rep.line_search_trials += tried;
    record(k, 3, h.gs);
    record(k, 5, tried);
    if (!accepted) {
      rep.status = XTVXY_LOGREG_LINE_SEARCH_FAILED;
      break;
    }
    record(k, 4, a);
    // ---- w += a s; t += a X s and the link quantities of the new iterate
    if ((st = launched(launch_lr_axpy(n, (float)a, s, w, stream))) != XTVXY_SUCCESS) return st;
    if ((st = launched(launch_lr_link(m, t, xs, (float)a, labels, u, v, part, stream))) != XTVXY_SUCCESS) return st;
    ++k;
  }
  if (hipStreamSynchronize(stream) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  rep.newton_iterations = (int32_t)k;
  rep.seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t_start).count();
  if (report) *report = rep;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_logreg_newton_cg_f32(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr,
                                        const int32_t* col_idx, const float* values, const float* labels, float* w,
                                        const xtvxy_logreg_options* opt, xtvxy_csr_unfused_plan unfused,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream,
                                        xtvxy_logreg_report* report, double* history, int64_t history_rows) {
  return newton_cg(m, n, nnz, row_ptr, col_idx, values, 4, labels, w, opt, unfused, workspace, workspace_bytes,
                   stream, report, history, history_rows);
}

xtvxy_status xtvxy_logreg_newton_cg_bf16(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr,
                                         const int32_t* col_idx, const uint16_t* values, const float* labels,
                                         float* w, const xtvxy_logreg_options* opt, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream, xtvxy_logreg_report* report,
                                         double* history, int64_t history_rows) {
  return newton_cg(m, n, nnz, row_ptr, col_idx, values, 2, labels, w, opt, nullptr, workspace, workspace_bytes,
                   stream, report, history, history_rows);
}

}  // extern "C"
