// Kernels of the Newton-CG logistic-regression solver (driven by logreg.cpp).
//
// "On optimizing machine learning workloads via kernel fusion" (abstract) places the pattern
// inside ML algorithms; in Newton-CG for L2-regularised logistic regression it is the
// Hessian-vector product. What surrounds it is streaming work over the m rows (the link
// function and the line search's objective change, each one pass over a few m-vectors) and
// small vector algebra over the n columns (CG updates, dot products). All of it is HBM- or
// latency-bound: plain coalesced grid-stride loops, no matrix cores.
//
// Every reduction is taken in fp64 and in a fixed order: each workgroup writes one partial sum
// per quantity to a row of `part`, and lr_finish_kernel adds a row's partials in index order, so
// a run is bitwise reproducible.
#include "device_util.h"
#include "internal.h"

namespace xtvxy {
namespace {

constexpr int kThreads = 256;       // streaming and finishing kernels
constexpr int kSmallThreads = 1024; // the one-workgroup CG update

// Sum of x over the workgroup, the same value in every thread; `red` holds BLK / 64 doubles.
template <int BLK>
__device__ inline double block_sum(double x, double* red) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // the previous use of red is over
  if (lane == 0) red[wave] = x;
  __syncthreads();
  double s = 0.0;
  for (int k = 0; k < BLK / 64; ++k) s += red[k];
  return s;
}

__device__ inline double softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

__device__ inline int64_t first_index() { return (int64_t)blockIdx.x * kThreads + threadIdx.x; }
__device__ inline int64_t grid_stride() { return (int64_t)gridDim.x * kThreads; }

// t += step * xs (when xs is given); with p = sigmoid(t): u = p - c, v = p (1 - p), and the
// partial sum of log(1 + e^t) - c t. q = sigmoid(-|t|) <= 1/2 is formed first so that neither
// u nor v subtracts nearly equal numbers: p = 1 - q for t >= 0 and p = q otherwise, and
// p (1 - p) = q (1 - q).
__global__ __launch_bounds__(kThreads) void lr_link_kernel(int64_t m, float* __restrict__ t,
                                                           const float* __restrict__ xs, float step,
                                                           const float* __restrict__ c, float* __restrict__ u,
                                                           float* __restrict__ v, double* __restrict__ part) {
  __shared__ double red[kThreads / 64];
  double loss = 0.0;
  for (int64_t i = first_index(); i < m; i += grid_stride()) {
    float ti = t[i];
    if (xs) {
      ti = ti + step * xs[i];
      t[i] = ti;
    }
    const float e = expf(-fabsf(ti));
    const float q = e / (1.0f + e);
    const float ci = c[i];
    u[i] = ti >= 0.0f ? (1.0f - ci) - q : q - ci;
    v[i] = q * (1.0f - q);
    const double td = ti;
    loss += softplus(td) - (double)ci * td;
  }
  loss = block_sum<kThreads>(loss, red);
  if (threadIdx.x == 0) part[blockIdx.x] = loss;
}

// Partial sums of the change of the rows' loss when t moves to t + a xs (in fp64).
__global__ __launch_bounds__(kThreads) void lr_trial_kernel(int64_t m, const float* __restrict__ t,
                                                            const float* __restrict__ xs, double a,
                                                            const float* __restrict__ c, double* __restrict__ part) {
  __shared__ double red[kThreads / 64];
  double sum = 0.0;
  for (int64_t i = first_index(); i < m; i += grid_stride()) {
    const double td = t[i], dd = a * (double)xs[i];
    sum += softplus(td + dd) - softplus(td) - (double)c[i] * dd;
  }
  sum = block_sum<kThreads>(sum, red);
  if (threadIdx.x == 0) part[blockIdx.x] = sum;
}

struct DotArgs {
  const float* x[3];
  const float* y[3];
  int k;
};

// Partial sums of up to three dot products of n-vectors, into rows row0 .. row0 + k - 1.
// The longest row: each wavefront's maximum of row_ptr[i + 1] - row_ptr[i], folded into *longest
// by one vector atomic maximum (the caller zeroes it).
__global__ __launch_bounds__(kThreads) void lr_max_row_kernel(int64_t m, const int32_t* __restrict__ rp,
                                                               uint32_t* longest) {
  uint32_t mx = 0u;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < m; i += (int64_t)gridDim.x * kThreads)
    mx = max(mx, (uint32_t)(rp[i + 1] - rp[i]));
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(longest, mx);
}

__global__ __launch_bounds__(kThreads) void lr_dots_kernel(int64_t n, DotArgs a, int row0, double* __restrict__ part) {
  __shared__ double red[kThreads / 64];
  double s[3] = {0.0, 0.0, 0.0};
  for (int64_t j = first_index(); j < n; j += grid_stride()) {
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (k < a.k) s[k] += (double)a.x[k][j] * (double)a.y[k][j];
  }
  for (int k = 0; k < a.k; ++k) {
    const double r = block_sum<kThreads>(s[k], red);
    if (threadIdx.x == 0) part[(size_t)(row0 + k) * kLrMaxParts + blockIdx.x] = r;
  }
}

// Sum of the first `count` partials of a row, in index order (the same value in every thread).
__device__ inline double row_sum(const double* part, int row, int count, double* red) {
  double s = 0.0;
  const double* p = part + (size_t)row * kLrMaxParts;
  for (int b = threadIdx.x; b < count; b += kThreads) s += p[b];
  return block_sum<kThreads>(s, red);
}

// One workgroup turns partial sums into the solver's scalars.
__global__ __launch_bounds__(kThreads) void lr_finish_kernel(int op, const double* __restrict__ part, int np_m,
                                                             int np_n, LrScalars* __restrict__ S, double a,
                                                             double lam) {
  __shared__ double red[kThreads / 64];
  const bool lead = threadIdx.x == 0;
  switch (op) {
    case kLrObjective: {  // row 0: loss terms (m-grid); rows 1, 2: w.w, g.g (n-grid)
      const double loss = row_sum(part, 0, np_m, red);
      const double ww = row_sum(part, 1, np_n, red);
      const double gg = row_sum(part, 2, np_n, red);
      if (lead) {
        S->f = loss + 0.5 * lam * ww;
        S->ww = ww;
        S->gg = gg;
      }
      break;
    }
    case kLrLine: {  // rows 1, 2, 3: g.s, w.s, s.s
      const double gs = row_sum(part, 1, np_n, red);
      const double ws = row_sum(part, 2, np_n, red);
      const double ss = row_sum(part, 3, np_n, red);
      if (lead) {
        S->gs = gs;
        S->ws = ws;
        S->ss = ss;
      }
      break;
    }
    case kLrTrial: {  // row 0: the rows' loss change at step a; the penalty's change in closed form
      const double rows = row_sum(part, 0, np_m, red);
      if (lead) S->df = rows + lam * (a * S->ws + 0.5 * a * a * S->ss);
      break;
    }
    case kLrCgAlpha: {  // row 1: d.Hd (nothing once CG has stopped)
      const double kappa = row_sum(part, 1, np_n, red);
      if (lead && !S->neg && !S->done) {
        S->kappa = kappa;
        if (kappa > 0.0) {
          S->alpha = S->rr / kappa;
        } else {
          S->neg = 1;  // also for NaN
          S->iters += 1;
        }
      }
      break;
    }
    case kLrCgBeta: {  // row 1: the new r.r
      const double rn = row_sum(part, 1, np_n, red);
      if (lead && !S->neg && !S->done) {
        S->beta = rn / S->rr;
        S->rr = rn;
        S->iters += 1;
        if (rn == 0.0) S->done = 1;
      }
      break;
    }
    default:
      break;
  }
}

// CG start: s = 0, r = g, d = -g, r.r = g.g.
__global__ __launch_bounds__(kThreads) void lr_cg_init_kernel(int64_t n, const float* __restrict__ g,
                                                              float* __restrict__ z, float* __restrict__ r,
                                                              float* __restrict__ d, LrScalars* __restrict__ S) {
  for (int64_t j = first_index(); j < n; j += grid_stride()) {
    const float gj = g[j];
    z[j] = 0.0f;
    r[j] = gj;
    d[j] = -gj;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    S->rr = S->gg;
    S->neg = 0;
    S->done = 0;
    S->iters = 0;
  }
}

// One CG iteration after q = H d, in one workgroup (n <= kLrSmallCg):
// kappa = d.q; on kappa <= 0 (or NaN) flag it and, at the first iteration, set s = d (= -g);
// else alpha = r.r / kappa, s += alpha d, r += alpha q, beta = r.r(new) / r.r, d = -r + beta d,
// and flag an exactly vanished residual. Once either flag is set the iteration does nothing, so
// the host may enqueue a fixed number of iterations without reading anything back.
__global__ __launch_bounds__(kSmallThreads) void lr_cg_small_kernel(int64_t n, const float* __restrict__ q,
                                                                    float* __restrict__ d, float* __restrict__ z,
                                                                    float* __restrict__ r,
                                                                    LrScalars* __restrict__ S, int first) {
  __shared__ double red[kSmallThreads / 64];
  const int tid = threadIdx.x;
  if (S->neg || S->done) return;  // the same value in every thread
  double kap = 0.0;
  for (int64_t j = tid; j < n; j += kSmallThreads) kap += (double)d[j] * (double)q[j];
  kap = block_sum<kSmallThreads>(kap, red);
  if (!(kap > 0.0)) {
    if (first)
      for (int64_t j = tid; j < n; j += kSmallThreads) z[j] = d[j];
    if (tid == 0) {
      S->kappa = kap;
      S->neg = 1;
      S->iters += 1;
    }
    return;
  }
  const double rr = S->rr;
  const double al = rr / kap;
  const float alf = (float)al;
  double rn = 0.0;
  for (int64_t j = tid; j < n; j += kSmallThreads) {
    const float dj = d[j];
    z[j] = z[j] + alf * dj;
    const float rj = r[j] + alf * q[j];
    r[j] = rj;
    rn += (double)rj * (double)rj;
  }
  rn = block_sum<kSmallThreads>(rn, red);  // every thread read S before this barrier
  const double be = rn / rr;
  const float bef = (float)be;
  for (int64_t j = tid; j < n; j += kSmallThreads) d[j] = -r[j] + bef * d[j];
  if (tid == 0) {
    S->kappa = kap;
    S->alpha = al;
    S->beta = be;
    S->rr = rn;
    S->iters += 1;
    if (rn == 0.0) S->done = 1;
  }
}

// The same iteration over many workgroups (n > kLrSmallCg): after d.q and alpha (lr_dots_kernel,
// lr_finish_kernel kLrCgAlpha), update s and r and take the partials of the new r.r (row 1).
__global__ __launch_bounds__(kThreads) void lr_cg_update_kernel(int64_t n, const float* __restrict__ q,
                                                                const float* __restrict__ d, float* __restrict__ z,
                                                                float* __restrict__ r,
                                                                const LrScalars* __restrict__ S, int first,
                                                                double* __restrict__ part) {
  __shared__ double red[kThreads / 64];
  const bool neg = S->neg != 0;
  double rn = 0.0;
  if (S->done) {
    // CG has stopped: nothing to update
  } else if (neg) {
    if (first)
      for (int64_t j = first_index(); j < n; j += grid_stride()) z[j] = d[j];
  } else {
    const float alf = (float)S->alpha;
    for (int64_t j = first_index(); j < n; j += grid_stride()) {
      z[j] = z[j] + alf * d[j];
      const float rj = r[j] + alf * q[j];
      r[j] = rj;
      rn += (double)rj * (double)rj;
    }
  }
  rn = block_sum<kThreads>(rn, red);
  if (threadIdx.x == 0) part[(size_t)1 * kLrMaxParts + blockIdx.x] = rn;
}

// d = -r + beta d (after lr_finish_kernel kLrCgBeta), unless the curvature test failed.
__global__ __launch_bounds__(kThreads) void lr_cg_direction_kernel(int64_t n, const float* __restrict__ r,
                                                                   float* __restrict__ d,
                                                                   const LrScalars* __restrict__ S) {
  if (S->neg || S->done) return;
  const float bef = (float)S->beta;
  for (int64_t j = first_index(); j < n; j += grid_stride()) d[j] = -r[j] + bef * d[j];
}

// y += a x
__global__ __launch_bounds__(kThreads) void lr_axpy_kernel(int64_t n, float a, const float* __restrict__ x,
                                                           float* __restrict__ y) {
  for (int64_t j = first_index(); j < n; j += grid_stride()) y[j] = y[j] + a * x[j];
}

dim3 grid_for(int64_t count) { return dim3((unsigned)lr_grid(count)); }

}  // namespace

hipError_t launch_lr_link(int64_t m, float* t, const float* xs, float step, const float* c, float* u, float* v,
                          double* part, hipStream_t s) {
  if (m == 0) return hipSuccess;
  hipLaunchKernelGGL(lr_link_kernel, grid_for(m), dim3(kThreads), 0, s, m, t, xs, step, c, u, v, part);
  return hipGetLastError();
}

hipError_t launch_lr_trial(int64_t m, const float* t, const float* xs, double a, const float* c, double* part,
                           hipStream_t s) {
  if (m == 0) return hipSuccess;
  hipLaunchKernelGGL(lr_trial_kernel, grid_for(m), dim3(kThreads), 0, s, m, t, xs, a, c, part);
  return hipGetLastError();
}

hipError_t launch_lr_max_row(int64_t m, const int32_t* row_ptr, uint32_t* longest, hipStream_t s) {
  hipError_t e = launch_zero(longest, sizeof(uint32_t), s);
  if (e != hipSuccess || m <= 0) return e;
  hipLaunchKernelGGL(lr_max_row_kernel, grid_for(m), dim3(kThreads), 0, s, m, row_ptr, longest);
  return hipGetLastError();
}

hipError_t launch_lr_dots(int64_t n, int k, const float* const* x, const float* const* y, int row0, double* part,
                          hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (k < 1 || k > 3 || row0 < 0 || row0 + k > kLrRows) return hipErrorInvalidValue;
  DotArgs a{};
  a.k = k;
  for (int i = 0; i < k; ++i) {
    a.x[i] = x[i];
    a.y[i] = y[i];
  }
  hipLaunchKernelGGL(lr_dots_kernel, grid_for(n), dim3(kThreads), 0, s, n, a, row0, part);
  return hipGetLastError();
}

hipError_t launch_lr_finish(int op, const double* part, int64_t m, int64_t n, LrScalars* S, double a, double lam,
                            hipStream_t s) {
  hipLaunchKernelGGL(lr_finish_kernel, dim3(1), dim3(kThreads), 0, s, op, part, lr_grid(m), lr_grid(n), S, a, lam);
  return hipGetLastError();
}

hipError_t launch_lr_cg_init(int64_t n, const float* g, float* z, float* r, float* d, LrScalars* S,
                             hipStream_t s) {
  hipLaunchKernelGGL(lr_cg_init_kernel, dim3(n > 0 ? (unsigned)lr_grid(n) : 1u), dim3(kThreads), 0, s, n, g, z, r,
                     d, S);
  return hipGetLastError();
}

hipError_t launch_lr_cg_step(int64_t n, const float* q, float* d, float* z, float* r, LrScalars* S, bool first,
                             double* part, hipStream_t s) {
  if (n <= kLrSmallCg) {
    hipLaunchKernelGGL(lr_cg_small_kernel, dim3(1), dim3(kSmallThreads), 0, s, n, q, d, z, r, S, first ? 1 : 0);
    return hipGetLastError();
  }
  const float* x[1] = {d};
  const float* y[1] = {q};
  hipError_t e = launch_lr_dots(n, 1, x, y, 1, part, s);
  if (e != hipSuccess) return e;
  e = launch_lr_finish(kLrCgAlpha, part, 0, n, S, 0.0, 0.0, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lr_cg_update_kernel, grid_for(n), dim3(kThreads), 0, s, n, q, d, z, r, S, first ? 1 : 0,
                     part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_lr_finish(kLrCgBeta, part, 0, n, S, 0.0, 0.0, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lr_cg_direction_kernel, grid_for(n), dim3(kThreads), 0, s, n, r, d, S);
  return hipGetLastError();
}

hipError_t launch_lr_axpy(int64_t n, float a, const float* x, float* y, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(lr_axpy_kernel, grid_for(n), dim3(kThreads), 0, s, n, a, x, y);
  return hipGetLastError();
}

}  // namespace xtvxy
