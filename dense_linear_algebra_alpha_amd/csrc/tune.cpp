// Empirical tuning of the launch plan, beside the analytical model.
//
// "On optimizing machine learning workloads via kernel fusion" (abstract) chooses launch
// parameters with an analytical model of the input and the GPU, and calls its choice
// near-optimal. The tuner measures that claim on the actual input: it times the fused call
// under a grid of candidate plans (every layout, tile shape, window and grid size the kernels
// accept for the shape, the model's own plan among them), re-times the fastest few together with
// the model's plan, and reports the best plan and the model's plan with their measured times.
// The model's regret is model_seconds / best_seconds - 1.
//
// Results are cached per (device, kind, shape) for the life of the process and can be saved to
// and loaded from a text file, one plan per line. The tuner is a set-up tool: it allocates its
// own workspace (the largest any candidate needs), synchronises the stream, and leaves in `out`
// the result of the last call it timed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "internal.h"

using namespace xtvxy;

namespace {

constexpr int kWarmup = 5;
constexpr int kFinalists = 6;  // re-timed together with the model's plan

struct Key {
  std::string device;
  int32_t kind;  // 0 dense fp32, 1 csr fp32 values, 2 dense bf16, 3 dense fp16, 4 csr bf16 values
  int64_t m, n, k;  // k: ldx (dense) or nnz (csr)
  int32_t aligned;
  bool operator<(const Key& o) const {
    return std::tie(device, kind, m, n, k, aligned) < std::tie(o.device, o.kind, o.m, o.n, o.k, o.aligned);
  }
};

std::mutex g_mutex;
std::map<Key, xtvxy_tune_report> g_cache;

xtvxy_status device_key(std::string* out) {
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return XTVXY_ERROR_LAUNCH;
  char buf[320];
  std::snprintf(buf, sizeof buf, "%s:%d", prop.gcnArchName, prop.multiProcessorCount);
  for (char* c = buf; *c; ++c)
    if (*c == ' ') *c = '_';
  *out = buf;
  return XTVXY_SUCCESS;
}

xtvxy_device_info current_info(xtvxy_status* st) {
  xtvxy_device_info d{};
  *st = xtvxy_get_device_info(-1, &d);
  return d;
}

int next_pow2(int64_t x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

std::vector<xtvxy_launch_params> dense_candidates(int64_t m, int64_t n, int64_t ldx, int vec,
                                                  const xtvxy_device_info& d, int elem_bytes) {
  std::vector<xtvxy_launch_params> out;
  auto add = [&](xtvxy_launch_params p) {
    p.block_threads = kBlock;
    p.vec = vec;
    p.rows_per_unit = 0;
    if (complete_dense(m, n, ldx, d, &p, elem_bytes) == XTVXY_SUCCESS) out.push_back(p);
  };
  const int cus = d.compute_units;
  for (int chunks : {1, 2, 4}) {  // wave rows
    const int lanes = next_pow2(ceil_div(n, (int64_t)vec * chunks));
    for (int lpr : {lanes, lanes * 2}) {
      if (lpr > 64) continue;
      for (int k : {1, 2, 4, 8, 16}) {
        xtvxy_launch_params p{};
        p.kernel = XTVXY_DENSE_WAVE_ROWS;
        p.chunks = chunks;
        p.lanes_per_row = lpr;
        p.group = 1;
        p.grid = (int64_t)cus * k;
        add(p);
      }
    }
  }
  for (int chunks : {1, 2, 4, 8}) {  // block rows
    for (int k : {1, 2, 4, 8}) {
      xtvxy_launch_params p{};
      p.kernel = XTVXY_DENSE_BLOCK_ROWS;
      p.chunks = chunks;
      p.group = 1;
      p.grid = (int64_t)cus * k;
      add(p);
    }
  }
  if (n > (int64_t)kBlock * vec) {  // group rows: the smallest group for each chunk count, and twice it
    for (int chunks : {1, 2, 4, 8}) {
      const int64_t g0 = ceil_div(n, (int64_t)kBlock * vec * chunks);
      for (int64_t g : {g0, 2 * g0}) {
        if (g < 2 || g > kGroupMaxMembers) continue;
        for (int k : {1, 2}) {
          xtvxy_launch_params p{};
          p.kernel = XTVXY_DENSE_GROUP_ROWS;
          p.chunks = chunks;
          p.group = (int32_t)g;
          p.grid = std::max<int64_t>(g, (int64_t)cus * k / g * g);
          add(p);
        }
      }
    }
  }
  return out;
}

std::vector<xtvxy_launch_params> csr_candidates(int64_t m, int64_t n, int64_t nnz, const xtvxy_device_info& d,
                                                const xtvxy_launch_params& model) {
  std::vector<xtvxy_launch_params> out;
  const int cus = d.compute_units;
  std::vector<std::pair<int32_t, int32_t>> windows;  // (output window, y window)
  auto win = [&](int64_t w, int64_t yw) {
    w = std::min<int64_t>(w, n);
    yw = std::min<int64_t>(yw, n);
    const std::pair<int32_t, int32_t> p{(int32_t)w, (int32_t)yw};
    if (std::find(windows.begin(), windows.end(), p) == windows.end()) windows.push_back(p);
  };
  win(model.lds_window, model.y_window);
  if ((int64_t)n * 8 <= 64 * 1024) {
    win(n, n);
    win(n, 0);
  } else {
    for (int64_t w : {4096, 8192, 12288, 16384, 24576}) {
      win(w, 0);
      win(w, w / 3);
    }
  }
  // (kernel, threads, entries per thread): workgroup tiles, and for narrow matrices (whose
  // windows hold all of n) the wavefront kernel too
  struct Shape {
    int32_t kernel, threads, ept;
  };
  std::vector<Shape> shapes = {{XTVXY_CSR_TILES, 256, 4}, {XTVXY_CSR_TILES, 256, 8}, {XTVXY_CSR_TILES, 512, 8}};
  if ((int64_t)n * 8 <= 64 * 1024)
    for (int32_t t : {256, 512, 1024}) shapes.push_back({XTVXY_CSR_WAVES, t, 8});
  for (const auto& sh : shapes) {
    for (const auto& wy : windows) {
      for (int32_t bc : {0, 16384, 32768}) {
        if (wy.first >= n && bc != 0) continue;
        if (sh.kernel == XTVXY_CSR_WAVES && wy.first < n) continue;
        for (int k : {1, 2, 3, 4, 6, 8}) {
          if ((int64_t)sh.threads * k > 2048) continue;  // threads per CU
          xtvxy_launch_params p{};
          p.kernel = sh.kernel;
          p.vec = 1;
          p.chunks = 1;
          p.group = 1;
          p.block_threads = sh.threads;
          p.entries_per_thread = sh.ept;
          p.lds_window = wy.first;
          p.y_window = wy.second;
          p.bin_columns = bc;
          p.grid = (int64_t)cus * k;
          if (complete_csr(m, n, nnz, d, &p) == XTVXY_SUCCESS) out.push_back(p);
        }
      }
    }
  }
  return out;
}

bool same_plan(const xtvxy_launch_params& a, const xtvxy_launch_params& b) {
  return a.kernel == b.kernel && a.vec == b.vec && a.block_threads == b.block_threads &&
         a.lanes_per_row == b.lanes_per_row && a.chunks == b.chunks && a.group == b.group && a.grid == b.grid &&
         a.rows_per_unit == b.rows_per_unit && a.entries_per_thread == b.entries_per_thread &&
         a.lds_window == b.lds_window && a.y_window == b.y_window && a.bin_columns == b.bin_columns;
}

// Mean seconds per call of `call` over `repeats` calls after kWarmup, from HIP events on the stream.
// Returns a negative value when the call reports an error (the candidate is skipped).
template <class F>
double time_calls(F call, int repeats, hipStream_t s, hipEvent_t e0, hipEvent_t e1, xtvxy_status* err) {
  *err = XTVXY_SUCCESS;
  for (int i = 0; i < kWarmup; ++i) {
    const xtvxy_status st = call();
    if (st != XTVXY_SUCCESS) {
      *err = st;
      return -1.0;
    }
  }
  if (hipEventRecord(e0, s) != hipSuccess) {
    *err = XTVXY_ERROR_LAUNCH;
    return -1.0;
  }
  for (int i = 0; i < repeats; ++i) {
    const xtvxy_status st = call();
    if (st != XTVXY_SUCCESS) {
      *err = st;
      return -1.0;
    }
  }
  float ms = 0.0f;
  if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
      hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
    *err = XTVXY_ERROR_LAUNCH;
    return -1.0;
  }
  return (double)ms * 1e-3 / repeats;
}

// Times every candidate, re-times the best few with the model's plan, fills the report.
template <class Run>
xtvxy_status tune(const std::vector<xtvxy_launch_params>& cands, const xtvxy_launch_params& model, Run run,
                  int repeats, hipStream_t s, xtvxy_tune_report* rep) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return XTVXY_ERROR_LAUNCH;
  }
  std::vector<std::pair<double, size_t>> timed;
  xtvxy_status fatal = XTVXY_SUCCESS;
  for (size_t i = 0; i < cands.size() && fatal == XTVXY_SUCCESS; ++i) {
    xtvxy_status err;
    const double t = time_calls([&] { return run(cands[i]); }, repeats, s, e0, e1, &err);
    if (err == XTVXY_ERROR_LAUNCH || err == XTVXY_ERROR_LIBRARY) fatal = err;
    if (t > 0.0) timed.push_back({t, i});
  }
  if (fatal == XTVXY_SUCCESS && timed.empty()) fatal = XTVXY_ERROR_INVALID_VALUE;
  if (fatal == XTVXY_SUCCESS) {
    std::sort(timed.begin(), timed.end());
    std::vector<xtvxy_launch_params> finals;
    for (size_t i = 0; i < timed.size() && (int)finals.size() < kFinalists; ++i) finals.push_back(cands[timed[i].second]);
    bool have_model = false;
    for (const auto& f : finals) have_model = have_model || same_plan(f, model);
    if (!have_model) finals.push_back(model);
    double best = 1e300, model_t = -1.0;
    size_t best_i = 0;
    for (size_t i = 0; i < finals.size() && fatal == XTVXY_SUCCESS; ++i) {
      xtvxy_status err;
      const double t = time_calls([&] { return run(finals[i]); }, 3 * repeats, s, e0, e1, &err);
      if (err == XTVXY_ERROR_LAUNCH || err == XTVXY_ERROR_LIBRARY) fatal = err;
      if (t <= 0.0) continue;
      if (same_plan(finals[i], model)) model_t = t;
      if (t < best) {
        best = t;
        best_i = i;
      }
    }
    if (fatal == XTVXY_SUCCESS && model_t <= 0.0) fatal = XTVXY_ERROR_INVALID_VALUE;  // the model's plan failed
    if (fatal == XTVXY_SUCCESS) {
      rep->model = model;
      rep->best = finals[best_i];
      rep->model_seconds = model_t;
      rep->best_seconds = best;
      rep->candidates = (int32_t)cands.size();
      rep->from_cache = 0;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return fatal;
}

struct DeviceBuffer {
  void* p = nullptr;
  ~DeviceBuffer() {
    if (p) (void)hipFree(p);
  }
};

bool cache_get(const Key& k, xtvxy_tune_report* rep) {
  std::lock_guard<std::mutex> lock(g_mutex);
  auto it = g_cache.find(k);
  if (it == g_cache.end()) return false;
  *rep = it->second;
  rep->from_cache = 1;
  return true;
}

void cache_put(const Key& k, const xtvxy_tune_report& rep) {
  std::lock_guard<std::mutex> lock(g_mutex);
  g_cache[k] = rep;
}

// One cache line: kind device m n k aligned, then the plan fields of best and model, then the times.
constexpr int kPlanInts = 13;
void plan_to_ints(const xtvxy_launch_params& p, long long* v) {
  const long long a[kPlanInts] = {p.kernel,     p.vec,        p.block_threads,      p.lanes_per_row, p.chunks,
                                  p.group,      p.grid,       p.rows_per_unit,      p.entries_per_thread,
                                  p.lds_window, p.y_window,   p.bin_columns,        p.workspace_bytes};
  std::memcpy(v, a, sizeof a);
}
void ints_to_plan(const long long* v, xtvxy_launch_params* p) {
  std::memset(p, 0, sizeof(*p));
  p->kernel = (int32_t)v[0];
  p->vec = (int32_t)v[1];
  p->block_threads = (int32_t)v[2];
  p->lanes_per_row = (int32_t)v[3];
  p->chunks = (int32_t)v[4];
  p->group = (int32_t)v[5];
  p->grid = v[6];
  p->rows_per_unit = v[7];
  p->entries_per_thread = (int32_t)v[8];
  p->lds_window = (int32_t)v[9];
  p->y_window = (int32_t)v[10];
  p->bin_columns = (int32_t)v[11];
  p->workspace_bytes = v[12];
}

}  // namespace

extern "C" {

static xtvxy_status dense_tune(int64_t m, int64_t n, float alpha, const void* X, int64_t ldx, const float* v,
                               const float* y, float beta, const float* z, float* out, int32_t repeats,
                               hipStream_t stream, xtvxy_tune_report* report, int elem_bytes, bool f16 = false) {
  if (!report) return XTVXY_ERROR_NULL_POINTER;
  if (repeats < 1 || repeats > 10000) return XTVXY_ERROR_INVALID_VALUE;
  bool quick = false;
  xtvxy_status st = check_dense_args(m, n, alpha, X, ldx, v, y, beta, z, out, &quick, elem_bytes);
  if (st != XTVXY_SUCCESS) return st;
  if (quick) return XTVXY_ERROR_INVALID_VALUE;  // nothing to tune: the call reads no X
  const int aligned = (reinterpret_cast<uintptr_t>(X) % 16 == 0) ? 1 : 0;
  Key key;
  if ((st = device_key(&key.device)) != XTVXY_SUCCESS) return st;
  key.kind = f16 ? 3 : elem_bytes == 2 ? 2 : 0;
  key.m = m;
  key.n = n;
  key.k = ldx;
  key.aligned = aligned;
  if (cache_get(key, report)) return XTVXY_SUCCESS;
  const xtvxy_device_info d = current_info(&st);
  if (st != XTVXY_SUCCESS) return st;
  xtvxy_launch_params model;
  st = elem_bytes == 2 ? xtvxy_dense_bf16_plan(m, n, ldx, aligned, nullptr, &model)
                       : xtvxy_dense_f32_plan(m, n, ldx, aligned, nullptr, &model);
  if (st != XTVXY_SUCCESS) return st;
  std::vector<xtvxy_launch_params> cands = dense_candidates(m, n, ldx, model.vec, d, elem_bytes);
  size_t ws_bytes = (size_t)model.workspace_bytes;
  for (const auto& c : cands) ws_bytes = std::max(ws_bytes, (size_t)c.workspace_bytes);
  DeviceBuffer ws;
  if (ws_bytes > 0 && hipMalloc(&ws.p, ws_bytes) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  auto run = [&](const xtvxy_launch_params& p) {
    if (f16)
      return xtvxy_dense_f16_ex(m, n, alpha, static_cast<const uint16_t*>(X), ldx, v, y, beta, z, out, ws.p,
                                ws_bytes, stream, &p);
    if (elem_bytes == 2)
      return xtvxy_dense_bf16_ex(m, n, alpha, static_cast<const uint16_t*>(X), ldx, v, y, beta, z, out, ws.p,
                                 ws_bytes, stream, &p);
    return xtvxy_dense_f32_ex(m, n, alpha, static_cast<const float*>(X), ldx, v, y, beta, z, out, ws.p, ws_bytes,
                              stream, &p);
  };
  xtvxy_tune_report rep{};
  if ((st = tune(cands, model, run, repeats, stream, &rep)) != XTVXY_SUCCESS) return st;
  cache_put(key, rep);
  *report = rep;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_dense_f32_tune(int64_t m, int64_t n, float alpha, const float* X, int64_t ldx, const float* v,
                                  const float* y, float beta, const float* z, float* out, int32_t repeats,
                                  hipStream_t stream, xtvxy_tune_report* report) {
  return dense_tune(m, n, alpha, X, ldx, v, y, beta, z, out, repeats, stream, report, 4);
}

xtvxy_status xtvxy_dense_bf16_tune(int64_t m, int64_t n, float alpha, const uint16_t* X, int64_t ldx,
                                   const float* v, const float* y, float beta, const float* z, float* out,
                                   int32_t repeats, hipStream_t stream, xtvxy_tune_report* report) {
  return dense_tune(m, n, alpha, X, ldx, v, y, beta, z, out, repeats, stream, report, 2);
}

xtvxy_status xtvxy_dense_f16_tune(int64_t m, int64_t n, float alpha, const uint16_t* X, int64_t ldx,
                                  const float* v, const float* y, float beta, const float* z, float* out,
                                  int32_t repeats, hipStream_t stream, xtvxy_tune_report* report) {
  return dense_tune(m, n, alpha, X, ldx, v, y, beta, z, out, repeats, stream, report, 2, true);
}

// CSR with fp32 (value_bytes 4) or bf16 (2) values; bf16 values take the tile and wavefront
// candidates only (the row-class kernel reads fp32 values).
static xtvxy_status csr_tune(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                             const int32_t* col_idx, const void* values, int value_bytes, const float* v,
                             const float* y, float beta, const float* z, float* out, int32_t repeats,
                             hipStream_t stream, xtvxy_tune_report* report) {
  if (!report) return XTVXY_ERROR_NULL_POINTER;
  if (repeats < 1 || repeats > 10000) return XTVXY_ERROR_INVALID_VALUE;
  bool quick = false;
  xtvxy_status st = check_csr_args(m, n, nnz, alpha, row_ptr, col_idx, static_cast<const float*>(values), v, y,
                                   beta, z, out, &quick, value_bytes);
  if (st != XTVXY_SUCCESS) return st;
  if (quick) return XTVXY_ERROR_INVALID_VALUE;
  Key key;
  if ((st = device_key(&key.device)) != XTVXY_SUCCESS) return st;
  key.kind = value_bytes == 2 ? 4 : 1;
  key.m = m;
  key.n = n;
  key.k = nnz;
  key.aligned = (reinterpret_cast<uintptr_t>(values) % 16 == 0 && reinterpret_cast<uintptr_t>(col_idx) % 16 == 0);
  if (cache_get(key, report)) return XTVXY_SUCCESS;
  const xtvxy_device_info d = current_info(&st);
  if (st != XTVXY_SUCCESS) return st;
  xtvxy_launch_params model;
  if ((st = xtvxy_csr_f32_plan(m, n, nnz, nullptr, &model)) != XTVXY_SUCCESS) return st;
  std::vector<xtvxy_launch_params> cands = csr_candidates(m, n, nnz, d, model);
  if (value_bytes == 2)
    cands.erase(std::remove_if(cands.begin(), cands.end(),
                               [](const xtvxy_launch_params& c) { return c.kernel == XTVXY_CSR_ROWS; }),
                cands.end());
  size_t ws_bytes = (size_t)model.workspace_bytes;
  for (const auto& c : cands) ws_bytes = std::max(ws_bytes, (size_t)c.workspace_bytes);
  DeviceBuffer ws;
  if (ws_bytes > 0 && hipMalloc(&ws.p, ws_bytes) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  auto run = [&](const xtvxy_launch_params& p) {
    if (value_bytes == 2)
      return xtvxy_csr_bf16_ex(m, n, nnz, alpha, row_ptr, col_idx, static_cast<const uint16_t*>(values), v, y, beta,
                               z, out, ws.p, ws_bytes, stream, &p);
    return xtvxy_csr_f32_ex(m, n, nnz, alpha, row_ptr, col_idx, static_cast<const float*>(values), v, y, beta, z,
                            out, ws.p, ws_bytes, stream, &p);
  };
  xtvxy_tune_report rep{};
  if ((st = tune(cands, model, run, repeats, stream, &rep)) != XTVXY_SUCCESS) return st;
  cache_put(key, rep);
  *report = rep;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_csr_f32_tune(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                                const int32_t* col_idx, const float* values, const float* v, const float* y,
                                float beta, const float* z, float* out, int32_t repeats, hipStream_t stream,
                                xtvxy_tune_report* report) {
  return csr_tune(m, n, nnz, alpha, row_ptr, col_idx, values, 4, v, y, beta, z, out, repeats, stream, report);
}

xtvxy_status xtvxy_csr_bf16_tune(int64_t m, int64_t n, int64_t nnz, float alpha, const int32_t* row_ptr,
                                 const int32_t* col_idx, const uint16_t* values, const float* v, const float* y,
                                 float beta, const float* z, float* out, int32_t repeats, hipStream_t stream,
                                 xtvxy_tune_report* report) {
  return csr_tune(m, n, nnz, alpha, row_ptr, col_idx, values, 2, v, y, beta, z, out, repeats, stream, report);
}

xtvxy_status xtvxy_tune_cache_lookup(int32_t kind, int64_t m, int64_t n, int64_t k, int32_t aligned,
                                     xtvxy_tune_report* report, int32_t* found) {
  if (!report || !found) return XTVXY_ERROR_NULL_POINTER;
  if (kind < 0 || kind > 4) return XTVXY_ERROR_INVALID_VALUE;
  Key key;
  const xtvxy_status st = device_key(&key.device);
  if (st != XTVXY_SUCCESS) return st;
  key.kind = kind;
  key.m = m;
  key.n = n;
  key.k = k;
  key.aligned = aligned ? 1 : 0;
  *found = cache_get(key, report) ? 1 : 0;
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_tune_cache_clear(void) {
  std::lock_guard<std::mutex> lock(g_mutex);
  g_cache.clear();
  return XTVXY_SUCCESS;
}

xtvxy_status xtvxy_tune_cache_save(const char* path) {
  if (!path) return XTVXY_ERROR_NULL_POINTER;
  std::FILE* f = std::fopen(path, "w");
  if (!f) return XTVXY_ERROR_INVALID_VALUE;
  std::lock_guard<std::mutex> lock(g_mutex);
  std::fprintf(f, "# xtvxy tune cache v1: device kind m n k aligned | best plan | model plan | best_s model_s cands\n");
  for (const auto& kv : g_cache) {
    const Key& k = kv.first;
    const xtvxy_tune_report& r = kv.second;
    long long b[kPlanInts], mo[kPlanInts];
    plan_to_ints(r.best, b);
    plan_to_ints(r.model, mo);
    std::fprintf(f, "%s %d %lld %lld %lld %d", k.device.c_str(), k.kind, (long long)k.m, (long long)k.n,
                 (long long)k.k, k.aligned);
    for (long long x : b) std::fprintf(f, " %lld", x);
    for (long long x : mo) std::fprintf(f, " %lld", x);
    std::fprintf(f, " %.9e %.9e %d\n", r.best_seconds, r.model_seconds, r.candidates);
  }
  const bool ok = std::fclose(f) == 0;
  return ok ? XTVXY_SUCCESS : XTVXY_ERROR_INVALID_VALUE;
}

xtvxy_status xtvxy_tune_cache_load(const char* path) {
  if (!path) return XTVXY_ERROR_NULL_POINTER;
  std::FILE* f = std::fopen(path, "r");
  if (!f) return XTVXY_ERROR_INVALID_VALUE;
  std::vector<std::pair<Key, xtvxy_tune_report>> entries;
  char line[4096];
  bool bad = false;
  while (std::fgets(line, sizeof line, f)) {
    if (line[0] == '#' || line[0] == '\n') continue;
    char dev[256];
    int kind = 0, aligned = 0, cands = 0, used = 0;
    long long m = 0, n = 0, k = 0;
    if (std::sscanf(line, "%255s %d %lld %lld %lld %d%n", dev, &kind, &m, &n, &k, &aligned, &used) != 6) {
      bad = true;
      break;
    }
    const char* p = line + used;
    long long vals[2 * kPlanInts];
    for (int i = 0; i < 2 * kPlanInts && !bad; ++i) {
      int u = 0;
      if (std::sscanf(p, " %lld%n", &vals[i], &u) != 1) bad = true;
      p += u;
    }
    double best_s = 0, model_s = 0;
    if (!bad && std::sscanf(p, " %lf %lf %d", &best_s, &model_s, &cands) != 3) bad = true;
    if (bad || kind < 0 || kind > 4 || m < 0 || n < 0 || k < 0 || !(best_s > 0) || !(model_s > 0)) {
      bad = true;
      break;
    }
    Key key{dev, kind, m, n, k, aligned ? 1 : 0};
    xtvxy_tune_report r{};
    ints_to_plan(vals, &r.best);
    ints_to_plan(vals + kPlanInts, &r.model);
    r.best_seconds = best_s;
    r.model_seconds = model_s;
    r.candidates = cands;
    entries.push_back({key, r});
  }
  std::fclose(f);
  if (bad) return XTVXY_ERROR_INVALID_VALUE;  // nothing is taken from a malformed file
  std::lock_guard<std::mutex> lock(g_mutex);
  for (const auto& e : entries) g_cache[e.first] = e.second;
  return XTVXY_SUCCESS;
}

}  // extern "C"
