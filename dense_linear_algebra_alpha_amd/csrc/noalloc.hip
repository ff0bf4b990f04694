// Allocation-free form of the dense fused entry point, for callers that cannot allocate device
// memory or hand the library a workspace (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation). The partial sums that xtvxy_dense_f32 keeps in the caller's
// workspace live here in `scratch`, a fixed-size array of this library in device memory: each GPU
// the library runs on holds its own copy until the process ends. The host side of the program
// cannot use the array's name as a device address (it names a host-side stand-in), so the array's
// address on each device is looked up once with hipGetSymbolAddress, with that device current, and
// only that address is passed to the kernels and the fill kernel that clears the exchange slots.
#include <mutex>

#include "internal.h"

namespace xtvxy {
namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;  // 32 MiB per device
constexpr int kMaxScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device (null: not looked up)

// Address of this device's `scratch` (the current device), looked up on the first call.
xtvxy_status scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return XTVXY_ERROR_LAUNCH;
  if (dev < 0 || dev >= kMaxScratchDevices) return XTVXY_ERROR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return XTVXY_ERROR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return XTVXY_SUCCESS;
}

}  // namespace
}  // namespace xtvxy

extern "C" xtvxy_status xtvxy_dense_f32_noalloc_max_workspace(size_t* bytes) {
  if (!bytes) return XTVXY_ERROR_NULL_POINTER;
  *bytes = xtvxy::kScratchBytes;
  return XTVXY_SUCCESS;
}

extern "C" xtvxy_status xtvxy_dense_f32_noalloc(int64_t m, int64_t n, float alpha, const float* X, int64_t ldx,
                                                const float* v, const float* y, float beta, const float* z,
                                                float* out, hipStream_t stream) {
  using namespace xtvxy;
  // the workspace xtvxy_dense_f32 would need for this shape (argument errors are reported here
  // or by the call below, before anything is enqueued)
  size_t need = 0;
  xtvxy_status st = xtvxy_dense_f32_workspace_size(m, n, ldx, &need);
  if (st != XTVXY_SUCCESS) return st;
  if (need > kScratchBytes) return XTVXY_ERROR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_on_current_device(&ws);
    if (st != XTVXY_SUCCESS) return st;
  }
  return xtvxy_dense_f32(m, n, alpha, X, ldx, v, y, beta, z, out, ws, need > 0 ? kScratchBytes : 0, stream);
}
