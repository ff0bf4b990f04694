// Device-side helpers shared by the xtvxy kernels: cross-lane sums built from
// gfx950 DPP and permlane-swap instructions, and row-chunk loads.
//
// Lane movements used (wave64):
//   DPP quad_perm [1,0,3,2] / [2,3,0,1]  lane i reads lane i^1 / i^2
//   DPP row_half_mirror                  lane i reads lane 7-i within its 8-lane half-row
//   DPP row_mirror                       lane i reads lane 15-i within its 16-lane row
//   DPP row_ror:k                        lane i reads lane (i+k) mod 16 within its row
//   v_permlane16_swap(x, y)              -> {x r0, y r0, x r2, y r2}, {x r1, y r1, x r3, y r3}
//   v_permlane32_swap(x, y)              -> {x lo, y lo}, {x hi, y hi}
// (r0..r3 are the 16-lane rows, lo/hi the 32-lane halves of a register.)
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace xtvxy {

typedef float f4 __attribute__((ext_vector_type(4)));

namespace dpp {
constexpr int kXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;
constexpr int kMirror = 0x140;
constexpr int kRor1 = 0x121, kRor2 = 0x122, kRor4 = 0x124, kRor8 = 0x128;
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;  // row_shr:k, lane i reads i-k in its row
constexpr int kBcast15 = 0x142;   // row_bcast:15, rows 1 and 3 (row mask 0xa) read lane 15 of the row before
constexpr int kBcast31 = 0x143;   // row_bcast:31, rows 2 and 3 (row mask 0xc) read lane 31
constexpr int kWaveShl1 = 0x130;  // wave_shl:1, lane i reads lane i+1
constexpr int kWaveShr1 = 0x138;  // wave_shr:1, lane i reads lane i-1
}  // namespace dpp

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// DPP move; lanes without a source lane, or outside the row mask, get `old`. The source
// lanes must be active: call from wavefront-uniform control flow.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_int(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_float(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL, ROWS, 0xf, false));
}

// Lane i gets the maximum of x over lanes 0..i (wavefront-uniform control flow).
__device__ __forceinline__ int wave_max_scan(int x) {
  constexpr int lo = INT32_MIN;
  x = max(x, dpp_int<dpp::kShr1>(lo, x));
  x = max(x, dpp_int<dpp::kShr2>(lo, x));
  x = max(x, dpp_int<dpp::kShr4>(lo, x));
  x = max(x, dpp_int<dpp::kShr8>(lo, x));
  x = max(x, dpp_int<dpp::kBcast15, 0xa>(lo, x));
  x = max(x, dpp_int<dpp::kBcast31, 0xc>(lo, x));
  return x;
}

template <int CTRL, int ROWS>
__device__ __forceinline__ void seg_sum_step(float& x, int key) {
  const float xs = dpp_float<CTRL, ROWS>(0.0f, x);
  const int ks = dpp_int<CTRL, ROWS>(~key, key);  // ~key never equals key
  x += (ks == key) ? xs : 0.0f;
}

// Segmented inclusive sum over a wavefront (wavefront-uniform control flow). Lanes with
// equal `key` must be contiguous (e.g. keys nondecreasing with the lane index); lane i
// gets the sum of x over the lanes j <= i with key_j == key_i. Each step adds the partial
// sum d lanes back when that lane carries the same key: by contiguity, every lane between
// carries it too, so the partial sums of one key never mix with another's.
__device__ __forceinline__ float wave_segmented_sum(float x, int key) {
  seg_sum_step<dpp::kShr1, 0xf>(x, key);
  seg_sum_step<dpp::kShr2, 0xf>(x, key);
  seg_sum_step<dpp::kShr4, 0xf>(x, key);
  seg_sum_step<dpp::kShr8, 0xf>(x, key);
  seg_sum_step<dpp::kBcast15, 0xa>(x, key);
  seg_sum_step<dpp::kBcast31, 0xc>(x, key);
  return x;
}

// x of lanes i and i^16 (aligned 32-lane halves), summed; same value in both lanes.
__device__ __forceinline__ float add_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x of lanes i and i^32, summed; same value in both lanes.
__device__ __forceinline__ float add_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of `width` lanes (power of two, <= 64); every lane of a
// group ends with the same, bitwise identical, total.
__device__ __forceinline__ float group_sum(float x, int width) {
  if (width >= 2) x += dpp_mov<dpp::kXor1>(x);
  if (width >= 4) x += dpp_mov<dpp::kXor2>(x);
  if (width >= 8) x += dpp_mov<dpp::kHalfMirror>(x);
  if (width >= 16) x += dpp_mov<dpp::kMirror>(x);
  if (width >= 32) x = add_xor16(x);
  if (width >= 64) x = add_xor32(x);
  return x;
}

// Sum of x over the lanes that share i mod `stride` (stride a power of two <= 64),
// i.e. over the 64/stride "slots" of a wavefront; every lane gets its class total.
__device__ __forceinline__ float slot_sum(float x, int stride) {
  if (stride <= 1) x += dpp_mov<dpp::kRor1>(x);
  if (stride <= 2) x += dpp_mov<dpp::kRor2>(x);
  if (stride <= 4) x += dpp_mov<dpp::kRor4>(x);
  if (stride <= 8) x += dpp_mov<dpp::kRor8>(x);
  if (stride <= 16) x = add_xor16(x);
  if (stride <= 32) x = add_xor32(x);
  return x;
}

// Eight per-lane partial sums s[0..7] of eight rows that each span the whole
// wavefront, reduced together: the returned value in lane i is the complete sum
// of row i >> 3. 18 lane-exchange instructions for eight rows instead of six
// exchanges per row.
__device__ __forceinline__ float wave_sum8_transposed(const float (&s)[8]) {
  float a[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // halves: lanes 0-31 keep row k, lanes 32-63 row k+4
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s[k]), __float_as_uint(s[k + 4]), false, false);
    a[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  float b[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // 16-lane rows: r0 keeps row k, r1 row k+2, r2 row k+4, r3 row k+6
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[k]), __float_as_uint(a[k + 2]), false, false);
    b[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool upper8 = (threadIdx.x & 8) != 0;  // 8-lane half of a row: the lower keeps b0, the upper b1
  const float keep = upper8 ? b[1] : b[0];
  const float send = upper8 ? b[0] : b[1];
  float c = keep + dpp_mov<dpp::kRor8>(send);
  c += dpp_mov<dpp::kXor1>(c);
  c += dpp_mov<dpp::kXor2>(c);
  c += dpp_mov<dpp::kHalfMirror>(c);
  return c;
}

typedef __attribute__((address_space(3))) unsigned int lds_uint;
typedef __attribute__((address_space(3))) float lds_float;

// Atomic fp32 add to an LDS word. On gfx950 the native LDS float atomic (ds_add_f32) retires
// about 0.33 lanes per clock per CU whatever the address pattern, while a compare-and-swap of
// the word's bits (ds_cmpst_rtn_b32) sustains about 1.9 lanes per clock on scattered
// addresses. A compare-and-swap fails when another lane changed the word first, which on
// skewed (hot-column) patterns happens to most lanes of an instruction and would serialise a
// retry loop; so there is one attempt, and the lanes that lose it use the native atomic.
// `p` must point into LDS.
__device__ __forceinline__ void lds_add_f32(float* p, float v) {
  lds_uint* w = (lds_uint*)p;  // address-space cast: the word lives in LDS
  unsigned int expected = *w;
  if (!__hip_atomic_compare_exchange_strong(w, &expected, __float_as_uint(__uint_as_float(expected) + v),
                                            __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) {
    __builtin_amdgcn_ds_faddf((lds_float*)p, v, 0, 0, false);
  }
}

// `VEC` consecutive floats of row `xr` starting at column `col` when `ok`, else zeros.
// With VEC == 4 the caller guarantees that a chunk lies entirely inside or outside
// the row (n % 4 == 0). The address is clamped instead of branched around, so the
// load is issued unconditionally and the result selected. X is streamed exactly once:
// the loads carry the non-temporal hint.
template <int VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ xr, int64_t col, bool ok, float (&o)[VEC]) {
  const int64_t c = ok ? col : 0;
  if constexpr (VEC == 4) {
    const f4 t = __builtin_nontemporal_load(reinterpret_cast<const f4*>(xr + c));
    o[0] = ok ? t.x : 0.0f;
    o[1] = ok ? t.y : 0.0f;
    o[2] = ok ? t.z : 0.0f;
    o[3] = ok ? t.w : 0.0f;
  } else {
    const float t = __builtin_nontemporal_load(xr + c);
    o[0] = ok ? t : 0.0f;
  }
}

// bf16 storage of X: an element is the upper 16 bits of an fp32 bit pattern.
typedef uint16_t bf16_t;
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

// A chunk of VEC consecutive elements of a row of X as it sits in registers: fp32 values, or
// bf16 kept packed two to a 32-bit word (half the registers of the widened values, so twice the
// rows fit in flight) and widened at each use by one shift or mask. get(k) is element k as fp32.
template <class E, int VEC>
struct XChunk {
  float v[VEC];
  __device__ __forceinline__ float get(int k) const { return v[k]; }
};
template <>
struct XChunk<bf16_t, 8> {
  unsigned int w[4];
  __device__ __forceinline__ float get(int k) const { return (k & 1) ? bf16_hi(w[k >> 1]) : bf16_lo(w[k >> 1]); }
  // the words become opaque to the compiler: values widened from them before are not reused
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(w[i]));
  }
};
template <>
struct XChunk<bf16_t, 1> {
  unsigned int w;
  __device__ __forceinline__ float get(int) const { return bf16_lo(w); }
  __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(w)); }
};

// fp16 storage of X: IEEE binary16, kept packed like bf16 and widened exactly (every fp16 value,
// subnormals, infinities and NaN included, is an fp32 value) by a conversion at each use.
typedef _Float16 f16_t;
__device__ __forceinline__ float f16_lo(unsigned int w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(unsigned int w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}
template <>
struct XChunk<f16_t, 8> {
  unsigned int w[4];
  __device__ __forceinline__ float get(int k) const { return (k & 1) ? f16_hi(w[k >> 1]) : f16_lo(w[k >> 1]); }
  // the words become opaque to the compiler: values widened from them before are not reused
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(w[i]));
  }
};
template <>
struct XChunk<f16_t, 1> {
  unsigned int w;
  __device__ __forceinline__ float get(int) const { return f16_lo(w); }
  __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(w)); }
};

// Chunk of row `xr` from column `col` when `ok`, else zeros. fp32 rows take load_chunk; bf16 and
// fp16 rows take one 16-byte load of 8 elements (VEC == 8: the caller guarantees 16-byte
// alignment and n % 8 == 0) or one 2-byte load (VEC == 1). Clamped address, unconditional non-temporal load,
// as in load_chunk.
template <class E, int VEC>
__device__ __forceinline__ void load_x(const E* __restrict__ xr, int64_t col, bool ok, XChunk<E, VEC>& o) {
  if constexpr (sizeof(E) == 4) {
    load_chunk<VEC>(reinterpret_cast<const float*>(xr), col, ok, o.v);
  } else {
    const int64_t c = ok ? col : 0;
    if constexpr (VEC == 8) {
      const u4 t = __builtin_nontemporal_load(reinterpret_cast<const u4*>(xr + c));
      o.w[0] = ok ? t.x : 0u;
      o.w[1] = ok ? t.y : 0u;
      o.w[2] = ok ? t.z : 0u;
      o.w[3] = ok ? t.w : 0u;
    } else {
      static_assert(VEC == 1, "16-bit rows load 8 or 1 elements");
      const unsigned int h = __builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(xr + c));
      o.w = ok ? h : 0u;
    }
  }
}

// Stored values of a CSR matrix: fp32, or bf16 (VT = bf16_t: the upper 16 bits of an fp32 bit
// pattern, widened exactly as it is loaded). Every load returns fp32.
template <class VT>
__device__ __forceinline__ float csr_value(const void* values, uint32_t p) {
  if constexpr (sizeof(VT) == 4) {
    return static_cast<const float*>(values)[p];
  } else {
    return __uint_as_float((uint32_t)static_cast<const bf16_t*>(values)[p] << 16);
  }
}
// Values q .. q+3 (q a multiple of 4) by one load: 16 bytes of fp32 (16-byte aligned values) or
// 8 bytes of bf16 (8-byte aligned values); the caller guarantees the alignment.
typedef unsigned int vu2 __attribute__((ext_vector_type(2)));
template <class VT>
__device__ __forceinline__ void csr_value_quad(const void* values, uint32_t q, float* o) {
  if constexpr (sizeof(VT) == 4) {
    const f4 vv = *reinterpret_cast<const f4*>(static_cast<const float*>(values) + q);
    o[0] = vv.x;
    o[1] = vv.y;
    o[2] = vv.z;
    o[3] = vv.w;
  } else {
    const vu2 w = *reinterpret_cast<const vu2*>(static_cast<const bf16_t*>(values) + q);
    o[0] = bf16_lo(w.x);
    o[1] = bf16_hi(w.x);
    o[2] = bf16_lo(w.y);
    o[3] = bf16_hi(w.y);
  }
}

}  // namespace xtvxy
