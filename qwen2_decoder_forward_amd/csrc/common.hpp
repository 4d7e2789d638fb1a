// Shared host/device helpers of the q2 library: status handling, tensor
// descriptor checks, bf16 conversion, wave-level reductions and MFMA types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "q2.h"

namespace q2 {

// ---------------------------------------------------------------- errors

q2_status fail(q2_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

#define Q2_HIP(expr)                                                                  \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess)                                                             \
      return ::q2::fail(Q2_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));      \
  } while (0)

#define Q2_CHECK(cond, st, ...)                     \
  do {                                              \
    if (!(cond)) return ::q2::fail(st, __VA_ARGS__); \
  } while (0)

#define Q2_TRY(expr)                 \
  do {                               \
    q2_status s_ = (expr);           \
    if (s_ != Q2_OK) return s_;      \
  } while (0)

// Status of the last kernel launch on this thread.
q2_status check_launch(const char* what);

// ---------------------------------------------------------------- tensors

inline int64_t dtype_size(int32_t dt) {
  return dt == Q2_F32 ? 4 : dt == Q2_BF16 ? 2 : dt == Q2_I64 ? 8 : dt == Q2_U8 ? 1 : 0;
}
inline bool dtype_valid(int32_t dt) { return dt == Q2_F32 || dt == Q2_BF16 || dt == Q2_I64 || dt == Q2_U8; }
inline bool is_float(int32_t dt) { return dt == Q2_F32 || dt == Q2_BF16; }

inline int64_t numel(const q2_tensor& t) {
  int64_t n = 1;
  for (int i = 0; i < t.ndim; ++i) n *= t.shape[i];
  return n;
}

// Validates the descriptor itself (pointer, rank, dtype, non-negative sizes).
q2_status check_desc(const q2_tensor* t, const char* name);
bool same_shape(const q2_tensor& a, const q2_tensor& b);
bool is_contiguous(const q2_tensor& t);

// View of a tensor as [rows, cols] where cols is the last dim (stride 1) and
// the outer dims collapse to one row stride.  Fails if the outer dims cannot
// be expressed with one stride or the last dim is not contiguous.
struct Rows {
  char* data;
  int64_t rows, cols, ld;   // ld in elements
  int32_t dtype;
};
q2_status as_rows(const q2_tensor* t, const char* name, Rows* out);

__host__ __device__ inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ---------------------------------------------------------------- device helpers

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;

// The 16 bytes of a uint4 as an MFMA operand of eight bf16 values.
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short short4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;

// bf16 <-> float.  Widening is exact; narrowing rounds to nearest, ties to even.
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// (gfx950 converts in hardware: v_cvt_pk_bf16_f32, round to nearest even,
// NaN stays NaN.)
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float float2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const float2_hw f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_hw));
}
__device__ __forceinline__ uint16_t f2bf(float f) { return static_cast<uint16_t>(pack_bf2(f, 0.f)); }
__device__ __forceinline__ float round_bf(float f) { return bf2f(f2bf(f)); }

// Storage traits: float (no rounding) and bf16 (uint16_t bit patterns).
template <typename T> struct St;
template <> struct St<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static __device__ __forceinline__ float rnd(float v) { return v; }
};
template <> struct St<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, float v) { *p = f2bf(v); }
  static __device__ __forceinline__ float rnd(float v) { return round_bf(v); }
};

// Sum / max over the 64 lanes of a wave (result in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// silu(g) = g / (1 + exp(-g)) in float32.
__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// Total order key for float maximum with lowest-index tie-break:
// key = (ordered bits of v) << 32 | ~index.  Larger key = better.  -0 and +0
// compare equal (both map to +0).
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint64_t>(~idx);
}
__device__ __forceinline__ float argmax_key_value(uint64_t key) {
  uint32_t u = static_cast<uint32_t>(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint32_t argmax_key_index(uint64_t key) { return ~static_cast<uint32_t>(key); }

__host__ __device__ inline int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

}  // namespace q2
