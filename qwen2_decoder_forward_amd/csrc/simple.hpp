// Launchers for the memory-bound operators (ops.hip), shared by the operator
// entry points and the model driver.
#pragma once

#include "common.hpp"

namespace q2 {

// out[m, :] = weight[ids[b, t0 + t], :] for m = b * T + t (ids strides in elements).
// Rows whose id is outside [0, V) are zero-filled.  With `sq` (bf16 only) it
// also writes each row's sums of squares per 16-feature tile, sq[m * sq_ld + f/16].
template <typename T>
q2_status launch_embedding(T* out, int64_t ldo, const int64_t* ids, int64_t ids_bs, int64_t ids_ts, int B, int Tn,
                           const T* weight, int64_t ldw, int V, int H, hipStream_t s, float* sq = nullptr,
                           int64_t sq_ld = 0);

// RMSNorm of `rows` rows; input row r is in + r*ldi.
template <typename T>
q2_status launch_rmsnorm(T* out, int64_t ldo, const T* in, int64_t ldi, const T* w, int rows, int H, float eps,
                         hipStream_t s);

// c = a + b and out = silu(gate) * up over [rows, cols] with row strides.
template <typename T>
q2_status launch_add(T* c, int64_t ldc, const T* a, int64_t lda, const T* b, int64_t ldb, int64_t rows, int cols,
                     hipStream_t s);
template <typename T>
q2_status launch_swiglu(T* o, int64_t ldo, const T* g, int64_t ldg, const T* u, int64_t ldu, int64_t rows, int cols,
                        hipStream_t s);

// cos/sin of pos * theta^(-2j/d) computed in float64, rounded to float32.
__device__ __forceinline__ float2 rope_cs(int64_t pos, int j, int d, float theta) {
  const double inv_freq = pow(static_cast<double>(theta), (-2.0 * j) / d);
  const double ang = static_cast<double>(pos) * inv_freq;
  return make_float2(static_cast<float>(cos(ang)), static_cast<float>(sin(ang)));
}

// table[p * (d/2) + j] = rope_cs(p, j) for p < npos.
q2_status launch_rope_table(float2* table, int npos, int d, float theta, hipStream_t s);

// Row gather used to pack weights: dst row map(s) <- src row s, `esize`-byte
// elements.  mode 0: s + off; 1: rotate-half pair order inside heads of d rows
// (row p -> 2p, row p + d/2 -> 2p + 1), plus off; 2: 2s + off.
q2_status launch_pack_rows(void* dst, int64_t dst_ld, const void* src, int64_t src_ld, int64_t nrows, int64_t ncols,
                           int esize, int mode, int d, int64_t off, hipStream_t s);

// Argmax helpers on packed (value, index) keys.
q2_status launch_argmax_rows(unsigned long long* keys, int64_t key_stride, const void* vals, int32_t dtype,
                             int64_t ldv, int rows, int V, hipStream_t s);

}  // namespace q2
