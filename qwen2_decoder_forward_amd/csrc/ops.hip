// Memory-bound operator kernels and the operator entry points of the C ABI.
#include <mutex>

#include "attention.hpp"
#include "epilogue.hpp"
#include "kvcache.hpp"
#include "simple.hpp"

namespace q2 {

namespace {

// ------------------------------------------------------------------ embedding

// out[m] = w[ids[m]]; with sq (bf16, H % 16 == 0, vector path) also the sum of
// squares of each 16-feature tile of the row: sq[m * sq_ld + f / 16].
template <typename T>
__global__ __launch_bounds__(256) void embedding_kernel(T* __restrict__ out, int64_t ldo, const int64_t* __restrict__ ids,
                                                        int64_t ids_bs, int64_t ids_ts, int Tn, const T* __restrict__ w,
                                                        int64_t ldw, int V, int H, float* __restrict__ sq,
                                                        int64_t sq_ld) {
  const int m = blockIdx.x;
  const int b = m / Tn;
  const int t = m - b * Tn;
  const int64_t id = ids[b * ids_bs + t * ids_ts];
  T* o = out + static_cast<int64_t>(m) * ldo;
  const bool ok = id >= 0 && id < V;
  const T* src = w + (ok ? id : 0) * ldw;
  constexpr int VEC = 16 / sizeof(T);
  const bool vec = (H % VEC == 0) && aligned16(o) && aligned16(src);
  if (vec) {
    const uint4 z = {0, 0, 0, 0};
    for (int i0 = 0; i0 < H; i0 += 256 * VEC) {
      const int i = i0 + threadIdx.x * VEC;
      uint4 v = z;
      if (i < H) {
        v = ok ? *reinterpret_cast<const uint4*>(src + i) : z;
        *reinterpret_cast<uint4*>(o + i) = v;
      }
      if constexpr (sizeof(T) == 2) {
        if (sq) {  // two consecutive threads hold one 16-feature tile
          float ss = 0.f;
          const uint32_t* ws = &v.x;
#pragma unroll
          for (int k = 0; k < 4; ++k) ss += bf_lo(ws[k]) * bf_lo(ws[k]) + bf_hi(ws[k]) * bf_hi(ws[k]);
          ss += __shfl_xor(ss, 1, 64);
          if (i < H && (threadIdx.x & 1) == 0) sq[m * sq_ld + i / 16] = ss;
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < H; i += 256) o[i] = ok ? src[i] : T(0);
  }
}

// ------------------------------------------------------------------ rmsnorm

// One wave per row: float32 sum of squares, y = x * (1 / sqrt(ms + eps)) * w, rounded once.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(T* __restrict__ out, int64_t ldo, const T* __restrict__ in,
                                                      int64_t ldi, const T* __restrict__ w, int rows, int H, float eps) {
  using S = St<T>;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const T* x = in + static_cast<int64_t>(row) * ldi;
  float ss = 0.f;
  for (int i = lane; i < H; i += 64) {
    const float v = S::ld(x + i);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);
  T* y = out + static_cast<int64_t>(row) * ldo;
  for (int i = lane; i < H; i += 64) S::st(y + i, (S::ld(x + i) * inv) * S::ld(w + i));
}

// bf16 rows with H % 8 == 0 and 16-byte aligned rows: one wave per row, the
// row held in registers (CH 16-byte chunks per lane), every load issued before
// the first use, so a row costs one memory round trip instead of H / 64.
template <int CH>
__global__ __launch_bounds__(256) void rmsnorm_vec_kernel(uint16_t* __restrict__ out, int64_t ldo,
                                                          const uint16_t* __restrict__ in, int64_t ldi,
                                                          const uint16_t* __restrict__ w, int rows, int H, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int nch = H >> 3;
  const uint16_t* x = in + static_cast<int64_t>(row) * ldi;
  // the norm weight does not depend on the row: its loads go out with the
  // row's, so the row costs a single memory round trip
  uint4 v[CH], wv[CH];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = lane + 64 * c;
    v[c] = i < nch ? *reinterpret_cast<const uint4*>(x + 8 * i) : uint4{0, 0, 0, 0};
    wv[c] = i < nch ? *reinterpret_cast<const uint4*>(w + 8 * i) : uint4{0, 0, 0, 0};
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint32_t* e = &v[c].x;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = bf_lo(e[k]), b = bf_hi(e[k]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);
  uint16_t* y = out + static_cast<int64_t>(row) * ldo;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = lane + 64 * c;
    if (i < nch) {
      const uint32_t* e = &v[c].x;
      const uint32_t* we = &wv[c].x;
      uint4 r;
      uint32_t* re = &r.x;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        re[k] = pack_bf2((bf_lo(e[k]) * inv) * bf_lo(we[k]), (bf_hi(e[k]) * inv) * bf_hi(we[k]));
      *reinterpret_cast<uint4*>(y + 8 * i) = r;
    }
  }
}

// ------------------------------------------------------------------ add / swiglu

template <typename T>
__global__ __launch_bounds__(256) void add_kernel(T* c, int64_t ldc, const T* a, int64_t lda, const T* b, int64_t ldb,
                                                  int64_t rows, int cols) {
  using S = St<T>;
  const int64_t n = rows * cols;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / cols;
    const int64_t j = i - r * cols;
    S::st(c + r * ldc + j, S::ld(a + r * lda + j) + S::ld(b + r * ldb + j));
  }
}

template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(T* o, int64_t ldo, const T* g, int64_t ldg, const T* u, int64_t ldu,
                                                     int64_t rows, int cols) {
  using S = St<T>;
  const int64_t n = rows * cols;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / cols;
    const int64_t j = i - r * cols;
    S::st(o + r * ldo + j, silu_f(S::ld(g + r * ldg + j)) * S::ld(u + r * ldu + j));
  }
}

// ------------------------------------------------------------------ rope

struct RopeGeom {
  int64_t i_bs, i_ts, i_hs;   // input strides: batch, token, head
  int64_t o_bs, o_ts, o_hs;
  int64_t p_bs, p_ts;         // position strides
  int B, Tn, nh, d;
};

template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(T* out, const T* in, const int64_t* pos, RopeGeom g, float theta) {
  using S = St<T>;
  const int half = g.d >> 1;
  const int64_t n = static_cast<int64_t>(g.B) * g.Tn * g.nh * half;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int j = static_cast<int>(i % half);
  int64_t r = i / half;
  const int h = static_cast<int>(r % g.nh);
  r /= g.nh;
  const int t = static_cast<int>(r % g.Tn);
  const int b = static_cast<int>(r / g.Tn);
  const float2 cs = rope_cs(pos[b * g.p_bs + t * g.p_ts], j, g.d, theta);
  const T* x = in + b * g.i_bs + t * g.i_ts + h * g.i_hs;
  T* y = out + b * g.o_bs + t * g.o_ts + h * g.o_hs;
  const float a = S::ld(x + j);
  const float c = S::ld(x + j + half);
  S::st(y + j, a * cs.x - c * cs.y);
  S::st(y + j + half, c * cs.x + a * cs.y);
}

__global__ __launch_bounds__(256) void rope_table_kernel(float2* table, int npos, int d, float theta) {
  const int half = d >> 1;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(npos) * half) return;
  table[i] = rope_cs(i / half, static_cast<int>(i % half), d, theta);
}

// ------------------------------------------------------------------ argmax

__global__ void keys_zero_kernel(unsigned long long* keys, int64_t stride, int rows) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < rows) keys[r * stride] = 0ull;
}

template <typename T>
__global__ __launch_bounds__(256) void argmax_kernel(unsigned long long* keys, int64_t key_stride, const T* vals,
                                                     int64_t ldv, int V) {
  __shared__ unsigned long long red[4];
  const int row = blockIdx.y;
  const T* x = vals + static_cast<int64_t>(row) * ldv;
  const int base = blockIdx.x * 8192;
  const int end = min(base + 8192, V);
  unsigned long long best = 0;
  for (int i = base + threadIdx.x; i < end; i += 256) {
    const unsigned long long k = argmax_key(St<T>::ld(x + i), static_cast<uint32_t>(i));
    best = k > best ? k : best;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long k = __shfl_xor(best, o, 64);
    best = k > best ? k : best;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) best = red[w] > best ? red[w] : best;
    atomicMax(keys + row * key_stride, best);
  }
}

__global__ void argmax_finalize_kernel(unsigned long long* keys, int64_t key_stride, float* val, int64_t val_stride,
                                       int rows) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const unsigned long long k = keys[r * key_stride];
  val[r * val_stride] = argmax_key_value(k);
  reinterpret_cast<int64_t*>(keys)[r * key_stride] = static_cast<int64_t>(argmax_key_index(k));
}

// ------------------------------------------------------------------ rearrange

struct Geom5 {
  int64_t shape[Q2_MAX_DIMS];
  int64_t so[Q2_MAX_DIMS];
  int64_t si[Q2_MAX_DIMS];
  int nd;
};

template <typename E>
__global__ __launch_bounds__(256) void rearrange_kernel(E* out, const E* in, Geom5 g, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    int64_t rem = i, oo = 0, oi = 0;
    for (int dd = g.nd - 1; dd >= 0; --dd) {
      const int64_t c = rem % g.shape[dd];
      rem /= g.shape[dd];
      oo += c * g.so[dd];
      oi += c * g.si[dd];
    }
    out[oo] = in[oi];
  }
}

// Rows of 16-byte vectors: the last dim is contiguous in both tensors and a
// row is a whole number of vectors.  shape/strides here describe the outer
// dims (elements), vecs = vectors per row.
__global__ __launch_bounds__(256) void rearrange_rows16_kernel(char* out, const char* in, Geom5 g, int64_t vecs,
                                                               int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    int64_t rem = i / vecs;
    const int64_t v = i - rem * vecs;
    int64_t oo = 0, oi = 0;
    for (int dd = g.nd - 1; dd >= 0; --dd) {
      const int64_t c = rem % g.shape[dd];
      rem /= g.shape[dd];
      oo += c * g.so[dd];
      oi += c * g.si[dd];
    }
    *reinterpret_cast<uint4*>(out + oo + v * 16) = *reinterpret_cast<const uint4*>(in + oi + v * 16);
  }
}

// ------------------------------------------------------------------ weight packing

__global__ __launch_bounds__(256) void pack_rows_kernel(char* dst, int64_t dst_ld, const char* src, int64_t src_ld,
                                                        int64_t nrows, int64_t row_bytes, int mode, int d, int64_t off) {
  const int64_t n = nrows * row_bytes;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t s = i / row_bytes;
    const int64_t c = i - s * row_bytes;
    int64_t r;
    if (mode == 1) {
      const int64_t h = s / d, p = s - h * d, half = d / 2;
      r = h * d + (p < half ? 2 * p : 2 * (p - half) + 1) + off;
    } else if (mode == 2) {
      r = 2 * s + off;
    } else {
      r = s + off;
    }
    dst[r * dst_ld + c] = src[s * src_ld + c];
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65535 * 8) g = 65535 * 8;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

}  // namespace

// ------------------------------------------------------------------ launchers

template <typename T>
q2_status launch_embedding(T* out, int64_t ldo, const int64_t* ids, int64_t ids_bs, int64_t ids_ts, int B, int Tn,
                           const T* weight, int64_t ldw, int V, int H, hipStream_t s, float* sq, int64_t sq_ld) {
  if (B * Tn == 0) return Q2_OK;
  if (sq)
    Q2_CHECK(sizeof(T) == 2 && H % 16 == 0 && aligned16(out) && aligned16(weight) && ldo % 8 == 0 && ldw % 8 == 0,
             Q2_EINVAL, "embedding: row sums of squares need aligned bf16 rows");
  hipLaunchKernelGGL(embedding_kernel<T>, dim3(B * Tn), dim3(256), 0, s, out, ldo, ids, ids_bs, ids_ts, Tn, weight, ldw,
                     V, H, sq, sq_ld);
  return check_launch("embedding");
}

template <typename T>
q2_status launch_rmsnorm(T* out, int64_t ldo, const T* in, int64_t ldi, const T* w, int rows, int H, float eps,
                         hipStream_t s) {
  if (rows == 0) return Q2_OK;
  if constexpr (sizeof(T) == 2) {
    const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const int ch = cdiv(H / 8, 64);
    if (H % 8 == 0 && ldo % 8 == 0 && ldi % 8 == 0 && a16(out) && a16(in) && a16(w) && ch <= 8) {
      const dim3 g(cdiv(rows, 4)), b(256);
      if (ch <= 2)
        hipLaunchKernelGGL(rmsnorm_vec_kernel<2>, g, b, 0, s, out, ldo, in, ldi, w, rows, H, eps);
      else if (ch <= 4)
        hipLaunchKernelGGL(rmsnorm_vec_kernel<4>, g, b, 0, s, out, ldo, in, ldi, w, rows, H, eps);
      else
        hipLaunchKernelGGL(rmsnorm_vec_kernel<8>, g, b, 0, s, out, ldo, in, ldi, w, rows, H, eps);
      return check_launch("rms_norm");
    }
  }
  hipLaunchKernelGGL(rmsnorm_kernel<T>, dim3(cdiv(rows, 4)), dim3(256), 0, s, out, ldo, in, ldi, w, rows, H, eps);
  return check_launch("rms_norm");
}

template <typename T>
q2_status launch_add(T* c, int64_t ldc, const T* a, int64_t lda, const T* b, int64_t ldb, int64_t rows, int cols,
                     hipStream_t s) {
  if (rows * cols == 0) return Q2_OK;
  hipLaunchKernelGGL(add_kernel<T>, dim3(grid_for(rows * cols)), dim3(256), 0, s, c, ldc, a, lda, b, ldb, rows, cols);
  return check_launch("add");
}

template <typename T>
q2_status launch_swiglu(T* o, int64_t ldo, const T* g, int64_t ldg, const T* u, int64_t ldu, int64_t rows, int cols,
                        hipStream_t s) {
  if (rows * cols == 0) return Q2_OK;
  hipLaunchKernelGGL(swiglu_kernel<T>, dim3(grid_for(rows * cols)), dim3(256), 0, s, o, ldo, g, ldg, u, ldu, rows, cols);
  return check_launch("swiglu");
}

template q2_status launch_embedding<float>(float*, int64_t, const int64_t*, int64_t, int64_t, int, int, const float*,
                                           int64_t, int, int, hipStream_t, float*, int64_t);
template q2_status launch_embedding<uint16_t>(uint16_t*, int64_t, const int64_t*, int64_t, int64_t, int, int,
                                              const uint16_t*, int64_t, int, int, hipStream_t, float*, int64_t);
template q2_status launch_rmsnorm<float>(float*, int64_t, const float*, int64_t, const float*, int, int, float,
                                         hipStream_t);
template q2_status launch_rmsnorm<uint16_t>(uint16_t*, int64_t, const uint16_t*, int64_t, const uint16_t*, int, int,
                                            float, hipStream_t);
template q2_status launch_add<float>(float*, int64_t, const float*, int64_t, const float*, int64_t, int64_t, int,
                                     hipStream_t);
template q2_status launch_add<uint16_t>(uint16_t*, int64_t, const uint16_t*, int64_t, const uint16_t*, int64_t,
                                        int64_t, int, hipStream_t);
template q2_status launch_swiglu<float>(float*, int64_t, const float*, int64_t, const float*, int64_t, int64_t, int,
                                        hipStream_t);
template q2_status launch_swiglu<uint16_t>(uint16_t*, int64_t, const uint16_t*, int64_t, const uint16_t*, int64_t,
                                           int64_t, int, hipStream_t);

q2_status launch_rope_table(float2* table, int npos, int d, float theta, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(npos) * (d / 2);
  if (n == 0) return Q2_OK;
  hipLaunchKernelGGL(rope_table_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, table, npos, d, theta);
  return check_launch("rope_table");
}

q2_status launch_pack_rows(void* dst, int64_t dst_ld, const void* src, int64_t src_ld, int64_t nrows, int64_t ncols,
                           int esize, int mode, int d, int64_t off, hipStream_t s) {
  const int64_t n = nrows * ncols * esize;
  if (n == 0) return Q2_OK;
  hipLaunchKernelGGL(pack_rows_kernel, dim3(grid_for(n)), dim3(256), 0, s, static_cast<char*>(dst), dst_ld * esize,
                     static_cast<const char*>(src), src_ld * esize, nrows, ncols * esize, mode, d, off);
  return check_launch("pack_rows");
}

q2_status launch_argmax_rows(unsigned long long* keys, int64_t key_stride, const void* vals, int32_t dtype,
                             int64_t ldv, int rows, int V, hipStream_t s) {
  if (rows == 0) return Q2_OK;
  hipLaunchKernelGGL(keys_zero_kernel, dim3(cdiv(rows, 256)), dim3(256), 0, s, keys, key_stride, rows);
  Q2_TRY(check_launch("argmax_init"));
  if (V == 0) return Q2_OK;
  dim3 grid(cdiv(V, 8192), rows);
  if (dtype == Q2_F32)
    hipLaunchKernelGGL(argmax_kernel<float>, grid, dim3(256), 0, s, keys, key_stride, static_cast<const float*>(vals),
                       ldv, V);
  else
    hipLaunchKernelGGL(argmax_kernel<uint16_t>, grid, dim3(256), 0, s, keys, key_stride,
                       static_cast<const uint16_t*>(vals), ldv, V);
  return check_launch("argmax");
}

}  // namespace q2

using namespace q2;

// ==================================================================== C ABI

extern "C" q2_status q2_embedding(const q2_tensor* out, const q2_tensor* ids, const q2_tensor* weight, void* stream) {
  clear_error();
  Rows o, w;
  Q2_TRY(as_rows(out, "out", &o));
  Q2_TRY(as_rows(weight, "weight", &w));
  Q2_TRY(check_desc(ids, "ids"));
  Q2_CHECK(ids->dtype == Q2_I64, Q2_EDTYPE, "ids must be int64");
  Q2_CHECK(is_float(o.dtype) && o.dtype == w.dtype, Q2_EDTYPE, "out and weight must share a float dtype");
  Q2_CHECK(weight->ndim == 2, Q2_ESHAPE, "weight must be [V, H]");
  Q2_CHECK(o.cols == w.cols, Q2_ESHAPE, "out and weight hidden sizes differ");
  Q2_CHECK(o.rows == numel(*ids), Q2_ESHAPE, "out rows (%lld) != number of ids (%lld)", (long long)o.rows,
           (long long)numel(*ids));
  Q2_CHECK(ids->ndim <= 2, Q2_ESHAPE, "ids must be [N] or [B, T]");
  const int B = ids->ndim == 2 ? static_cast<int>(ids->shape[0]) : 1;
  const int Tn = static_cast<int>(ids->shape[ids->ndim - 1]);
  const int64_t bs = ids->ndim == 2 ? ids->stride[0] : 0;
  const int64_t ts = ids->stride[ids->ndim - 1];
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (o.dtype == Q2_F32)
    return launch_embedding<float>(reinterpret_cast<float*>(o.data), o.ld, static_cast<const int64_t*>(ids->data), bs,
                                   ts, B, Tn, reinterpret_cast<const float*>(w.data), w.ld, static_cast<int>(w.rows),
                                   static_cast<int>(w.cols), s);
  return launch_embedding<uint16_t>(reinterpret_cast<uint16_t*>(o.data), o.ld, static_cast<const int64_t*>(ids->data),
                                    bs, ts, B, Tn, reinterpret_cast<const uint16_t*>(w.data), w.ld,
                                    static_cast<int>(w.rows), static_cast<int>(w.cols), s);
}

// Caller-owned workspace of an operator call: a contiguous, 16-byte aligned
// tensor of any dtype whose bytes the call may overwrite (NULL: none).
static q2_status workspace_of(const q2_tensor* ws, void** ptr, size_t* bytes) {
  *ptr = nullptr;
  *bytes = 0;
  if (!ws) return Q2_OK;
  Q2_TRY(check_desc(ws, "workspace"));
  Q2_CHECK(is_contiguous(*ws), Q2_ESTRIDE, "workspace must be contiguous");
  Q2_CHECK(aligned16(ws->data), Q2_ESTRIDE, "workspace must be 16-byte aligned");
  *ptr = ws->data;
  *bytes = static_cast<size_t>(numel(*ws) * dtype_size(ws->dtype));
  return Q2_OK;
}

// Checks the operands of q2_linear and fills the product's descriptor.
static q2_status linear_args(const q2_tensor* out, const q2_tensor* in, const q2_tensor* weight,
                             const q2_tensor* bias, GemmArgs* args, int32_t* dtype) {
  Rows o, x, w;
  Q2_TRY(as_rows(out, "out", &o));
  Q2_TRY(as_rows(in, "in", &x));
  Q2_TRY(as_rows(weight, "weight", &w));
  Q2_CHECK(weight->ndim == 2, Q2_ESHAPE, "weight must be [N, K]");
  Q2_CHECK(x.cols == w.cols, Q2_ESHAPE, "in features (%lld) != weight columns (%lld)", (long long)x.cols,
           (long long)w.cols);
  Q2_CHECK(o.cols == w.rows, Q2_ESHAPE, "out features (%lld) != weight rows (%lld)", (long long)o.cols,
           (long long)w.rows);
  Q2_CHECK(o.rows == x.rows, Q2_ESHAPE, "out rows (%lld) != in rows (%lld)", (long long)o.rows, (long long)x.rows);
  Q2_CHECK(x.rows <= INT32_MAX && w.rows <= INT32_MAX && w.cols <= INT32_MAX, Q2_ESHAPE, "linear: size too large");
  Q2_CHECK(x.dtype == w.dtype && is_float(x.dtype), Q2_EDTYPE, "in and weight must share a float dtype");
  Q2_CHECK(o.dtype == x.dtype || (x.dtype == Q2_BF16 && o.dtype == Q2_F32), Q2_EDTYPE, "unsupported out dtype");
  if (bias) {
    Q2_TRY(check_desc(bias, "bias"));
    Q2_CHECK(bias->dtype == w.dtype, Q2_EDTYPE, "bias dtype must match weight");
    Q2_CHECK(bias->ndim == 1 && bias->shape[0] == w.rows, Q2_ESHAPE, "bias must be [N]");
    Q2_CHECK(bias->stride[0] == 1 || bias->shape[0] <= 1, Q2_ESTRIDE, "bias must be contiguous");
  }
  GemmArgs a{};
  a.W = w.data;
  a.ldw = w.ld;
  a.X = x.data;
  a.ldx = x.ld;
  a.M = static_cast<int>(x.rows);
  a.N = static_cast<int>(w.rows);
  a.K = static_cast<int>(w.cols);
  a.epi.kind = EPI_STORE;
  a.epi.out = o.data;
  a.epi.ldo = o.ld;
  a.epi.out_f32 = o.dtype == Q2_F32;
  a.epi.bias = bias ? bias->data : nullptr;
  if (x.dtype == Q2_BF16) {
    Q2_CHECK(a.K % 8 == 0, Q2_ESHAPE, "bf16 linear: K must be a multiple of 8");
    Q2_CHECK(aligned16(x.data) && aligned16(w.data) && (x.ld % 8 == 0 || x.rows <= 1) &&
                 (w.ld % 8 == 0 || w.rows <= 1),
             Q2_ESTRIDE, "bf16 linear: in and weight rows must be 16-byte aligned");
  }
  *args = a;
  *dtype = x.dtype;
  return Q2_OK;
}

static size_t linear_partial_bytes(int32_t dtype, int64_t M, int64_t N, int64_t K) {
  if (dtype != Q2_BF16 || M > GEMV_MAX_M || M == 0 || N == 0) return 0;
  return gemm_scratch_bytes(static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
}

extern "C" q2_status q2_linear(const q2_tensor* out, const q2_tensor* in, const q2_tensor* weight,
                               const q2_tensor* bias, const q2_tensor* workspace, void* stream) {
  clear_error();
  GemmArgs a{};
  int32_t dt = 0;
  Q2_TRY(linear_args(out, in, weight, bias, &a, &dt));
  Q2_TRY(workspace_of(workspace, &a.scratch, &a.scratch_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == Q2_F32) return gemm_f32(a, s);
  a.unsplit_if_short = true;
  return gemm_bf16(a, s);
}

// ------------------------------------------------------------ allocation-free linear

// Split-K partials of q2_linear_noalloc: a fixed array in the library's code
// object, one copy per GPU, held until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host it only names the symbol):
// it uses the device address hipGetSymbolAddress returns for the current GPU.
static __device__ __align__(256) unsigned char scratch[Q2_LINEAR_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of the current GPU's copy of `scratch`, looked up on the
// first call on that GPU.
static q2_status noalloc_scratch(void** out) {
  int dev = 0;
  Q2_HIP(hipGetDevice(&dev));
  Q2_CHECK(dev >= 0 && dev < kMaxDevices, Q2_EINVAL, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    Q2_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    Q2_CHECK(p != nullptr, Q2_EHIP, "hipGetSymbolAddress returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return Q2_OK;
}

extern "C" q2_status q2_linear_noalloc(const q2_tensor* out, const q2_tensor* in, const q2_tensor* weight,
                                       const q2_tensor* bias, void* stream) {
  clear_error();
  GemmArgs a{};
  int32_t dt = 0;
  Q2_TRY(linear_args(out, in, weight, bias, &a, &dt));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == Q2_F32) return gemm_f32(a, s);
  const size_t need = linear_partial_bytes(dt, a.M, a.N, a.K);
  Q2_CHECK(need <= Q2_LINEAR_NOALLOC_SCRATCH_BYTES, Q2_ESHAPE,
           "q2_linear_noalloc: %d x %d x %d needs %zu bytes of split-K partials, more than its %zu-byte "
           "scratch (use q2_linear with a workspace)",
           a.M, a.N, a.K, need, static_cast<size_t>(Q2_LINEAR_NOALLOC_SCRATCH_BYTES));
  if (need) {
    Q2_TRY(noalloc_scratch(&a.scratch));
    a.scratch_bytes = Q2_LINEAR_NOALLOC_SCRATCH_BYTES;
  }
  // the same plan as q2_linear with a workspace of at least `need` bytes
  return gemm_bf16(a, s);
}

extern "C" q2_status q2_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t dtype, size_t* bytes) {
  clear_error();
  Q2_CHECK(bytes != nullptr, Q2_EINVAL, "bytes is null");
  Q2_CHECK(M >= 0 && N >= 0 && K >= 0 && M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX, Q2_ESHAPE,
           "sizes must be in [0, 2^31)");
  Q2_CHECK(dtype == Q2_F32 || dtype == Q2_BF16, Q2_EDTYPE, "dtype must be f32 or bf16");
  *bytes = linear_partial_bytes(dtype, M, N, K);
  return Q2_OK;
}

extern "C" q2_status q2_rms_norm(const q2_tensor* out, const q2_tensor* in, const q2_tensor* weight, float eps,
                                 void* stream) {
  clear_error();
  Rows o, x, w;
  Q2_TRY(as_rows(out, "out", &o));
  Q2_TRY(as_rows(in, "in", &x));
  Q2_TRY(as_rows(weight, "weight", &w));
  Q2_CHECK(is_float(x.dtype) && o.dtype == x.dtype && w.dtype == x.dtype, Q2_EDTYPE, "dtypes must match (f32/bf16)");
  Q2_CHECK(o.rows == x.rows && o.cols == x.cols, Q2_ESHAPE, "out and in shapes differ");
  Q2_CHECK(weight->ndim == 1 && w.cols == x.cols, Q2_ESHAPE, "weight must be [H]");
  Q2_CHECK(x.rows <= INT32_MAX, Q2_ESHAPE, "too many rows");
  Q2_CHECK(eps >= 0.f, Q2_EINVAL, "eps must be non-negative");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (x.dtype == Q2_F32)
    return launch_rmsnorm<float>(reinterpret_cast<float*>(o.data), o.ld, reinterpret_cast<const float*>(x.data), x.ld,
                                 reinterpret_cast<const float*>(w.data), static_cast<int>(x.rows),
                                 static_cast<int>(x.cols), eps, s);
  return launch_rmsnorm<uint16_t>(reinterpret_cast<uint16_t*>(o.data), o.ld, reinterpret_cast<const uint16_t*>(x.data),
                                  x.ld, reinterpret_cast<const uint16_t*>(w.data), static_cast<int>(x.rows),
                                  static_cast<int>(x.cols), eps, s);
}

extern "C" q2_status q2_rope(const q2_tensor* out, const q2_tensor* in, const q2_tensor* pos, float theta,
                             void* stream) {
  clear_error();
  Q2_TRY(check_desc(out, "out"));
  Q2_TRY(check_desc(in, "in"));
  Q2_TRY(check_desc(pos, "pos"));
  Q2_CHECK(is_float(in->dtype) && out->dtype == in->dtype, Q2_EDTYPE, "in/out must share a float dtype");
  Q2_CHECK(pos->dtype == Q2_I64, Q2_EDTYPE, "pos must be int64");
  Q2_CHECK(same_shape(*out, *in), Q2_ESHAPE, "out and in shapes differ");
  Q2_CHECK(in->ndim == 3 || in->ndim == 4, Q2_ESHAPE, "in must be [T, nh, d] or [B, T, nh, d]");
  const int nd = in->ndim;
  Q2_CHECK(in->stride[nd - 1] == 1 && out->stride[nd - 1] == 1, Q2_ESTRIDE, "head dim must be contiguous");
  RopeGeom g{};
  const bool bat = nd == 4;
  g.B = bat ? static_cast<int>(in->shape[0]) : 1;
  g.Tn = static_cast<int>(in->shape[nd - 3]);
  g.nh = static_cast<int>(in->shape[nd - 2]);
  g.d = static_cast<int>(in->shape[nd - 1]);
  Q2_CHECK(g.d % 2 == 0, Q2_ESHAPE, "head dim must be even");
  g.i_bs = bat ? in->stride[0] : 0;
  g.i_ts = in->stride[nd - 3];
  g.i_hs = in->stride[nd - 2];
  g.o_bs = bat ? out->stride[0] : 0;
  g.o_ts = out->stride[nd - 3];
  g.o_hs = out->stride[nd - 2];
  if (pos->ndim == 1) {
    Q2_CHECK(pos->shape[0] == g.Tn, Q2_ESHAPE, "pos must have T entries");
    g.p_bs = 0;
    g.p_ts = pos->stride[0];
  } else {
    Q2_CHECK(pos->ndim == 2 && bat && pos->shape[0] == g.B && pos->shape[1] == g.Tn, Q2_ESHAPE, "pos must be [B, T]");
    g.p_bs = pos->stride[0];
    g.p_ts = pos->stride[1];
  }
  const int64_t n = static_cast<int64_t>(g.B) * g.Tn * g.nh * (g.d / 2);
  if (n == 0) return Q2_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (in->dtype == Q2_F32)
    hipLaunchKernelGGL(rope_kernel<float>, dim3(cdiv(n, 256)), dim3(256), 0, s, static_cast<float*>(out->data),
                       static_cast<const float*>(in->data), static_cast<const int64_t*>(pos->data), g, theta);
  else
    hipLaunchKernelGGL(rope_kernel<uint16_t>, dim3(cdiv(n, 256)), dim3(256), 0, s, static_cast<uint16_t*>(out->data),
                       static_cast<const uint16_t*>(in->data), static_cast<const int64_t*>(pos->data), g, theta);
  return check_launch("rope");
}

extern "C" q2_status q2_self_attention(const q2_tensor* out, const q2_tensor* q, const q2_tensor* k,
                                       const q2_tensor* v, float scale, const q2_tensor* workspace, void* stream) {
  clear_error();
  Q2_TRY(check_desc(out, "out"));
  Q2_TRY(check_desc(q, "q"));
  Q2_TRY(check_desc(k, "k"));
  Q2_TRY(check_desc(v, "v"));
  Q2_CHECK(is_float(q->dtype) && out->dtype == q->dtype && k->dtype == q->dtype && v->dtype == q->dtype, Q2_EDTYPE,
           "q, k, v, out must share a float dtype");
  Q2_CHECK(same_shape(*out, *q), Q2_ESHAPE, "out and q shapes differ");
  Q2_CHECK(same_shape(*k, *v), Q2_ESHAPE, "k and v shapes differ");
  Q2_CHECK((q->ndim == 3 || q->ndim == 4) && k->ndim == q->ndim, Q2_ESHAPE,
           "q must be [T, nh, d] / [B, T, nh, d] and k, v [S, nkv, d] / [B, S, nkv, d]");
  const int nd = q->ndim;
  const bool bat = nd == 4;
  for (const q2_tensor* t : {out, q, k, v})
    Q2_CHECK(t->stride[nd - 1] == 1, Q2_ESTRIDE, "head dim must be contiguous");
  AttnArgs a{};
  a.B = bat ? static_cast<int>(q->shape[0]) : 1;
  Q2_CHECK(!bat || k->shape[0] == a.B, Q2_ESHAPE, "batch sizes differ");
  a.T = static_cast<int>(q->shape[nd - 3]);
  a.nh = static_cast<int>(q->shape[nd - 2]);
  a.d = static_cast<int>(q->shape[nd - 1]);
  a.S = static_cast<int>(k->shape[nd - 3]);
  a.nkv = static_cast<int>(k->shape[nd - 2]);
  Q2_CHECK(k->shape[nd - 1] == a.d, Q2_ESHAPE, "head dims differ");
  Q2_CHECK(a.nkv > 0 && a.nh % a.nkv == 0, Q2_ESHAPE, "nh (%d) must be a multiple of nkv (%d)", a.nh, a.nkv);
  Q2_CHECK(a.S >= a.T, Q2_ESHAPE, "S (%d) must be >= T (%d)", a.S, a.T);
  a.q = q->data;
  a.q_bs = bat ? q->stride[0] : 0;
  a.q_ts = q->stride[nd - 3];
  a.q_hs = q->stride[nd - 2];
  a.o = out->data;
  a.o_bs = bat ? out->stride[0] : 0;
  a.o_ts = out->stride[nd - 3];
  a.o_hs = out->stride[nd - 2];
  a.k = k->data;
  a.k_bs = bat ? k->stride[0] : 0;
  a.k_ss = k->stride[nd - 3];
  a.k_hs = k->stride[nd - 2];
  a.v = v->data;
  a.v_bs = bat ? v->stride[0] : 0;
  a.v_ss = v->stride[nd - 3];
  a.v_hs = v->stride[nd - 2];
  a.scale = scale;
  a.s_max = a.S;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q->dtype == Q2_F32) return attention_f32(a, s);
  Q2_CHECK(a.d == 128, Q2_ESHAPE, "bf16 attention supports head_dim 128 only");
  for (const q2_tensor* t : {out, q, k, v}) {
    Q2_CHECK(aligned16(t->data), Q2_ESTRIDE, "bf16 attention: pointers must be 16-byte aligned");
    for (int i = 0; i < nd - 1; ++i)
      Q2_CHECK(t->stride[i] % 8 == 0 || t->shape[i] <= 1, Q2_ESTRIDE, "bf16 attention: strides must be multiples of 8");
  }
  Q2_TRY(workspace_of(workspace, &a.scratch, &a.scratch_bytes));
  a.unsplit_if_short = true;
  return attention_bf16(a, s);
}

extern "C" q2_status q2_self_attention_workspace_bytes(int32_t B, int32_t T, int32_t S, int32_t nh, int32_t nkv,
                                                       int32_t d, int32_t dtype, size_t* bytes) {
  clear_error();
  Q2_CHECK(bytes != nullptr, Q2_EINVAL, "bytes is null");
  Q2_CHECK(B >= 0 && T >= 0 && S >= T && nkv > 0 && nh % nkv == 0 && d > 0, Q2_ESHAPE, "bad attention sizes");
  Q2_CHECK(dtype == Q2_F32 || dtype == Q2_BF16, Q2_EDTYPE, "dtype must be f32 or bf16");
  *bytes = (dtype == Q2_BF16 && B > 0 && T > 0) ? attention_scratch_bytes(B, T, S, nh, nkv, d) : 0;
  return Q2_OK;
}

static q2_status elementwise3(const q2_tensor* o, const q2_tensor* x, const q2_tensor* y, Rows* ro, Rows* rx,
                              Rows* ry) {
  Q2_TRY(as_rows(o, "out", ro));
  Q2_TRY(as_rows(x, "a", rx));
  Q2_TRY(as_rows(y, "b", ry));
  Q2_CHECK(same_shape(*o, *x) && same_shape(*o, *y), Q2_ESHAPE, "shapes differ");
  Q2_CHECK(is_float(ro->dtype) && rx->dtype == ro->dtype && ry->dtype == ro->dtype, Q2_EDTYPE,
           "dtypes must match (f32/bf16)");
  Q2_CHECK(ro->cols <= INT32_MAX, Q2_ESHAPE, "last dim too large");
  return Q2_OK;
}

extern "C" q2_status q2_swiglu(const q2_tensor* out, const q2_tensor* gate, const q2_tensor* up, void* stream) {
  clear_error();
  Rows o, g, u;
  Q2_TRY(elementwise3(out, gate, up, &o, &g, &u));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (o.dtype == Q2_F32)
    return launch_swiglu<float>(reinterpret_cast<float*>(o.data), o.ld, reinterpret_cast<const float*>(g.data), g.ld,
                                reinterpret_cast<const float*>(u.data), u.ld, o.rows, static_cast<int>(o.cols), s);
  return launch_swiglu<uint16_t>(reinterpret_cast<uint16_t*>(o.data), o.ld, reinterpret_cast<const uint16_t*>(g.data),
                                 g.ld, reinterpret_cast<const uint16_t*>(u.data), u.ld, o.rows,
                                 static_cast<int>(o.cols), s);
}

extern "C" q2_status q2_add(const q2_tensor* c, const q2_tensor* a, const q2_tensor* b, void* stream) {
  clear_error();
  Rows o, x, y;
  Q2_TRY(elementwise3(c, a, b, &o, &x, &y));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (o.dtype == Q2_F32)
    return launch_add<float>(reinterpret_cast<float*>(o.data), o.ld, reinterpret_cast<const float*>(x.data), x.ld,
                             reinterpret_cast<const float*>(y.data), y.ld, o.rows, static_cast<int>(o.cols), s);
  return launch_add<uint16_t>(reinterpret_cast<uint16_t*>(o.data), o.ld, reinterpret_cast<const uint16_t*>(x.data),
                              x.ld, reinterpret_cast<const uint16_t*>(y.data), y.ld, o.rows, static_cast<int>(o.cols),
                              s);
}

extern "C" q2_status q2_argmax(const q2_tensor* max_idx, const q2_tensor* max_val, const q2_tensor* vals,
                               void* stream) {
  clear_error();
  Rows v;
  Q2_TRY(as_rows(vals, "vals", &v));
  Q2_TRY(check_desc(max_idx, "max_idx"));
  Q2_TRY(check_desc(max_val, "max_val"));
  Q2_CHECK(is_float(v.dtype), Q2_EDTYPE, "vals must be f32 or bf16");
  Q2_CHECK(max_idx->dtype == Q2_I64, Q2_EDTYPE, "max_idx must be int64");
  Q2_CHECK(max_val->dtype == Q2_F32, Q2_EDTYPE, "max_val must be f32");
  Q2_CHECK(numel(*max_idx) == v.rows && numel(*max_val) == v.rows, Q2_ESHAPE, "one index and one value per row");
  Q2_CHECK(is_contiguous(*max_idx) && is_contiguous(*max_val), Q2_ESTRIDE, "max_idx and max_val must be contiguous");
  Q2_CHECK(v.cols >= 1 && v.cols <= INT32_MAX, Q2_ESHAPE, "rows must have 1 .. 2^31-1 entries");
  Q2_CHECK(v.rows <= 65535, Q2_ESHAPE, "at most 65535 rows");
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* keys = static_cast<unsigned long long*>(max_idx->data);
  Q2_TRY(launch_argmax_rows(keys, 1, v.data, v.dtype, v.ld, static_cast<int>(v.rows), static_cast<int>(v.cols), s));
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(cdiv(v.rows, 256)), dim3(256), 0, s, keys, 1,
                     static_cast<float*>(max_val->data), 1, static_cast<int>(v.rows));
  return check_launch("argmax_finalize");
}

extern "C" q2_status q2_rearrange(const q2_tensor* out, const q2_tensor* in, void* stream) {
  clear_error();
  Q2_TRY(check_desc(out, "out"));
  Q2_TRY(check_desc(in, "in"));
  Q2_CHECK(out->dtype == in->dtype, Q2_EDTYPE, "dtypes differ");
  Q2_CHECK(same_shape(*out, *in), Q2_ESHAPE, "shapes differ");
  const int64_t n = numel(*in);
  if (n == 0) return Q2_OK;
  const int es = static_cast<int>(dtype_size(in->dtype));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nd = in->ndim;
  // vector path: last dim contiguous in both, whole 16-byte vectors per row, aligned rows
  const int64_t row_bytes = in->shape[nd - 1] * es;
  bool vec = (in->stride[nd - 1] == 1 || in->shape[nd - 1] == 1) && (out->stride[nd - 1] == 1 || out->shape[nd - 1] == 1) &&
             row_bytes % 16 == 0 && aligned16(in->data) && aligned16(out->data);
  for (int i = 0; vec && i < nd - 1; ++i)
    vec = ((in->stride[i] * es) % 16 == 0) && ((out->stride[i] * es) % 16 == 0);
  if (vec) {
    Geom5 g{};
    g.nd = nd - 1;
    for (int i = 0; i < nd - 1; ++i) {
      g.shape[i] = in->shape[i];
      g.so[i] = out->stride[i] * es;
      g.si[i] = in->stride[i] * es;
    }
    const int64_t vecs = row_bytes / 16;
    const int64_t total = (n / in->shape[nd - 1]) * vecs;
    hipLaunchKernelGGL(rearrange_rows16_kernel, dim3(grid_for(total)), dim3(256), 0, s, static_cast<char*>(out->data),
                       static_cast<const char*>(in->data), g, vecs, total);
    return check_launch("rearrange");
  }
  Geom5 g{};
  g.nd = nd;
  for (int i = 0; i < nd; ++i) {
    g.shape[i] = in->shape[i];
    g.so[i] = out->stride[i];
    g.si[i] = in->stride[i];
  }
  if (es == 1)
    hipLaunchKernelGGL(rearrange_kernel<uint8_t>, dim3(grid_for(n)), dim3(256), 0, s, static_cast<uint8_t*>(out->data),
                       static_cast<const uint8_t*>(in->data), g, n);
  else if (es == 2)
    hipLaunchKernelGGL(rearrange_kernel<uint16_t>, dim3(grid_for(n)), dim3(256), 0, s, static_cast<uint16_t*>(out->data),
                       static_cast<const uint16_t*>(in->data), g, n);
  else if (es == 4)
    hipLaunchKernelGGL(rearrange_kernel<uint32_t>, dim3(grid_for(n)), dim3(256), 0, s, static_cast<uint32_t*>(out->data),
                       static_cast<const uint32_t*>(in->data), g, n);
  else
    hipLaunchKernelGGL(rearrange_kernel<uint64_t>, dim3(grid_for(n)), dim3(256), 0, s, static_cast<uint64_t*>(out->data),
                       static_cast<const uint64_t*>(in->data), g, n);
  return check_launch("rearrange");
}

// ------------------------------------------------------------------ FP8 KV-cache codec

// Rows of 128 values as the codec's [N, 128] operand (row stride in elements).
static q2_status kv_rows(const q2_tensor* t, const char* name, int32_t dtype, Rows* r) {
  Q2_TRY(as_rows(t, name, r));
  Q2_CHECK(r->dtype == dtype, Q2_EDTYPE, "%s has the wrong dtype", name);
  Q2_CHECK(r->cols == KV_BLOCK, Q2_ESHAPE, "%s rows must hold %d elements", name, KV_BLOCK);
  Q2_CHECK(aligned16(r->data) && (r->rows <= 1 || (r->ld * dtype_size(dtype)) % 16 == 0), Q2_ESTRIDE,
           "%s rows must be 16-byte aligned", name);
  return Q2_OK;
}

static q2_status kv_scales(const q2_tensor* t, int64_t rows) {
  Q2_TRY(check_desc(t, "scales"));
  Q2_CHECK(t->dtype == Q2_F32, Q2_EDTYPE, "scales must be f32");
  Q2_CHECK(numel(*t) == rows && is_contiguous(*t), Q2_ESHAPE, "scales must be %lld contiguous floats",
           static_cast<long long>(rows));
  return Q2_OK;
}

extern "C" q2_status q2_kv_quantize(const q2_tensor* codes, const q2_tensor* scales, const q2_tensor* x,
                                    void* stream) {
  clear_error();
  Rows c, xr;
  Q2_TRY(kv_rows(codes, "codes", Q2_U8, &c));
  Q2_TRY(kv_rows(x, "x", Q2_BF16, &xr));
  Q2_CHECK(c.rows == xr.rows, Q2_ESHAPE, "codes and x row counts differ");
  Q2_TRY(kv_scales(scales, xr.rows));
  return launch_kv_quantize(reinterpret_cast<uint8_t*>(c.data), c.ld, static_cast<float*>(scales->data),
                            reinterpret_cast<const uint16_t*>(xr.data), xr.ld, xr.rows,
                            static_cast<hipStream_t>(stream));
}

extern "C" q2_status q2_kv_dequantize(const q2_tensor* x, const q2_tensor* codes, const q2_tensor* scales,
                                      void* stream) {
  clear_error();
  Rows c, xr;
  Q2_TRY(kv_rows(codes, "codes", Q2_U8, &c));
  Q2_TRY(kv_rows(x, "x", Q2_BF16, &xr));
  Q2_CHECK(c.rows == xr.rows, Q2_ESHAPE, "codes and x row counts differ");
  Q2_TRY(kv_scales(scales, xr.rows));
  return launch_kv_dequantize(reinterpret_cast<uint16_t*>(xr.data), xr.ld, reinterpret_cast<const uint8_t*>(c.data),
                              c.ld, static_cast<const float*>(scales->data), xr.rows, static_cast<hipStream_t>(stream));
}
