// KV-cache kernels: FP8 block quantisation and dequantisation (one wave per
// 128-element block: lane l holds elements 2l and 2l + 1), the model's store
// of new k / v rows into its cache (bf16 or FP8, contiguous or paged), and
// the expansion of cached positions to contiguous bf16 for the prefill
// attention.
#include "kvcache.hpp"

namespace q2 {

namespace {

// One block: x (bf16 pair of this lane) -> 2 codes of this lane; returns the scale.
__device__ __forceinline__ float quant_pair(uint32_t xw, uint32_t& codes2) {
  const float x0 = bf_lo(xw), x1 = bf_hi(xw);
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float scale = amax / 448.0f;
  const float y0 = amax == 0.f ? x0 : x0 / scale;
  const float y1 = amax == 0.f ? x1 : x1 / scale;
  codes2 = e4m3_encode(y0) | (e4m3_encode(y1) << 8);
  return amax == 0.f ? 0.f : scale;
}

__global__ __launch_bounds__(256) void kv_quantize_kernel(uint8_t* __restrict__ codes, int64_t ldc,
                                                          float* __restrict__ scales, const uint16_t* __restrict__ x,
                                                          int64_t ldx, int64_t n) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n) return;  // whole waves leave together
  const int lane = threadIdx.x & 63;
  const uint32_t xw = *reinterpret_cast<const uint32_t*>(x + row * ldx + 2 * lane);
  uint32_t c2;
  const float scale = quant_pair(xw, c2);
  *reinterpret_cast<uint16_t*>(codes + row * ldc + 2 * lane) = static_cast<uint16_t>(c2);
  if (lane == 0) scales[row] = scale;
}

__global__ __launch_bounds__(256) void kv_dequantize_kernel(uint16_t* __restrict__ x, int64_t ldx,
                                                            const uint8_t* __restrict__ codes, int64_t ldc,
                                                            const float* __restrict__ scales, int64_t n) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int lane = threadIdx.x & 63;
  const uint32_t c2 = *reinterpret_cast<const uint16_t*>(codes + row * ldc + 2 * lane);
  const float sc = scales[row];
  const float2v v = e4m3_decode2(c2, false);
  *reinterpret_cast<uint32_t*>(x + row * ldx + 2 * lane) = pack_bf2(v.x * sc, v.y * sc);
}

// Rows (b, h, t, kind) of the staged k / v, one wave each.
__global__ __launch_bounds__(256) void kv_store_kernel(KvLayout c, const uint16_t* __restrict__ k_stage,
                                                       const uint16_t* __restrict__ v_stage, int B, int T,
                                                       const int* __restrict__ lens, const int* __restrict__ d_len,
                                                       int len0) {
  const int64_t rows = static_cast<int64_t>(B) * c.nkv * T;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= 2 * rows) return;
  const bool isv = r >= rows;
  const int64_t i = isv ? r - rows : r;      // (b * nkv + h) * T + t
  const int t = static_cast<int>(i % T);
  const int64_t bh = i / T;
  const int h = static_cast<int>(bh % c.nkv);
  const int b = static_cast<int>(bh / c.nkv);
  const int pos = (lens ? lens[b] : d_len ? *d_len : len0) + t;
  if (!kv_mapped(c, b, pos)) return;  // whole waves leave together
  const int lane = threadIdx.x & 63;
  const uint16_t* src = (isv ? v_stage : k_stage) + i * KV_BLOCK;
  const uint32_t xw = *reinterpret_cast<const uint32_t*>(src + 2 * lane);
  const int64_t row = kv_row(c, b, h, pos);
  if (c.fp8) {
    uint32_t c2;
    const float scale = quant_pair(xw, c2);
    uint8_t* dst = static_cast<uint8_t*>(isv ? c.vc : c.kc) + row * KV_BLOCK;
    *reinterpret_cast<uint16_t*>(dst + 2 * lane) = static_cast<uint16_t>(c2);
    if (lane == 0) (isv ? c.vs : c.ks)[row] = scale;
  } else {
    uint16_t* dst = static_cast<uint16_t*>(isv ? c.vc : c.kc) + row * KV_BLOCK;
    *reinterpret_cast<uint32_t*>(dst + 2 * lane) = xw;
  }
}

// Cache rows (b, h, j < S, kind) -> bf16 [B][nkv][S_cap][128], 16 lanes per
// row (8 elements each), 16 rows per workgroup.
__global__ __launch_bounds__(256) void kv_expand_kernel(uint16_t* __restrict__ out_k, uint16_t* __restrict__ out_v,
                                                        int64_t S_cap, KvLayout c, int B, int S) {
  const int64_t rows = static_cast<int64_t>(B) * c.nkv * S;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  if (r >= 2 * rows) return;
  const bool isv = r >= rows;
  const int64_t i = isv ? r - rows : r;      // (b * nkv + h) * S + j
  const int j = static_cast<int>(i % S);
  const int64_t bh = i / S;
  const int h = static_cast<int>(bh % c.nkv);
  const int b = static_cast<int>(bh / c.nkv);
  const int q = threadIdx.x & 15;
  const int64_t row = kv_row(c, b, h, j);
  uint16_t* dst = (isv ? out_v : out_k) + (bh * S_cap + j) * KV_BLOCK + 8 * q;
  if (c.fp8) {
    const uint2 codes = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(isv ? c.vc : c.kc) +
                                                        row * KV_BLOCK + 8 * q);
    *reinterpret_cast<uint4*>(dst) = e4m3_dequant8(codes, (isv ? c.vs : c.ks)[row]);
  } else {
    *reinterpret_cast<uint4*>(dst) =
        *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(isv ? c.vc : c.kc) + row * KV_BLOCK + 8 * q);
  }
}

}  // namespace

q2_status launch_kv_quantize(uint8_t* codes, int64_t ldc, float* scales, const uint16_t* x, int64_t ldx, int64_t n,
                             hipStream_t s) {
  if (n == 0) return Q2_OK;
  hipLaunchKernelGGL(kv_quantize_kernel, dim3(static_cast<unsigned>((n + 3) / 4)), dim3(256), 0, s, codes, ldc,
                     scales, x, ldx, n);
  return check_launch("kv_quantize");
}

q2_status launch_kv_dequantize(uint16_t* x, int64_t ldx, const uint8_t* codes, int64_t ldc, const float* scales,
                               int64_t n, hipStream_t s) {
  if (n == 0) return Q2_OK;
  hipLaunchKernelGGL(kv_dequantize_kernel, dim3(static_cast<unsigned>((n + 3) / 4)), dim3(256), 0, s, x, ldx, codes,
                     ldc, scales, n);
  return check_launch("kv_dequantize");
}

q2_status launch_kv_store(const KvLayout& c, const uint16_t* k_stage, const uint16_t* v_stage, int B, int T,
                          const int* lens, const int* d_len, int len0, hipStream_t s) {
  const int64_t rows = 2 * static_cast<int64_t>(B) * c.nkv * T;
  if (rows == 0) return Q2_OK;
  hipLaunchKernelGGL(kv_store_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s, c, k_stage, v_stage,
                     B, T, lens, d_len, len0);
  return check_launch("kv_store");
}

q2_status launch_kv_expand(uint16_t* out_k, uint16_t* out_v, int64_t S_cap, const KvLayout& c, int B, int S,
                           hipStream_t s) {
  const int64_t rows = 2 * static_cast<int64_t>(B) * c.nkv * S;
  if (rows == 0) return Q2_OK;
  Q2_CHECK(S <= S_cap, Q2_ESHAPE, "kv expand: %d positions exceed the buffer's %lld", S, static_cast<long long>(S_cap));
  hipLaunchKernelGGL(kv_expand_kernel, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0, s, out_k, out_v,
                     S_cap, c, B, S);
  return check_launch("kv_expand");
}

}  // namespace q2
