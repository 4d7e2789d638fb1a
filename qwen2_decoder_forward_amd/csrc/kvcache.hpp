// FP8 KV cache: blocks of 128 elements (one token of one KV head) stored as
// FP8 E4M3 codes with one float32 scale per block ("新一代大模型Day0推理适配与
// 性能调优教程", step 5: the KV cache quantised to FP8 per token x per head x
// 128-element block, accumulation kept in high precision).
//
// Code format (OCP FP8 E4M3, "FN": no infinities): sign, 4 exponent bits
// (bias 7), 3 mantissa bits.  Exponent field 0 holds the subnormals m * 2^-9;
// fields 1..15 hold (1 + m/8) * 2^(e-7), except 0x7F / 0xFF (NaN, never
// written).  Largest finite value 448.
//
// Block quantisation (float32 throughout):
//   amax  = max |x_i|                       (x: the bf16 values)
//   scale = amax / 448                      (0 when amax = 0)
//   code  = E4M3(x_i / scale), round to nearest, ties to even, |.| saturated
//           at 448; the sign bit is the sign of x_i / scale (x_i itself when
//           scale = 0), so -0 codes as 0x80
// Dequantisation, to the storage type the attention reads:
//   x'_i = bf16(value(code_i) * scale)      (float32 product, then RNE)
#pragma once

#include "common.hpp"

namespace q2 {

constexpr int KV_BLOCK = 128;

// E4M3 code of y (finite), round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sgn = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {          // |y| >= 448 (every larger value rounds past the top code)
    code = 0x7Eu;
  } else if (a >= 0x3C800000u) {   // 2^-6 <= |y| < 448: normal codes
    const uint32_t E = a >> 23;    // biased float32 exponent, 121 .. 135
    const uint32_t mant = a & 0x7FFFFFu;
    // 23 fraction bits to 3, ties to even; r = 8 carries into the exponent field
    const uint32_t r = (mant + 0x7FFFFu + ((mant >> 20) & 1u)) >> 20;
    code = ((E - 120u) << 3) + r;
  } else {                         // |y| < 2^-6: multiples of 2^-9
    const uint32_t E = a >> 23;
    const int shift = 141 - static_cast<int>(E);  // |y| * 2^9 = full >> shift
    if (E == 0 || shift > 31) {
      code = 0;
    } else {
      const uint32_t full = 0x800000u | (a & 0x7FFFFFu);
      uint32_t q = full >> shift;
      const uint32_t rem = full & ((1u << shift) - 1u);
      const uint32_t half = 1u << (shift - 1);
      q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
      code = q;                    // q = 8 is the smallest normal code
    }
  }
  return code | sgn;
}

// Two E4M3 codes (bytes 0 and 1 of `w` when !hi, bytes 2 and 3 when hi) to
// float32 (exact) by the hardware conversion.
typedef float float2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2v e4m3_decode2(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true)
            : __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
}

// Eight codes (8 bytes) times `scale`, rounded to bf16: 16 bytes.
__device__ __forceinline__ uint4 e4m3_dequant8(uint2 c, float scale) {
  const float2v a = e4m3_decode2(c.x, false), b = e4m3_decode2(c.x, true);
  const float2v e = e4m3_decode2(c.y, false), f = e4m3_decode2(c.y, true);
  uint4 r;
  r.x = pack_bf2(a.x * scale, a.y * scale);
  r.y = pack_bf2(b.x * scale, b.y * scale);
  r.z = pack_bf2(e.x * scale, e.y * scale);
  r.w = pack_bf2(f.x * scale, f.y * scale);
  return r;
}

// Rows of 128 bf16 values -> codes and scales (row strides in elements / bytes).
q2_status launch_kv_quantize(uint8_t* codes, int64_t ldc, float* scales, const uint16_t* x, int64_t ldx, int64_t n,
                             hipStream_t s);
// Codes and scales -> bf16 rows.
q2_status launch_kv_dequantize(uint16_t* x, int64_t ldx, const uint8_t* codes, int64_t ldc, const float* scales,
                               int64_t n, hipStream_t s);

// One layer's cache as rows of 128 elements: the bf16 values, or the FP8
// codes (1 byte each) with one float32 scale per row.  Row (b, h, j) --
// sequence b, KV head h, position j -- is
//   contiguous: b * bs + h * hs + j
//   paged:      table[b * tstride + j / P] * nkv * P + h * P + j % P
// (a page holds P consecutive positions of all KV heads of one sequence,
// table maps a sequence's page index to a page of the pool).
struct KvLayout {
  void* kc;
  void* vc;
  float* ks;        // FP8 scales (null for bf16)
  float* vs;
  int fp8;
  int64_t bs, hs;   // contiguous strides, in rows
  const int* table; // paged: [max_batch][tstride] page numbers, or null
  int64_t tstride;
  int P;            // positions per page (a multiple of 64)
  int nkv;
};

// (The host gives a page to every position a call writes or reads; a
// position without one, table entry -1, would be a bug: it maps to page 0
// here rather than outside the pool, and kv_store skips it.)
__device__ __forceinline__ int64_t kv_row(const KvLayout& c, int b, int h, int j) {
  if (c.table)
    return static_cast<int64_t>(max(c.table[b * c.tstride + j / c.P], 0)) * c.nkv * c.P + h * c.P + j % c.P;
  return b * c.bs + h * c.hs + j;
}

__device__ __forceinline__ bool kv_mapped(const KvLayout& c, int b, int j) {
  return !c.table || c.table[b * c.tstride + j / c.P] >= 0;
}

// Store this call's new k and v rows, staged as bf16 [B][nkv][T][128]
// (k_stage, v_stage), at positions pos_b .. pos_b + T - 1 of each sequence
// b: pos_b = lens[b] when lens is set, else *d_len when set, else len0.
// bf16 caches copy the rows; FP8 caches quantise them.
q2_status launch_kv_store(const KvLayout& c, const uint16_t* k_stage, const uint16_t* v_stage, int B, int T,
                          const int* lens, const int* d_len, int len0, hipStream_t s);

// Positions [0, S) of B sequences as bf16 K and V arrays [B][nkv][S_cap][128]
// (out_k, out_v), for the prefill attention: a gather of pages and/or the
// dequantisation of FP8 rows.
q2_status launch_kv_expand(uint16_t* out_k, uint16_t* out_v, int64_t S_cap, const KvLayout& c, int B, int S,
                           hipStream_t s);

}  // namespace q2
