// Causal grouped-query attention: scores = (q . k) * scale, causal mask,
// max-subtracted softmax in float32, probabilities times v.
//
// bf16, d = 128, two kernels:
//  * attn_decode  few query rows per KV head (T * group <= 16, the decode
//                 step): one workgroup per (sequence, KV head, key chunk).  All
//                 query heads of the group share each K/V load.  Q K^T runs
//                 on MFMA with K rows streamed straight from memory as the A
//                 operand; P V runs on MFMA with V transposed through LDS.
//                 With several chunks (split-KV) attn_combine merges the
//                 partial results.
//  * attn_prefill 128 queries of one head per workgroup (32 per wave), K and
//                 V^T tiles of 64 keys double-buffered in LDS, online softmax,
//                 32x32x16 MFMAs.
// float32, any d <= 256: attn_f32, one wave per (query, head).
//
// MFMA layout facts used below (16x16 tiles): the A operand lane l holds row
// l%16, the B operand lane l holds column l%16, both with the reduction
// index block l/16; the result lane l holds rows 4*(l/16)+i, column l%16.
// Q K^T is computed transposed (S^T = K Q^T), so a lane's four results are
// four consecutive keys of one query: exactly the B-operand layout of the
// 16x16x16 MFMA that computes O^T = V^T P^T.  No shuffles are needed between
// the two products.
#include <algorithm>

#include "attention.hpp"
#include "kvcache.hpp"

namespace q2 {

namespace {

constexpr int D = 128;
// bf16 per V^T LDS row in attn_decode: 16 keys + pad.  Rows of 9 banks (36
// bytes), so that the fragment reads (16 consecutive rows) fall in distinct
// banks; the transposed writes (rows 8 apart) are spread by a rotation of
// each row's key groups (dec_block).  Rows are 4-byte aligned only, so both
// go as pairs of 32-bit accesses.
constexpr int VT_DEC = 18;
constexpr float NEG_INF = -__builtin_huge_valf();

__device__ __forceinline__ short4_t as_short4(uint2 v) {
  short4_t r;
  __builtin_memcpy(&r, &v, 8);
  return r;
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Marks a loaded value as arrived.  The query fragments are loaded once and
// used in every iteration of a key loop that also issues loads; without this
// the compiler cannot tell across the loop's back edge whether they are still
// pending and waits for every outstanding load (the next block's prefetch
// included) before the first product of each iteration.
__device__ __forceinline__ void settle(uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }

// Order the wave's own LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// Element i (0..7) of a 16-byte vector of bf16.
__device__ __forceinline__ uint32_t elem16(const uint4& v, int i) {
  const uint32_t w = (&v.x)[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Write four keys' 8-element d-chunks transposed: row (d0 + i) gets the 4 keys
// at column `col` (4 consecutive bf16 = 8 bytes; ALIGN8: 8-byte aligned, else
// two 4-byte stores).
// (v_perm_b32 picks the two 16-bit elements: selector bytes 0-3 address its
// second operand, 4-7 its first.)
template <bool ALIGN8>
__device__ __forceinline__ void store_vt4(uint16_t* base, int row_stride, int d0, int col, const uint4 (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
    uint2 w;
    w.x = __builtin_amdgcn_perm((&v[1].x)[i >> 1], (&v[0].x)[i >> 1], sel);
    w.y = __builtin_amdgcn_perm((&v[3].x)[i >> 1], (&v[2].x)[i >> 1], sel);
    if constexpr (ALIGN8) {
      *reinterpret_cast<uint2*>(base + (d0 + i) * row_stride + col) = w;
    } else {
      uint32_t* p = reinterpret_cast<uint32_t*>(base + (d0 + i) * row_stride + col);
      p[0] = w.x;
      p[1] = w.y;
    }
  }
}

// Online-softmax update of one column held by 4 lane groups x 4 values.
// s[] are masked (-inf) scaled scores; returns alpha and writes probabilities.
__device__ __forceinline__ float softmax_step(float* s, int n, float& m_run, float& l_run) {
  float mt = NEG_INF;
  for (int i = 0; i < n; ++i) mt = fmaxf(mt, s[i]);
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float m_new = fmaxf(m_run, mt);
  const float base = (m_new == NEG_INF) ? 0.f : m_new;
  const float alpha = (m_run == NEG_INF) ? 0.f : __expf(m_run - base);
  float ps = 0.f;
  for (int i = 0; i < n; ++i) {
    const float p = (s[i] == NEG_INF) ? 0.f : __expf(s[i] - base);
    s[i] = p;
    ps += p;
  }
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  l_run = l_run * alpha + ps;
  m_run = m_new;
  return alpha;
}

// ------------------------------------------------------------------ decode (split-KV)

// One 16-key block of the decode loop for the calling wave: S^T = K Q^T,
// online softmax, O^T += V^T P^T (V^T through the wave's LDS tile).
__device__ __forceinline__ void dec_block(const uint4 (&kf)[4], const uint4 (&vf)[4], const uint4 (&qf)[4],
                                          uint16_t* vt, int j0, int j_end, int lim, float scale, int col, int G,
                                          floatx4_t (&oacc)[8], float& m_run, float& l_run) {
  floatx4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[kk]), as_bf16x8(qf[kk]), sacc, 0, 0, 0);
  // rows d hold their four 4-key groups rotated by (d / 32) % 4 places: the
  // 16 lanes of one transposed write (rows 8 apart) then cover 16 distinct
  // bank pairs
  store_vt4<false>(vt, VT_DEC, 8 * col, 4 * ((G + (col >> 2)) & 3), vf);

  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kj = j0 + 4 * G + i;
    s[i] = (kj < j_end && kj <= lim) ? sacc[i] * scale : NEG_INF;
  }
  const float alpha = softmax_step(s, 4, m_run, l_run);
  uint2 pw;
  pw.x = pack_bf2(s[0], s[1]);
  pw.y = pack_bf2(s[2], s[3]);
  const short4_t pf = as_short4(pw);
  // a running max that did not move leaves alpha exactly 1: skip the rescale
  // (after the first blocks it rarely moves)
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      oacc[dt][0] *= alpha; oacc[dt][1] *= alpha; oacc[dt][2] *= alpha; oacc[dt][3] *= alpha;
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const uint32_t* vp =
        reinterpret_cast<const uint32_t*>(vt + (16 * dt + col) * VT_DEC + 4 * ((G + (dt >> 1)) & 3));
    const uint2 vv = make_uint2(vp[0], vp[1]);
    oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_short4(vv), pf, oacc[dt], 0, 0, 0);
  }
  wave_lds_sync();
}

// KVM_STRIDED: K / V addressed by the strides of AttnArgs.  KVM_BF16 /
// KVM_FP8: addressed as rows of the model's cache layout (a.cache, paged
// when PAGED); FP8 rows are E4M3 codes with a scale per key, dequantised to
// bf16 in registers just before their block's products.  A 16-key block
// never straddles a page (pages hold a multiple of 64 positions), so one
// row lookup serves a block.
enum KvMode : int { KVM_STRIDED = 0, KVM_BF16 = 1, KVM_FP8 = 2 };

// Cache row of key jc (a wave-uniform block start) of sequence b, KV head g.
template <bool PAGED>
__device__ __forceinline__ int64_t block_row(const KvLayout& c, int b, int g, int jc) {
  if constexpr (PAGED) {
    // one page-table entry per block, the same for the whole wave: read
    // through the constant address space (the table does not change during
    // the kernel), so it is a scalar load, which the vector loads in flight
    // do not have to drain before
    typedef const __attribute__((address_space(4))) int ConstInt;
    const int e = __builtin_amdgcn_readfirstlane(b * static_cast<int>(c.tstride) + jc / c.P);
    const int page = ((ConstInt*)(c.table))[e];
    return static_cast<int64_t>(max(page, 0)) * c.nkv * c.P + g * c.P + jc % c.P;
  } else {
    return b * c.bs + g * c.hs + jc;
  }
}

// The key loop keeps three register sets of K / V loads: while one block is
// multiplied, the next two are in flight.  It runs whole groups of three
// blocks, then the last one or two, with no exit inside a group: with a
// single path around the loop the compiler's wait counts stay exact (exits
// in the middle of an unrolled body merge their pending loads into the
// loop head and make every iteration wait for more than its own block).
// The scheduling barriers keep each block's loads issued before the
// previous block's arithmetic.
#define Q2_DEC_RING(LOAD, BLOCK, S0, S1, S2)                                                          \
  {                                                                                                  \
    const int nblk = j0 < j_end ? (j_end - j0 + 63) >> 6 : 0;                                        \
    LOAD(S0, j0)                                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    LOAD(S1, j0 + 64)                                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                               \
      settle(qf[kk]);                                                                                \
      if (!rvalid) qf[kk] = z;                                                                       \
    }                                                                                                \
    int it = 0;                                                                                      \
    for (; it + 3 <= nblk; it += 3, j0 += 192) {                                                     \
      LOAD(S2, j0 + 128)                                                                             \
      __builtin_amdgcn_sched_barrier(0);                                                             \
      BLOCK(S0, j0)                                                                                  \
      LOAD(S0, j0 + 192)                                                                             \
      __builtin_amdgcn_sched_barrier(0);                                                             \
      BLOCK(S1, j0 + 64)                                                                             \
      LOAD(S1, j0 + 256)                                                                             \
      __builtin_amdgcn_sched_barrier(0);                                                             \
      BLOCK(S2, j0 + 128)                                                                            \
    }                                                                                                \
    if (it < nblk) BLOCK(S0, j0)                                                                     \
    if (it + 1 < nblk) BLOCK(S1, j0 + 64)                                                            \
  }

template <int KVM, bool PAGED>
__global__ __launch_bounds__(256, 2) void attn_decode_kernel(AttnArgs a, int chunk, int nsplit,
                                                             float* __restrict__ part_o, float2* __restrict__ part_ml) {
  // the V^T tiles of the key loop and the merge buffers of the four waves
  // are never live together (a barrier separates them): one LDS region
  constexpr int VT_BYTES = 4 * D * VT_DEC * 2, O_BYTES = 4 * D * 17 * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[VT_BYTES > O_BYTES ? VT_BYTES : O_BYTES];
  __shared__ float sM[4][16], sL[4][16];
  uint16_t (*sVt)[D * VT_DEC] = reinterpret_cast<uint16_t (*)[D * VT_DEC]>(smem);
  float (*sO)[D][17] = reinterpret_cast<float (*)[D][17]>(smem);

  const int split = blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / a.nkv;
  const int g = bg - b * a.nkv;
  const int group = a.nh / a.nkv;
  const int R = a.T * group;
  const int S = a.lens ? (a.lens[b] + a.T) : a.d_len ? (*a.d_len + a.T) : a.S;
  const int P = S - a.T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int G = lane >> 4;
  const int j_begin = split * chunk;
  const int j_end = min(j_begin + chunk, S);

  // query row `col` of this KV head's group: token t, head g*group + hh
  const bool rvalid = col < R;
  const int t = rvalid ? col / group : 0;
  const int head = g * group + (rvalid ? col - t * group : 0);
  const int lim = rvalid ? P + t : S - 1;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.q_bs + t * a.q_ts + head * a.q_hs;
  // loaded for every lane (rows past R read a valid head) and zeroed past R
  // only after the first key blocks' loads are out, so that no wait for them
  // comes first.  Fragment kk of lane group G holds d = kd(kk, G) .. + 7; the
  // K fragments use the same order (any order of d gives the same q . k).
  // bf16 rows: kd = 32 kk + 8 G, so one load instruction covers 64
  // contiguous bytes of each of 16 rows.  FP8 rows (128 bytes): kd = 64
  // (kk / 2) + 16 G + 8 (kk % 2), so a lane's four fragments are two 16-byte
  // loads and one instruction again covers 64 contiguous bytes of each row.
  uint4 qf[4];
  const uint4 z = {0, 0, 0, 0};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = ld16(qp + (KVM == KVM_FP8 ? 64 * (kk >> 1) + 16 * G + 8 * (kk & 1) : 32 * kk + 8 * G));

  uint16_t* vt = sVt[wave];

  float m_run = NEG_INF, l_run = 0.f;
  floatx4_t oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  int j0 = j_begin + 16 * wave;
  // Loads are unconditional: keys past the split's end re-read its last key
  // jl (their scores are masked and their probabilities exactly 0), and a
  // block's rows are looked up at its start clamped likewise.
  const int jl = max(j_end - 1, 0);
  if constexpr (KVM == KVM_FP8) {
  // K codes: two 16-byte loads per lane (the fragment order above); V:
  // 8-byte code loads; each key's scale
  const uint8_t* kc8 = static_cast<const uint8_t*>(a.cache.kc);
  const uint8_t* vc8 = static_cast<const uint8_t*>(a.cache.vc);
  struct Set8 {
    uint4 kr[2];
    uint2 vr[4];
    float ks, vs[4];
  };
#define Q2_DEC_LOAD8(S_, J0_)                                                                         \
  {                                                                                                  \
    const int jc_ = min((J0_), jl & ~15);                                                            \
    const int64_t r0_ = block_row<PAGED>(a.cache, b, g, jc_) - jc_;                                  \
    const int key_ = max(min((J0_) + col, jl), 0);                                                   \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) S_.kr[h] =                                         \
        *reinterpret_cast<const uint4*>(kc8 + (r0_ + key_) * D + 64 * h + 16 * G);                   \
    S_.ks = a.cache.ks[r0_ + key_];                                                                  \
    _Pragma("unroll") for (int s_ = 0; s_ < 4; ++s_) {                                               \
      const int vk_ = max(min((J0_) + 4 * G + s_, jl), 0);                                           \
      S_.vr[s_] = *reinterpret_cast<const uint2*>(vc8 + (r0_ + vk_) * D + 8 * col);                  \
      S_.vs[s_] = a.cache.vs[r0_ + vk_];                                                             \
    }                                                                                                \
  }
#define Q2_DEC_BLOCK8(S_, J0_)                                                                        \
  {                                                                                                  \
    uint4 kf_[4], vf_[4];                                                                            \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                                  \
      kf_[2 * h] = e4m3_dequant8(make_uint2(S_.kr[h].x, S_.kr[h].y), S_.ks);                         \
      kf_[2 * h + 1] = e4m3_dequant8(make_uint2(S_.kr[h].z, S_.kr[h].w), S_.ks);                     \
    }                                                                                                \
    _Pragma("unroll") for (int s_ = 0; s_ < 4; ++s_) vf_[s_] = e4m3_dequant8(S_.vr[s_], S_.vs[s_]);  \
    dec_block(kf_, vf_, qf, vt, (J0_), j_end, lim, a.scale, col, G, oacc, m_run, l_run);             \
  }
  Set8 s0, s1, s2;
  Q2_DEC_RING(Q2_DEC_LOAD8, Q2_DEC_BLOCK8, s0, s1, s2)
#undef Q2_DEC_LOAD8
#undef Q2_DEC_BLOCK8
  } else {
  // strided: row j of this head at base + j * stride; cache layout: rows of
  // D elements looked up per block.  K rows j0 + col: 4 x 16 B (d = 32kk +
  // 8G .. +8); V rows j0 + 4G + s, d-chunk 8*col.
  const bool lay = KVM == KVM_BF16;
  const uint16_t* kbase = lay ? static_cast<const uint16_t*>(a.cache.kc)
                              : static_cast<const uint16_t*>(a.k) + b * a.k_bs + g * a.k_hs;
  const uint16_t* vbase = lay ? static_cast<const uint16_t*>(a.cache.vc)
                              : static_cast<const uint16_t*>(a.v) + b * a.v_bs + g * a.v_hs;
  const int64_t kss = lay ? D : a.k_ss, vss = lay ? D : a.v_ss;
  struct Set16 {
    uint4 kf[4], vf[4];
  };
#define Q2_DEC_LOAD(S_, J0_)                                                                         \
  {                                                                                                  \
    int64_t r0_ = 0;                                                                                 \
    if (lay) {                                                                                       \
      const int jc_ = min((J0_), jl & ~15);                                                          \
      r0_ = block_row<PAGED>(a.cache, b, g, jc_) - jc_;                                              \
    }                                                                                                \
    const int key_ = max(min((J0_) + col, jl), 0);                                                   \
    _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) S_.kf[kk] =                                     \
        ld16(kbase + (r0_ + key_) * kss + 32 * kk + 8 * G);                                          \
    _Pragma("unroll") for (int s_ = 0; s_ < 4; ++s_) {                                               \
      const int vk_ = max(min((J0_) + 4 * G + s_, jl), 0);                                           \
      S_.vf[s_] = ld16(vbase + (r0_ + vk_) * vss + 8 * col);                                         \
    }                                                                                                \
  }
#define Q2_DEC_BLOCK(S_, J0_) dec_block(S_.kf, S_.vf, qf, vt, (J0_), j_end, lim, a.scale, col, G, oacc, m_run, l_run);
  Set16 s0, s1, s2;
  Q2_DEC_RING(Q2_DEC_LOAD, Q2_DEC_BLOCK, s0, s1, s2)
#undef Q2_DEC_LOAD
#undef Q2_DEC_BLOCK
  }
#undef Q2_DEC_RING
  __syncthreads();  // every wave is done with its V^T tile before sO reuses the region

  // merge the four waves
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sO[wave][16 * dt + 4 * G + i][col] = oacc[dt][i];
  if (G == 0) {
    sM[wave][col] = m_run;
    sL[wave][col] = l_run;
  }
  __syncthreads();
  const int r = threadIdx.x >> 4;          // row 0..15
  const int d0 = (threadIdx.x & 15) * 8;   // 8 consecutive d
  float mw[4];
  float M = NEG_INF;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = sM[w][r];
    M = fmaxf(M, mw[w]);
  }
  const float base = (M == NEG_INF) ? 0.f : M;
  float L = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float f = (mw[w] == NEG_INF) ? 0.f : __expf(mw[w] - base);
    L += f * sL[w][r];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] += f * sO[w][d0 + i][r];
  }
  if (nsplit == 1) {
    if (r < R) {
      const int tt = r / group;
      const int hh = g * group + (r - tt * group);
      uint16_t* op = static_cast<uint16_t*>(a.o) + b * a.o_bs + tt * a.o_ts + hh * a.o_hs + d0;
      const float inv = 1.f / L;
      uint4 w;
      w.x = pack_bf2(o[0] * inv, o[1] * inv);
      w.y = pack_bf2(o[2] * inv, o[3] * inv);
      w.z = pack_bf2(o[4] * inv, o[5] * inv);
      w.w = pack_bf2(o[6] * inv, o[7] * inv);
      *reinterpret_cast<uint4*>(op) = w;
    }
    return;
  }
  const int64_t slot = (static_cast<int64_t>(bg) * nsplit + split) * 16 + r;
  float* po = part_o + slot * D + d0;
#pragma unroll
  for (int i = 0; i < 8; ++i) po[i] = o[i];
  if ((threadIdx.x & 15) == 0) part_ml[slot] = make_float2(M, L);
}

template <int SMAX>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, int nsplit, const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml) {
  const int bg = blockIdx.x;
  const int b = bg / a.nkv;
  const int g = bg - b * a.nkv;
  const int group = a.nh / a.nkv;
  const int R = a.T * group;
  const int r = threadIdx.x >> 4;
  const int d0 = (threadIdx.x & 15) * 8;
  if (r >= R) return;
  const int64_t base_slot = static_cast<int64_t>(bg) * nsplit * 16 + r;
  // Up to SMAX splits' partials are loaded before any is used (clamped
  // indices: a fixed load count, one memory round trip); a split with no
  // keys has M = -inf, L = 0, o = 0 and weight 0.  The maximum is taken over
  // all splits first and the sums run in split order.
  float M = NEG_INF;
  float L = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  if (nsplit <= SMAX) {
    float2 ml[SMAX];
    float4 p0[SMAX], p1[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int64_t slot = base_slot + min(s, nsplit - 1) * 16;
      ml[s] = part_ml[slot];
      const float4* po = reinterpret_cast<const float4*>(part_o + slot * D + d0);
      p0[s] = po[0];
      p1[s] = po[1];
    }
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
      if (s < nsplit) M = fmaxf(M, ml[s].x);
    const float base = (M == NEG_INF) ? 0.f : M;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      if (s < nsplit) {
        const float f = ml[s].x == NEG_INF ? 0.f : __expf(ml[s].x - base);
        L += f * ml[s].y;
        o[0] += f * p0[s].x; o[1] += f * p0[s].y; o[2] += f * p0[s].z; o[3] += f * p0[s].w;
        o[4] += f * p1[s].x; o[5] += f * p1[s].y; o[6] += f * p1[s].z; o[7] += f * p1[s].w;
      }
    }
  } else {
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[base_slot + s * 16].x);
    const float base = (M == NEG_INF) ? 0.f : M;
#pragma unroll 4
    for (int s = 0; s < nsplit; ++s) {
      const float2 ml = part_ml[base_slot + s * 16];
      const float4* po = reinterpret_cast<const float4*>(part_o + (base_slot + s * 16) * D + d0);
      const float4 p0 = po[0], p1 = po[1];
      const float f = ml.x == NEG_INF ? 0.f : __expf(ml.x - base);
      L += f * ml.y;
      o[0] += f * p0.x; o[1] += f * p0.y; o[2] += f * p0.z; o[3] += f * p0.w;
      o[4] += f * p1.x; o[5] += f * p1.y; o[6] += f * p1.z; o[7] += f * p1.w;
    }
  }
  const int tt = r / group;
  const int hh = g * group + (r - tt * group);
  uint16_t* op = static_cast<uint16_t*>(a.o) + b * a.o_bs + tt * a.o_ts + hh * a.o_hs + d0;
  const float inv = 1.f / L;
  uint4 w;
  w.x = pack_bf2(o[0] * inv, o[1] * inv);
  w.y = pack_bf2(o[2] * inv, o[3] * inv);
  w.z = pack_bf2(o[4] * inv, o[5] * inv);
  w.w = pack_bf2(o[6] * inv, o[7] * inv);
  *reinterpret_cast<uint4*>(op) = w;
}

// ------------------------------------------------------------------ prefill (flash)
//
// 128 queries of one head per workgroup, 32 per wave, 32x32x16 bf16 MFMAs.
// Keys move in tiles of 64 through two LDS buffers: the next tile's K and V
// are loaded into registers while the current one is multiplied, then
// written to the other buffer (one barrier per tile).  Two workgroups per
// CU, so one's softmax arithmetic overlaps the other's products.
//
// S^T = K Q^T: K rows are the A operand, the wave's 32 queries the B operand
// (held in registers for the whole kernel), so element 4v+e of a 32x32 result
// is key 8v + 4*(lane/32) + e of query lane%32: each lane owns 16 scores of
// one query and a row's softmax needs one exchange with lane ^ 32.
// O^T = V^T P^T then takes a lane's own probabilities as its B operand: for
// key chunk c (16 keys) lane half h holds keys 16c + 4h + {0..3} and
// 16c + 8 + 4h + {0..3}.  V^T is written to LDS with bits 2 and 3 of the key
// index swapped, which makes exactly those eight keys contiguous for the A
// operand.  P is rounded to bf16 for that product.
//
// K rows are padded from 256 to 272 bytes (17 sixteen-byte slots), so every
// fragment read address is one per-lane base plus a constant.  V^T rows are
// padded to 72 keys (144 bytes) and the 8-key chunk k of row d sits at
// k ^ ((d / 16) % 8).  Measured on gfx950 (SQ_LDS_BANK_CONFLICT of
// single-wave probes of these exact access patterns): the K reads and writes
// take no conflict cycles; the V^T fragment reads and the 8-byte transposing
// writes conflict two ways.  160-byte V^T rows remove the read conflicts but
// cost 4 KB more LDS and measured no faster, so the smaller tile stays.

constexpr int PF_QB = 128;   // queries per workgroup
constexpr int PF_KT = 64;    // keys per tile
constexpr int PF_VT = 72;    // bf16 per V^T LDS row
constexpr int PF_KR = 17;    // 16-byte slots per K LDS row

__device__ __forceinline__ int pf_keyperm(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// One 64-key tile of the prefill loop for the calling wave: S^T from the
// K tile, online softmax of the wave's 32 queries, O^T += V^T P^T.
// The running max and sum are kept in base-2 units (scale * log2 e folded
// in), so each probability is one fma and one exp2, and the sum is taken
// over the bf16-rounded probabilities that the V product uses; a tile entirely inside every query's causal
// window skips the mask; the accumulator is rescaled only when some lane's
// running maximum moved (alpha == 1 exactly otherwise).  exp2(-inf) = 0
// covers masked keys.
__device__ __forceinline__ void pf_tile(const uint4* __restrict__ sKb, const uint16_t* __restrict__ sVtb, int j0,
                                        bool full, int lim, float sl2, int qr, int hl, const uint4 (&qf)[8],
                                        floatx16_t (&oacc)[4], float& m_run, float& l_run) {
  // S^T for two 32-key halves
  floatx16_t sacc[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[kh][e] = 0.f;
    // all eight fragments are read before the first product, so the reads
    // overlap one another instead of each product waiting on its own
    const uint4* kr = sKb + (32 * kh + qr) * PF_KR + hl;
    uint4 kf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[ks] = kr[2 * ks];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[ks]), as_bf16x8(qf[ks]), sacc[kh], 0, 0, 0);
  }
  // schedule: the first half's eight reads, then its products each followed
  // by one read of the second half, then the second half's products
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  // running max of query qr's raw scores (lanes qr and qr + 32), masked
  // keys at -inf; the scale goes into one fma per probability:
  // p = exp2(s * scale * log2 e - m)
  float mt = NEG_INF;
  if (full) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kh][i]);
  } else {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kj = j0 + 32 * kh + 8 * v + 4 * hl + e;
          const float x = kj <= lim ? sacc[kh][4 * v + e] : NEG_INF;
          sacc[kh][4 * v + e] = x;
          mt = fmaxf(mt, x);
        }
  }
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float m_new = fmaxf(m_run, mt * sl2);
  const float base = m_new == NEG_INF ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - base);
  // the row sum adds the bf16 probabilities that multiply V, two per dot2
  float ps = 0.f;
  const bf16x2_hw ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  bf16x8_t pf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 w;
    uint32_t* ws = &w.x;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int v = 2 * (c & 1) + half;
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(sacc[c >> 1][4 * v + e], sl2, -base));
      ws[2 * half] = pack_bf2(pr[0], pr[1]);
      ws[2 * half + 1] = pack_bf2(pr[2], pr[3]);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_hw, ws[2 * half]), ones, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_hw, ws[2 * half + 1]), ones, ps, false);
    }
    pf[c] = as_bf16x8(w);
  }
  ps += __shfl_xor(ps, 32, 64);
  l_run = l_run * alpha + ps;
  m_run = m_new;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
  }
  // O^T += V^T P^T.  Row 32 dt + qr has swizzle key 2 dt + qr / 16, so the
  // lane's chunk 2 c + hl sits at 2 (c ^ dt) + (hl ^ qr / 16): a per-lane
  // base plus a constant for each (dt, c).
  const uint16_t* vl = sVtb + qr * PF_VT + 8 * (hl ^ (qr >> 4));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    uint4 vf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) vf[c] = *reinterpret_cast<const uint4*>(vl + 32 * dt * PF_VT + 16 * (c ^ dt));
#pragma unroll
    for (int c = 0; c < 4; ++c)
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[c]), pf[c], oacc[dt], 0, 0, 0);
  }
  // schedule: four reads ahead of the products
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Grid (nh, items, B).  The nsq last query blocks (the longest causal rows)
// are split in two halves of their key tiles, items 2 i and 2 i + 1 for
// block nqb - 1 - i; each half leaves its unnormalised output and running
// (max, sum) in base-2 units at part_o / part_ml, merged by
// attn_prefill_combine.  The other blocks follow, last first, whole.
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(AttnArgs a, int nsq, float* __restrict__ part_o,
                                                              float2* __restrict__ part_ml) {
  __shared__ uint4 sK[2][PF_KT * PF_KR];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][D * PF_VT];

  const int nqb = (a.T + PF_QB - 1) / PF_QB;
  // heads vary fastest, query blocks from the last (longest causal rows)
  // down: workgroups are dispatched roughly longest first, so the short
  // blocks dispatched last share a CU with a long one only briefly
  const int y = blockIdx.y;
  const int part = y < 2 * nsq ? (y & 1) : -1;
  const int qb = y < 2 * nsq ? nqb - 1 - (y >> 1) : nqb - 1 - nsq - (y - 2 * nsq);
  const int h = blockIdx.x;
  const int b = blockIdx.z;
  const int group = a.nh / a.nkv;
  const int g = h / group;
  const int S = a.d_len ? (*a.d_len + a.T) : a.S;
  const int P = S - a.T;
  const int q0 = qb * PF_QB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;      // lane half
  const int qr = lane & 31;      // query row within the wave

  const int tq = q0 + 32 * wave + qr;
  const bool qvalid = tq < a.T;
  const int lim = qvalid ? P + tq : S - 1;
  uint4 qf[8];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.q_bs +
                         static_cast<int64_t>(qvalid ? tq : 0) * a.q_ts + h * a.q_hs;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = ld16(qp + 16 * ks + 8 * hl);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) settle(qf[ks]);
  }

  const int kv_end = min(S, P + min(q0 + PF_QB, a.T));
  const int wave_first = q0 + 32 * wave;
  const int wave_lim = wave_first < a.T ? P + min(wave_first + 31, a.T - 1) : -1;

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.k_bs + g * a.k_hs;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.v_bs + g * a.v_hs;

  // tile loads: K chunk q = tid + 256 i is key q / 16, chunk q % 16; V: this
  // thread's 8-wide d chunk vc of keys 4 vg .. 4 vg + 3, where the 16-lane
  // groups 0..3 of wave w take key groups 4 w + {0, 2, 1, 3} (groups 0 and
  // 2 share an 8-key chunk after the key permutation).
  const int vc = tid & 15, vq = (tid >> 4) & 3;
  const int vg = 4 * (tid >> 6) + (((vq & 1) << 1) | (vq >> 1));
  // The loads go through buffer descriptors whose base is the tile's first
  // key and whose range ends at kv_end: each lane's byte offset is fixed for
  // the kernel, and keys past kv_end read as zeros (hardware range check), so
  // their scores are masked and their probabilities exactly zero.  The host
  // keeps kv_end * row stride below 2^31 bytes.
  const int kbytes = static_cast<int>(a.k_ss) * 2, vbytes = static_cast<int>(a.v_ss) * 2;
  int koff[4], voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    koff[i] = ((tid >> 4) + 16 * i) * kbytes + (tid & 15) * 16;
    voff[i] = (4 * vg + i) * vbytes + vc * 16;
  }
  uint4 rk[4], rv[4];
#define Q2_PF_LOAD(RK_, RV_, J0_)                                                                    \
  {                                                                                                  \
    const int j_ = (J0_);                                                                            \
    const int n_ = max(kv_end - j_, 0);                                                              \
    const __amdgpu_buffer_rsrc_t kr_ = __builtin_amdgcn_make_buffer_rsrc(                            \
        const_cast<uint16_t*>(kbase) + static_cast<int64_t>(j_) * a.k_ss, 0, n_ * kbytes, 0x00020000); \
    const __amdgpu_buffer_rsrc_t vr_ = __builtin_amdgcn_make_buffer_rsrc(                            \
        const_cast<uint16_t*>(vbase) + static_cast<int64_t>(j_) * a.v_ss, 0, n_ * vbytes, 0x00020000); \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                    \
      RK_[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr_, koff[i], 0, 0));  \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                    \
      RV_[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr_, voff[i], 0, 0));  \
  }
#define Q2_PF_STORE(BUF_, RK_, RV_)                                                                  \
  {                                                                                                  \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                  \
      const int q_ = tid + 256 * i;                                                                  \
      const int r_ = q_ >> 4;                                                                        \
      sK[BUF_][r_ * PF_KR + (q_ & 15)] = RK_[i];                                                     \
    }                                                                                                \
    store_vt4<true>(sVt[BUF_], PF_VT, 8 * vc, pf_keyperm(4 * vg) ^ (((vc >> 1) & 7) << 3), RV_);           \
  }

  float m_run = NEG_INF, l_run = 0.f;
  floatx16_t oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;

  const int ntiles = (kv_end + PF_KT - 1) / PF_KT;
  const int jt0 = part == 1 ? ntiles / 2 : 0;
  const int jt1 = part == 0 ? ntiles / 2 : ntiles;
  // The loads are issued unconditionally (past kv_end they read zeros), so
  // the compiler's count of loads in flight does not depend on the path.
  // The wave's first query decides whether a tile needs the mask.
  const float sl2 = a.scale * 1.4426950408889634f;
  const int wave_full = wave_first < a.T ? P + wave_first : -1;
  Q2_PF_LOAD(rk, rv, jt0 * PF_KT)
  Q2_PF_STORE(0, rk, rv)
  __syncthreads();
  for (int jt = jt0; jt < jt1; ++jt) {
    const int buf = (jt - jt0) & 1;
    const int j0 = jt * PF_KT;
    Q2_PF_LOAD(rk, rv, j0 + PF_KT)
    if (j0 <= wave_lim)
      pf_tile(sK[buf], sVt[buf], j0, j0 + PF_KT - 1 <= wave_full, lim, sl2, qr, hl, qf, oacc, m_run, l_run);
    if (jt + 1 < jt1) Q2_PF_STORE(buf ^ 1, rk, rv)
    __syncthreads();
  }
#undef Q2_PF_LOAD
#undef Q2_PF_STORE
  if (!qvalid) return;
  if (part >= 0) {
    // lane half hl holds d = 32 dt + 8 v + 4 hl .. + 3 of query row 32 wave + qr
    const int64_t pi = ((static_cast<int64_t>(b) * a.nh + h) * nsq + (nqb - 1 - qb)) * 2 + part;
    const int r = 32 * wave + qr;
    float* po = part_o + (pi * PF_QB + r) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        *reinterpret_cast<float4*>(po + 32 * dt + 8 * v + 4 * hl) =
            make_float4(oacc[dt][4 * v], oacc[dt][4 * v + 1], oacc[dt][4 * v + 2], oacc[dt][4 * v + 3]);
    if (hl == 0) part_ml[pi * PF_QB + r] = make_float2(m_run, l_run);
    return;
  }
  const float inv = 1.f / l_run;
  uint16_t* op = static_cast<uint16_t*>(a.o) + b * a.o_bs + static_cast<int64_t>(tq) * a.o_ts + h * a.o_hs;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      uint2 w;
      w.x = pack_bf2(oacc[dt][4 * v] * inv, oacc[dt][4 * v + 1] * inv);
      w.y = pack_bf2(oacc[dt][4 * v + 2] * inv, oacc[dt][4 * v + 3] * inv);
      *reinterpret_cast<uint2*>(op + 32 * dt + 8 * v + 4 * hl) = w;
    }
}

// Merges the two halves of each split query block.  Workgroup x of a head
// takes rows 16 (x % 8) .. + 15 of block nqb - 1 - x / 8; 16 adjacent lanes
// cover a row's 128 features in 32-byte pieces, so every load instruction
// reads whole rows.
__global__ __launch_bounds__(256) void attn_prefill_combine(AttnArgs a, int nsq, const float* __restrict__ part_o,
                                                            const float2* __restrict__ part_ml) {
  const int i = blockIdx.x >> 3, h = blockIdx.y, b = blockIdx.z;
  const int nqb = (a.T + PF_QB - 1) / PF_QB;
  const int qb = nqb - 1 - i;
  const int r = (blockIdx.x & 7) * 16 + (threadIdx.x >> 4);
  const int d0 = (threadIdx.x & 15) * 8;
  const int tq = qb * PF_QB + r;
  if (tq >= a.T) return;
  const int64_t pi = ((static_cast<int64_t>(b) * a.nh + h) * nsq + i) * 2;
  const float2 ml0 = part_ml[pi * PF_QB + r], ml1 = part_ml[(pi + 1) * PF_QB + r];
  const float4* p0 = reinterpret_cast<const float4*>(part_o + (pi * PF_QB + r) * D + d0);
  const float4* p1 = reinterpret_cast<const float4*>(part_o + ((pi + 1) * PF_QB + r) * D + d0);
  const float4 x0 = p0[0], x1 = p0[1], y0 = p1[0], y1 = p1[1];
  // the first half always holds key 0; the second may hold no visible key
  const float mx = fmaxf(ml0.x, ml1.x);
  const float w0 = __builtin_amdgcn_exp2f(ml0.x - mx);
  const float w1 = ml1.x == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(ml1.x - mx);
  const float inv = 1.f / (w0 * ml0.y + w1 * ml1.y);
  uint4 w;
  w.x = pack_bf2((w0 * x0.x + w1 * y0.x) * inv, (w0 * x0.y + w1 * y0.y) * inv);
  w.y = pack_bf2((w0 * x0.z + w1 * y0.z) * inv, (w0 * x0.w + w1 * y0.w) * inv);
  w.z = pack_bf2((w0 * x1.x + w1 * y1.x) * inv, (w0 * x1.y + w1 * y1.y) * inv);
  w.w = pack_bf2((w0 * x1.z + w1 * y1.z) * inv, (w0 * x1.w + w1 * y1.w) * inv);
  uint16_t* op = static_cast<uint16_t*>(a.o) + b * a.o_bs + static_cast<int64_t>(tq) * a.o_ts + h * a.o_hs + d0;
  *reinterpret_cast<uint4*>(op) = w;
}

// Query blocks of a prefill call whose key ranges are split (host view of
// the lengths): those with more than half the key tiles of the last block.
// Only when the longest block (at least 8 tiles) would outlast the whole
// grid's work spread over two workgroups per CU by half again: otherwise
// the chip is full anyway and the split's partials only cost traffic.
int prefill_split_blocks(int B, int nh, int T, int S) {
  const int nqb = cdiv(T, PF_QB);
  const int P = S - T;
  auto nt = [&](int qb) { return cdiv(std::min(S, P + std::min((qb + 1) * PF_QB, T)), PF_KT); };
  const int top = nt(nqb - 1);
  if (top < 8) return 0;
  int64_t work = 0;
  for (int qb = 0; qb < nqb; ++qb) work += nt(qb);
  work *= static_cast<int64_t>(B) * nh;
  if (2 * static_cast<int64_t>(top) * 512 <= 3 * work) return 0;
  int n = 0;
  for (int qb = nqb - 1; qb >= 0 && nt(qb) > cdiv(top, 2); --qb) ++n;
  return n;
}

size_t prefill_split_bytes(int B, int nh, int nsq) {
  return static_cast<size_t>(B) * nh * nsq * 2 * PF_QB * (D * sizeof(float) + sizeof(float2));
}

// ------------------------------------------------------------------ float32

__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  extern __shared__ float sp[];
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  const int group = a.nh / a.nkv;
  const int g = h / group;
  const int S = a.d_len ? (*a.d_len + a.T) : a.S;
  const int vis = S - a.T + t + 1;
  const float* q = static_cast<const float*>(a.q) + b * a.q_bs + static_cast<int64_t>(t) * a.q_ts + h * a.q_hs;
  const float* kb = static_cast<const float*>(a.k) + b * a.k_bs + g * a.k_hs;
  const float* vb = static_cast<const float*>(a.v) + b * a.v_bs + g * a.v_hs;
  float mx = NEG_INF;
  for (int j = lane; j < vis; j += 64) {
    const float* k = kb + static_cast<int64_t>(j) * a.k_ss;
    float s = 0.f;
    for (int i = 0; i < a.d; ++i) s = fmaf(q[i], k[i], s);
    s *= a.scale;
    sp[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  float sum = 0.f;
  for (int j = lane; j < vis; j += 64) {
    const float p = __expf(sp[j] - mx);
    sp[j] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  __syncthreads();
  float* o = static_cast<float*>(a.o) + b * a.o_bs + static_cast<int64_t>(t) * a.o_ts + h * a.o_hs;
  for (int i = lane; i < a.d; i += 64) {
    float acc = 0.f;
    for (int j = 0; j < vis; ++j) acc = fmaf(sp[j], vb[static_cast<int64_t>(j) * a.v_ss + i], acc);
    o[i] = acc / sum;
  }
}

struct DecodePlan {
  int chunk, nsplit;
};

// Splits per (sequence, KV head): as many as keep the grid within two
// workgroups per CU (512 in all; each split's partials cost a write and a
// read), each of at least 64 keys; then the split lengths are evened out
// (multiples of 64 keys).  Filling the two slots of every CU matters for
// long caches: at 1.5 workgroups per CU half the CUs stream twice the keys.
// Once 8 splits already give every CU a workgroup (B * nkv >= 32), at most 8:
// the merge then loads every split's partials in one memory round trip
// (attn_combine_kernel<8>) and there are fewer partials (7B batch-8 decode at
// 1280 keys: 7 splits instead of 10, +1.4 %).
DecodePlan plan_decode(int B, int s_max, int nkv) {
  DecodePlan p;
  const int64_t heads = static_cast<int64_t>(B) * nkv;
  int64_t fit = std::max<int64_t>(1, 512 / heads);
  if (heads * 8 >= 256) fit = std::min<int64_t>(fit, 8);
  const int nsplit = static_cast<int>(std::min<int64_t>(std::max(1, cdiv(s_max, 64)), fit));
  p.chunk = cdiv(cdiv(s_max, nsplit), 64) * 64;
  p.nsplit = std::max(1, cdiv(s_max, p.chunk));
  return p;
}

}  // namespace

int attention_decode_splits(int B, int T, int s_max, int nh, int nkv, int d) {
  if (d != D || T * (nh / nkv) > 16) return 0;
  return plan_decode(B, s_max, nkv).nsplit;
}

size_t attention_scratch_bytes(int B, int T, int s_max, int nh, int nkv, int d) {
  if (d != D) return 0;
  if (T * (nh / nkv) > 16) return prefill_split_bytes(B, nh, cdiv(T, PF_QB));  // at most every block split
  DecodePlan p = plan_decode(B, s_max, nkv);
  if (p.nsplit == 1) return 0;
  const size_t slots = static_cast<size_t>(B) * nkv * p.nsplit * 16;
  return slots * (D * sizeof(float) + sizeof(float2));
}

q2_status attention_bf16(const AttnArgs& a, hipStream_t s) {
  Q2_CHECK(a.d == D, Q2_ESHAPE, "bf16 attention supports head_dim 128 only (got %d)", a.d);
  if (a.B == 0 || a.T == 0) return Q2_OK;
  const int group = a.nh / a.nkv;
  if (a.T * group <= 16) {
    const int s_max = (a.d_len || a.lens) ? a.s_max : a.S;
    DecodePlan p = plan_decode(a.B, s_max, a.nkv);
    float* part_o = nullptr;
    float2* part_ml = nullptr;
    if (p.nsplit > 1 && a.unsplit_if_short) {
      const size_t slots = static_cast<size_t>(a.B) * a.nkv * p.nsplit * 16;
      if (!a.scratch || a.scratch_bytes < slots * (D * sizeof(float) + sizeof(float2))) {
        p.nsplit = 1;
        p.chunk = cdiv(s_max, 64) * 64;
      }
    }
    if (p.nsplit > 1) {
      const size_t slots = static_cast<size_t>(a.B) * a.nkv * p.nsplit * 16;
      const size_t need = slots * (D * sizeof(float) + sizeof(float2));
      Q2_CHECK(a.scratch && a.scratch_bytes >= need, Q2_EINVAL, "attention: split-KV scratch too small");
      part_o = static_cast<float*>(a.scratch);
      part_ml = reinterpret_cast<float2*>(part_o + slots * D);
    }
    const dim3 grid(p.nsplit, a.B * a.nkv);
    const bool paged = a.use_cache && a.cache.table;
    if (a.use_cache && a.cache.fp8 && paged)
      hipLaunchKernelGGL((attn_decode_kernel<KVM_FP8, true>), grid, dim3(256), 0, s, a, p.chunk, p.nsplit, part_o,
                         part_ml);
    else if (a.use_cache && a.cache.fp8)
      hipLaunchKernelGGL((attn_decode_kernel<KVM_FP8, false>), grid, dim3(256), 0, s, a, p.chunk, p.nsplit, part_o,
                         part_ml);
    else if (paged)
      hipLaunchKernelGGL((attn_decode_kernel<KVM_BF16, true>), grid, dim3(256), 0, s, a, p.chunk, p.nsplit, part_o,
                         part_ml);
    else if (a.use_cache)
      hipLaunchKernelGGL((attn_decode_kernel<KVM_BF16, false>), grid, dim3(256), 0, s, a, p.chunk, p.nsplit, part_o,
                         part_ml);
    else
      hipLaunchKernelGGL((attn_decode_kernel<KVM_STRIDED, false>), grid, dim3(256), 0, s, a, p.chunk, p.nsplit,
                         part_o, part_ml);
    Q2_TRY(check_launch("attn_decode"));
    if (p.nsplit > 1 && !a.leave_partials) {
      if (p.nsplit <= 8)
        hipLaunchKernelGGL(attn_combine_kernel<8>, dim3(a.B * a.nkv), dim3(256), 0, s, a, p.nsplit, part_o, part_ml);
      else
        hipLaunchKernelGGL(attn_combine_kernel<16>, dim3(a.B * a.nkv), dim3(256), 0, s, a, p.nsplit, part_o, part_ml);
      Q2_TRY(check_launch("attn_combine"));
    }
    return Q2_OK;
  }
  Q2_CHECK(!a.use_cache && !a.lens, Q2_EINVAL,
           "prefill attention reads strided bf16 K/V of equal-length sequences (expand the cache first)");
  // the prefill kernel's buffer loads address a head's keys with 32-bit
  // byte offsets
  const int64_t max_keys = a.d_len ? a.s_max : a.S;
  Q2_CHECK(max_keys * std::max(a.k_ss, a.v_ss) * 2 < (int64_t(1) << 31), Q2_ESHAPE,
           "bf16 prefill attention: %lld keys at row strides %lld / %lld exceed 2 GiB per head",
           static_cast<long long>(max_keys), static_cast<long long>(a.k_ss), static_cast<long long>(a.v_ss));
  const int nqb = cdiv(a.T, PF_QB);
  int nsq = prefill_split_blocks(a.B, a.nh, a.T, a.S);
  if (nsq && (!a.scratch || a.scratch_bytes < prefill_split_bytes(a.B, a.nh, nsq))) nsq = 0;
  float* part_o = static_cast<float*>(a.scratch);
  float2* part_ml =
      nsq ? reinterpret_cast<float2*>(part_o + static_cast<size_t>(a.B) * a.nh * nsq * 2 * PF_QB * D) : nullptr;
  hipLaunchKernelGGL(attn_prefill_kernel, dim3(a.nh, nqb + nsq, a.B), dim3(256), 0, s, a, nsq, part_o, part_ml);
  Q2_TRY(check_launch("attn_prefill"));
  if (nsq == 0) return Q2_OK;
  hipLaunchKernelGGL(attn_prefill_combine, dim3(nsq * 8, a.nh, a.B), dim3(256), 0, s, a, nsq, part_o, part_ml);
  return check_launch("attn_prefill_combine");
}

q2_status attention_f32(const AttnArgs& a, hipStream_t s) {
  Q2_CHECK(a.d <= 256, Q2_ESHAPE, "fp32 attention supports head_dim <= 256");
  if (a.B == 0 || a.T == 0) return Q2_OK;
  const int s_max = a.d_len ? a.s_max : a.S;
  Q2_CHECK(s_max <= 16384, Q2_ESHAPE, "fp32 attention supports at most 16384 keys");
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.T, a.nh, a.B), dim3(64), s_max * sizeof(float), s, a);
  return check_launch("attn_f32");
}

}  // namespace q2
