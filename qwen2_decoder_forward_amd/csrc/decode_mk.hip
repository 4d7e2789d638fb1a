// Persistent decode step: the whole decoder forward for one new token per
// sequence (batch <= 16, bf16, head_dim 128) in one cooperative launch.
//
// Why: at batch 1 a decode step is ~170 dependent kernels of a few
// microseconds each, and every one of them ramps the chip up and drains it.
// Here one workgroup per CU stays resident for the whole step and the stages
// are separated by grid barriers; each workgroup issues the weight loads of
// its next stage before it waits at the barrier, so the barrier latency
// overlaps the start of the next weight stream.
//
// Stages per layer (the operator chain of "LLAISYS 训练营结项报告", section
// 3.2, fourth layer, fused):
//   A  QKV GEMV: input RMSNorm in the prologue (for layers > 0 the previous
//      layer's split-K down partials and residual are summed there as well),
//      bias, RoPE, q stored, k and v written into the KV cache
//   B  split-KV attention, one wave per (sequence, KV head, key chunk)
//   C  o_proj GEMV: prologue merges the attention partials; epilogue adds the
//      residual
//   D  gate/up GEMV: post-attention RMSNorm in the prologue, SwiGLU epilogue
//   E  down GEMV, split over K into float32 partials
// then the final RMSNorm + LM head with the packed argmax, and one workgroup
// picks the next token.
//
// Memory coherence across the 8 XCDs (each with its own L2): every
// activation buffer is written exactly once per launch, with agent-scope
// (write-through) stores, before any workgroup reads it, so plain cached
// loads never see a stale line; weights and KV rows written by earlier
// launches are plain loads too.  The barrier flags use agent-scope loads and
// stores.  Every wait is bounded: a barrier that times out sets an error word
// and the step runs to its end without waiting (the results are then
// garbage, and q2_model_check reports the error).
#include <algorithm>

#include "decode_mk.hpp"

// Timing hook: expands to nothing unless a measurement harness defines it.
#ifndef MK_TRACE_POINT
#define MK_TRACE_POINT(k)
#endif
#ifndef MK_TRACE_SUB
#define MK_TRACE_SUB(step, k)
#endif

namespace q2 {

namespace {

constexpr int MK_WAVES = MK_THREADS / 64;
constexpr int KB = 128;           // K per GEMV block
constexpr int D = 128;
constexpr int VT = 20;            // bf16 per V^T LDS row in the attention stage
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr long SPIN_MAX = 1L << 20;

// Plain loads from global memory (pointers read from the layer table carry
// no address space; the casts keep these global rather than flat loads).
typedef unsigned int gu4 __attribute__((ext_vector_type(4)));
typedef float gf4 __attribute__((ext_vector_type(4)));
typedef float gf2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  const gu4 v = *(const __attribute__((address_space(1))) gu4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 lds16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ float4 ldg4f(const float* p) {
  const gf4 v = *(const __attribute__((address_space(1))) gf4*)(p);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float2 ldg2f(const float2* p) {
  const gf2 v = *(const __attribute__((address_space(1))) gf2*)(p);
  return make_float2(v.x, v.y);
}
template <typename T>
__device__ __forceinline__ T ldg(const T* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}

__device__ __forceinline__ void co_st16(uint16_t* p, float v) {
  __hip_atomic_store(p, f2bf(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void co_st32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void co_stf(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned co_ld32(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ grid barrier
//
// Every workgroup publishes the barrier's epoch in its own flag (arrive);
// workgroup 0 waits for all flags and then publishes the epoch in the release
// word, which the others wait for (wait).  (One release line per workgroup
// measured slower here: the 256 stores delay the release.)  A thread's stores have completed
// (s_waitcnt) before its workgroup's flag is written.  Between arrive and wait
// a workgroup may issue loads that do not depend on the other workgroups (the
// next stage's weights), so that they overlap the wait.
__device__ __forceinline__ void grid_arrive(const MkArgs& a, unsigned& epoch) {
  ++epoch;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) co_st32(a.bar_flags + blockIdx.x, epoch);
}

__device__ void grid_wait(const MkArgs& a, unsigned epoch, bool& dead) {
  if (threadIdx.x < 64 && !dead) {
    const int lane = threadIdx.x;
    long spins = 0;
    if (blockIdx.x == 0) {
      for (;;) {
        bool ok = true;
        for (int i = lane; i < static_cast<int>(gridDim.x); i += 64)
          ok &= static_cast<int>(co_ld32(a.bar_flags + i) - epoch) >= 0;
        if (__all(ok)) break;
        if (++spins > SPIN_MAX) {
          dead = true;
          break;
        }
      }
      if (lane == 0) co_st32(a.bar_release, epoch);
    } else {
      for (;;) {
        if (static_cast<int>(co_ld32(a.bar_release) - epoch) >= 0) break;
        if (++spins > SPIN_MAX) {
          dead = true;
          break;
        }
      }
    }
    if (dead && lane == 0) co_st32(a.err, 1u);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ GEMV pieces
//
// Most GEMVs are split by 16-row weight tiles, each tile handled by ONE wave
// over the whole K: lane (row r = lane % 16, group g = lane / 16) loads four
// 16-byte pieces of weight row n0 + r per 128-wide K block and feeds four
// 16x16x32 MFMAs (weight rows = A operand, token rows from LDS = B operand).
// The wave keeps two rounds of RB blocks in flight and applies the epilogue
// straight from its accumulators (lane l holds features n0 + 4 (l / 16) + i of
// token l % 16), so the waves of a workgroup never wait for one another.
// Tiles go round-robin over the workgroups first, then over their waves.

constexpr int RB = 2;  // K blocks per load round of a wave

#define MK_LOAD(R_, WP_, WOK_, KB0_)                                                                 \
  _Pragma("unroll") for (int b_ = 0; b_ < RB; ++b_) {                                               \
    const int kk_ = (KB0_) + b_;                                                                    \
    if (kk_ < nkb) {                                                                                \
      _Pragma("unroll") for (int u_ = 0; u_ < 4; ++u_) {                                            \
        const int k_ = kk_ * KB + 32 * u_ + 8 * g;                                                  \
        R_[b_][u_] = ld16((WP_) + (((WOK_) && k_ < K) ? static_cast<int64_t>(kk_) * KB + 32 * u_ : 0)); \
      }                                                                                             \
    }                                                                                               \
  }
#define MK_MMA_LDS(R_, WOK_, KB0_)                                                                   \
  _Pragma("unroll") for (int b_ = 0; b_ < RB; ++b_) {                                               \
    const int kk_ = (KB0_) + b_;                                                                    \
    if (kk_ < nkb) {                                                                                \
      _Pragma("unroll") for (int u_ = 0; u_ < 4; ++u_) {                                            \
        const int k_ = kk_ * KB + 32 * u_ + 8 * g;                                                  \
        const bool kin_ = k_ < K;                                                                   \
        uint4 xv_ = lds16(xps + ((xok && kin_) ? kk_ * KB + 32 * u_ : -8 * g));                     \
        if (!(xok && kin_)) xv_ = z4;                                                               \
        const uint4 wv_ = ((WOK_) && kin_) ? R_[b_][u_] : z4;                                       \
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv_), as_bf16x8(xv_), acc, 0, 0, 0); \
      }                                                                                             \
    }                                                                                               \
  }

// rnd(x * inv * w) for 8 bf16 lanes.
__device__ __forceinline__ uint4 norm8(uint4 x, uint4 w, float inv) {
  uint4 r;
  const uint32_t* xs = &x.x;
  const uint32_t* ws = &w.x;
  uint32_t* rs = &r.x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    rs[i] = pack_bf2((bf_lo(xs[i]) * inv) * bf_lo(ws[i]), (bf_hi(xs[i]) * inv) * bf_hi(ws[i]));
  return r;
}

__device__ __forceinline__ float sumsq8(uint4 x) {
  const uint32_t* xs = &x.x;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = bf_lo(xs[i]), b = bf_hi(xs[i]);
    s += a * a + b * b;
  }
  return s;
}

// Residual rows entering a layer (or the final norm): the embedding (layer 0)
// or rnd(x_mid + rnd(sum of the down partials)), 8 features at k.
__device__ __forceinline__ uint4 resid_row8(const MkArgs& a, int l, int m, int k) {
  if (l == 0) {
    const int64_t id = ldg(a.ids_buf + m);
    return ld16(a.embed + id * a.H + k);
  }
  const uint4 xm = ld16(a.xmid + (static_cast<int64_t>(l - 1) * a.B + m) * a.H + k);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* pp = a.down_part + static_cast<int64_t>(l - 1) * a.down_splits * a.B * a.H;
  // all partial loads issued before the sums (MK_DOWN_SPLITS at most), summed in split order
  float4 p0[MK_DOWN_SPLITS], p1[MK_DOWN_SPLITS];
#pragma unroll
  for (int s = 0; s < MK_DOWN_SPLITS; ++s) {
    if (s < a.down_splits) {
      const float* q = pp + (static_cast<int64_t>(s) * a.B + m) * a.H + k;
      p0[s] = ldg4f(q);
      p1[s] = ldg4f(q + 4);
    }
  }
#pragma unroll
  for (int s = 0; s < MK_DOWN_SPLITS; ++s) {
    if (s < a.down_splits) {
      acc[0] += p0[s].x; acc[1] += p0[s].y; acc[2] += p0[s].z; acc[3] += p0[s].w;
      acc[4] += p1[s].x; acc[5] += p1[s].y; acc[6] += p1[s].z; acc[7] += p1[s].w;
    }
  }
  const uint32_t* xs = &xm.x;
  uint4 r;
  uint32_t* rs = &r.x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    rs[i] = pack_bf2(bf_lo(xs[i]) + round_bf(acc[2 * i]), bf_hi(xs[i]) + round_bf(acc[2 * i + 1]));
  return r;
}

// Prologue of the norm-fused GEMVs: rmsnorm of the B token rows into s_x
// (row stride ld_s).  src 0: the residual entering layer l (the embedding for
// l = 0, else the reduced down partials plus x_mid; workgroup 0 also stores it
// in xres[l]); src 1: x_mid of layer l.  Rows are split over the waves (8 / B
// waves per row when B < 8); each row's sum of squares is combined in a fixed
// order.
__device__ void stage_norm(const MkArgs& a, int l, int src, const uint16_t* w_norm, uint16_t* s_x, int ld_s,
                           float* s_ss, int wave, int lane) {
  constexpr int MAXC = MK_NORM_CHUNKS;  // chunks per lane and row (H / 8 <= 64 * MAXC * waves per row)
  const int K = a.H, CPR = K / 8;
  const int wpr = a.B >= MK_WAVES ? 1 : MK_WAVES / a.B;
  const int rows_per_pass = MK_WAVES / wpr;
  const int part = wave % wpr;
  uint16_t* s_w = s_x + a.B * ld_s;  // the norm weights, shared by all rows
  // the weights go to LDS while the rows load (every load issued up front)
  for (int c = threadIdx.x; c < CPR; c += MK_THREADS)
    *reinterpret_cast<uint4*>(s_w + 8 * c) = ld16(w_norm + 8 * c);
  for (int m0 = 0; m0 < a.B; m0 += rows_per_pass) {
    const int m = m0 + wave / wpr;
    const bool active = m < a.B && wave / wpr < rows_per_pass;
    float ss = 0.f;
    if (active) {
      uint16_t* row = s_x + m * ld_s;
      uint4 xs[MAXC];
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        const int c = part * 64 + lane + j * 64 * wpr;
        if (c < CPR)
          xs[j] = src == 0 ? resid_row8(a, l, m, 8 * c)
                           : ld16(a.xmid + (static_cast<int64_t>(l) * a.B + m) * a.H + 8 * c);
      }
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        const int c = part * 64 + lane + j * 64 * wpr;
        if (c < CPR) {
          const int k = 8 * c;
          if (src == 0 && blockIdx.x == 0) {
            uint32_t* dst = reinterpret_cast<uint32_t*>(a.xres + (static_cast<int64_t>(l) * a.B + m) * a.H + k);
            co_st32(dst, xs[j].x);
            co_st32(dst + 1, xs[j].y);
            co_st32(dst + 2, xs[j].z);
            co_st32(dst + 3, xs[j].w);
          }
          ss += sumsq8(xs[j]);
          *reinterpret_cast<uint4*>(row + k) = xs[j];
        }
      }
    }
    ss = wave_sum(ss);
    if (active && lane == 0) s_ss[m * MK_WAVES + part] = ss;
  }
  __syncthreads();
  for (int m0 = 0; m0 < a.B; m0 += rows_per_pass) {
    const int m = m0 + wave / wpr;
    if (m >= a.B || wave / wpr >= rows_per_pass) continue;
    float t = 0.f;
    for (int p = 0; p < wpr; ++p) t += s_ss[m * MK_WAVES + p];
    const float inv = 1.0f / sqrtf(t / static_cast<float>(K) + a.eps);
    uint16_t* row = s_x + m * ld_s;
    for (int c = part * 64 + lane; c < CPR; c += 64 * wpr)
      *reinterpret_cast<uint4*>(row + 8 * c) = norm8(lds16(row + 8 * c), lds16(s_w + 8 * c), inv);
  }
}

// Prologue of o_proj: the attention output of sequence m, features k .. k+7
// (head k / 128), merged from the split partials and rounded to bf16.
__device__ __forceinline__ uint4 attn_merge8(const MkArgs& a, int l, int nsplit, int m, int k) {
  const int h = k >> 7;
  const int d0 = k & 127;
  const int group = a.nh / a.nkv;
  const int g = h / group;
  const int r = h - g * group;
  const int64_t base = ((static_cast<int64_t>(l) * a.B + m) * a.nkv + g) * a.att_nsplit_max * 16 + r;
  // all loads of the split partials are independent: issue them together
  float2 ml[MK_ATT_SPLITS];
  float4 p0[MK_ATT_SPLITS], p1[MK_ATT_SPLITS];
#pragma unroll
  for (int sp = 0; sp < MK_ATT_SPLITS; ++sp) {
    if (sp < nsplit) {
      ml[sp] = ldg2f(a.att_ml + base + sp * 16);
      const float* po = a.att_o + (base + sp * 16) * D + d0;
      p0[sp] = ldg4f(po);
      p1[sp] = ldg4f(po + 4);
    }
  }
  float mx = NEG_INF;
#pragma unroll
  for (int sp = 0; sp < MK_ATT_SPLITS; ++sp)
    if (sp < nsplit) mx = fmaxf(mx, ml[sp].x);
  const float bse = mx == NEG_INF ? 0.f : mx;
  float lsum = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < MK_ATT_SPLITS; ++sp) {
    if (sp >= nsplit || ml[sp].x == NEG_INF) continue;
    const float f = __expf(ml[sp].x - bse);
    lsum += f * ml[sp].y;
    o[0] += f * p0[sp].x; o[1] += f * p0[sp].y; o[2] += f * p0[sp].z; o[3] += f * p0[sp].w;
    o[4] += f * p1[sp].x; o[5] += f * p1[sp].y; o[6] += f * p1[sp].z; o[7] += f * p1[sp].w;
  }
  const float inv = 1.f / lsum;
  uint4 r4;
  r4.x = pack_bf2(o[0] * inv, o[1] * inv);
  r4.y = pack_bf2(o[2] * inv, o[3] * inv);
  r4.z = pack_bf2(o[4] * inv, o[5] * inv);
  r4.w = pack_bf2(o[6] * inv, o[7] * inv);
  return r4;
}

// ------------------------------------------------------------------ attention stage
//
// One wave per item (sequence b, KV head g, key chunk).  The query rows of the
// KV head's group are the B operand (16 columns), K rows straight from memory
// the A operand of S^T = K Q^T; V goes transposed through the wave's own LDS
// rows for O^T = V^T P^T.  The unnormalised output, running max and sum of
// each query row are written as the chunk's partial.

__device__ __forceinline__ uint32_t elem16(const uint4& v, int i) {
  const uint32_t w = (&v.x)[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}

__device__ void attn_item(const MkArgs& a, int l, int S, int chunk, int nsplit, int item, uint16_t* vt, int lane) {
  const int split = item % nsplit;
  const int bg = item / nsplit;
  const int b = bg / a.nkv;
  const int g = bg - b * a.nkv;
  const int group = a.nh / a.nkv;
  const int col = lane & 15;
  const int G = lane >> 4;
  const int P = S - 1;
  const int j_begin = split * chunk;
  const int j_end = min(j_begin + chunk, S);
  const uint4 z4 = {0, 0, 0, 0};

  const bool rvalid = col < group;
  const int head = g * group + (rvalid ? col : 0);
  const uint16_t* qp = a.qbuf + (static_cast<int64_t>(l) * a.B + b) * (a.nh * D) + head * D;
  uint4 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = rvalid ? ld16(qp + 32 * kk + 8 * G) : z4;
  const MkLayer& L = a.layers[l];
  const uint16_t* kbase = L.kc + b * a.kv_bstride + g * a.kv_hstride;
  const uint16_t* vbase = L.vc + b * a.kv_bstride + g * a.kv_hstride;

  float m_run = NEG_INF, l_run = 0.f;
  floatx4_t oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  for (int j0 = j_begin; j0 < j_end; j0 += 16) {
    const int key = j0 + col;
    uint4 kf[4], vf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      kf[kk] = key < j_end ? ld16(kbase + static_cast<int64_t>(key) * D + 32 * kk + 8 * G) : z4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int vk = j0 + 4 * G + s;
      vf[s] = vk < j_end ? ld16(vbase + static_cast<int64_t>(vk) * D + 8 * col) : z4;
    }
    floatx4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[kk]), as_bf16x8(qf[kk]), sacc, 0, 0, 0);
    // V rows 4G + s, d chunk 8 col, transposed: row d gets the four keys at column 4G
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint2 w;
      w.x = elem16(vf[0], i) | (elem16(vf[1], i) << 16);
      w.y = elem16(vf[2], i) | (elem16(vf[3], i) << 16);
      *reinterpret_cast<uint2*>(vt + (8 * col + i) * VT + 4 * G) = w;
    }
    // online softmax of query column col over its four keys per lane group
    float s[4];
    float mt = NEG_INF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kj = j0 + 4 * G + i;
      s[i] = (kj < j_end && kj <= P) ? sacc[i] * a.scale : NEG_INF;
      mt = fmaxf(mt, s[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float bse = m_new == NEG_INF ? 0.f : m_new;
    const float alpha = m_run == NEG_INF ? 0.f : __expf(m_run - bse);
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = s[i] == NEG_INF ? 0.f : __expf(s[i] - bse);
      ps += s[i];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    uint2 pw;
    pw.x = pack_bf2(s[0], s[1]);
    pw.y = pack_bf2(s[2], s[3]);
    short4_t pf;
    __builtin_memcpy(&pf, &pw, 8);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's V^T writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      oacc[dt][0] *= alpha;
      oacc[dt][1] *= alpha;
      oacc[dt][2] *= alpha;
      oacc[dt][3] *= alpha;
      const uint2 vv = *reinterpret_cast<const uint2*>(vt + (16 * dt + col) * VT + 4 * G);
      short4_t va;
      __builtin_memcpy(&va, &vv, 8);
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pf, oacc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }
  // partial of query row col: o[d = 16 dt + 4 G + i], max, sum
  const int64_t slot = ((static_cast<int64_t>(l) * a.B + b) * a.nkv + g) * a.att_nsplit_max * 16 +
                       static_cast<int64_t>(split) * 16 + col;
  float* po = a.att_o + slot * D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) co_stf(po + 16 * dt + 4 * G + i, oacc[dt][i]);
  if (G == 0) {
    float* ml = reinterpret_cast<float*>(a.att_ml + slot);
    co_stf(ml, m_run);
    co_stf(ml + 1, l_run);
  }
}

// ------------------------------------------------------------------ epilogues
//
// Register epilogues of a wave tile: lane (m = lane % 16, g = lane / 16)
// holds features n = n0 + 4 g + {0, 1, 2, 3} of token m; pairs (n, n+1) and
// (n+2, n+3).  Rounding points are those of the unfused operator chain.

__device__ __forceinline__ void epi_qkv_pair(const MkArgs& a, int l, int pos, int m, int n, float v0, float v1) {
  const MkLayer& L = a.layers[l];
  const uint32_t bb = ldg(reinterpret_cast<const uint32_t*>(L.b_qkv + n));
  const float x0 = round_bf(v0 + bf_lo(bb));
  const float x1 = round_bf(v1 + bf_hi(bb));
  const int head = n >> 7;
  const int r = n & 127;
  if (head < a.nh + a.nkv) {
    const int p = r >> 1;
    const float2 cs = ldg2f(a.rope + static_cast<int64_t>(pos) * 64 + p);
    const float ra = x0 * cs.x - x1 * cs.y, rb = x1 * cs.x + x0 * cs.y;
    uint16_t* dst = head < a.nh ? a.qbuf + (static_cast<int64_t>(l) * a.B + m) * (a.nh * D) + head * D
                                : L.kc + m * a.kv_bstride + (head - a.nh) * a.kv_hstride + static_cast<int64_t>(pos) * D;
    co_st16(dst + p, ra);
    co_st16(dst + p + 64, rb);
  } else {
    uint16_t* dst =
        L.vc + m * a.kv_bstride + (head - a.nh - a.nkv) * a.kv_hstride + static_cast<int64_t>(pos) * D + r;
    co_st32(reinterpret_cast<uint32_t*>(dst), pack_bf2(x0, x1));
  }
}

__device__ __forceinline__ void epi_resid_pair(const MkArgs& a, int l, int m, int n, float v0, float v1) {
  const int64_t off = (static_cast<int64_t>(l) * a.B + m) * a.H + n;
  const uint32_t xin = ldg(reinterpret_cast<const uint32_t*>(a.xres + off));
  co_st32(reinterpret_cast<uint32_t*>(a.xmid + off),
          pack_bf2(bf_lo(xin) + round_bf(v0), bf_hi(xin) + round_bf(v1)));
}

__device__ __forceinline__ void epi_swiglu_pair(const MkArgs& a, int l, int m, int n, float v0, float v1) {
  co_st16(a.act + (static_cast<int64_t>(l) * a.B + m) * a.I + (n >> 1), silu_f(round_bf(v0)) * round_bf(v1));
}

// ------------------------------------------------------------------ the kernel
//
// The step is a sequence of 5 L + 1 stages (A..E per layer, then the LM head),
// each followed by a grid barrier, then the token pick.

enum Stage : int { ST_QKV = 0, ST_ATTN = 1, ST_O = 2, ST_GU = 3, ST_DOWN = 4, ST_HEAD = 5 };

struct Gemv {
  const uint16_t* W;
  int ldw, N, K, nkb, ntiles;
};

__device__ __forceinline__ Gemv stage_gemv(const MkArgs& a, int l, int st) {
  Gemv gv{};
  const int H = a.H, QD = a.nh * D, QKV = (a.nh + 2 * a.nkv) * D;
  const MkLayer* L = a.layers + (l < a.L ? l : 0);
  switch (st) {
    case ST_QKV: gv.W = L->w_qkv; gv.ldw = H; gv.N = QKV; gv.K = H; break;
    case ST_O: gv.W = L->w_o; gv.ldw = QD; gv.N = H; gv.K = QD; break;
    case ST_GU: gv.W = L->w_gu; gv.ldw = H; gv.N = 2 * a.I; gv.K = H; break;
    case ST_DOWN: gv.W = L->w_d; gv.ldw = a.I; gv.N = H; gv.K = a.I; break;
    default: gv.W = a.lm_head; gv.ldw = H; gv.N = a.V; gv.K = H; break;
  }
  gv.nkb = (gv.K + KB - 1) / KB;
  gv.ntiles = (gv.N + 15) / 16;
  return gv;
}

// Work split of a GEMV stage: QKV, o_proj and down give one 16-row tile (and
// K split, for down) to a workgroup whose waves share the K blocks (few
// tiles: every wave of the chip should still have loads in flight); gate/up
// and the LM head give whole tiles to single waves.
__device__ __forceinline__ bool wg_tiles(int st) { return st == ST_QKV || st == ST_O || st == ST_DOWN; }

__global__ __launch_bounds__(MK_THREADS) void decode_mk_kernel(MkArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int G = gridDim.x;
  const uint4 z4 = {0, 0, 0, 0};

  // LDS: staged X rows (or the attention V^T rows) | wave partial tiles | row sums
  uint16_t* s_x = reinterpret_cast<uint16_t*>(smem);
  floatx4_t* red = reinterpret_cast<floatx4_t*>(smem + a.lds_x_bytes);
  float* s_ss = reinterpret_cast<float*>(smem + a.lds_x_bytes + MK_WAVES * 64 * sizeof(floatx4_t) + 16 * 17 * 4);

  unsigned epoch = a.epoch0;
  bool dead = false;
  const int pos = *a.d_len;      // position of the new token
  const int S = pos + 1;         // keys it sees
  // key chunks per (sequence, KV head): at most MK_ATT_SPLITS, multiples of 16 keys
  const int chunk = 16 * max(1, (S + 16 * MK_ATT_SPLITS - 1) / (16 * MK_ATT_SPLITS));
  const int nsplit = (S + chunk - 1) / chunk;
  const int QD = a.nh * D;
  const bool xok = (lane & 15) < a.B;
  const int xrow = xok ? (lane & 15) : 0;
  const int wave_g = blockIdx.x + G * wave;  // this wave's first tile in a wave-tile stage

  uint4 r0[RB][4], r1[RB][4];
  Gemv gv{};
  int K = 0, nkb = 0, splits = 1, bps = 0;
  bool pre = false;

  // First load round of stage `st` of layer `l` for this wave: the weights do
  // not depend on the previous stage, so this is issued before its barrier.
#define MK_PREFETCH(L_, ST_)                                                                        \
  {                                                                                                 \
    gv = stage_gemv(a, (L_), (ST_));                                                                \
    K = gv.K;                                                                                       \
    nkb = gv.nkb;                                                                                   \
    splits = (ST_) == ST_DOWN ? a.down_splits : 1;                                                  \
    bps = (ST_) == ST_DOWN ? a.down_bps : gv.nkb;                                                   \
    pre = false;                                                                                    \
    if (wg_tiles(ST_)) {                                                                            \
      if (static_cast<int>(blockIdx.x) < gv.ntiles * splits) {                                      \
        const int t_ = blockIdx.x / splits, sp_ = blockIdx.x - t_ * splits;                         \
        const int kb0_ = sp_ * bps, kb1_ = min(nkb, kb0_ + bps);                                    \
        const int row_ = t_ * 16 + (lane & 15);                                                     \
        const bool wok_ = row_ < gv.N;                                                              \
        const uint16_t* wp_ = gv.W + static_cast<int64_t>(wok_ ? row_ : 0) * gv.ldw + 8 * g;        \
        _Pragma("unroll") for (int b_ = 0; b_ < RB; ++b_) {                                         \
          const int kk_ = kb0_ + wave + MK_WAVES * b_;                                              \
          if (kk_ < kb1_) {                                                                         \
            _Pragma("unroll") for (int u_ = 0; u_ < 4; ++u_) {                                      \
              const int k_ = kk_ * KB + 32 * u_ + 8 * g;                                            \
              r0[b_][u_] = ld16(wp_ + ((wok_ && k_ < K) ? static_cast<int64_t>(kk_) * KB + 32 * u_ : 0)); \
            }                                                                                       \
          }                                                                                         \
        }                                                                                           \
        pre = true;                                                                                 \
      }                                                                                             \
    } else if (wave_g < gv.ntiles) {                                                                \
      const int row_ = wave_g * 16 + (lane & 15);                                                   \
      const bool wok_ = row_ < gv.N;                                                                \
      const uint16_t* wp_ = gv.W + static_cast<int64_t>(wok_ ? row_ : 0) * gv.ldw + 8 * g;          \
      MK_LOAD(r0, wp_, wok_, 0)                                                                     \
      pre = true;                                                                                   \
    }                                                                                               \
  }

  MK_PREFETCH(0, ST_QKV)

  const int nstage = 5 * a.L + 1;
  for (int step = 0; step < nstage; ++step) {
    const int l = step / 5;
    const int st = step == nstage - 1 ? ST_HEAD : step - 5 * l;
    const MkLayer* L = a.layers + (l < a.L ? l : 0);

    if (st == ST_ATTN) {
      const int nitem = a.B * a.nkv * nsplit;
      uint16_t* vt = s_x + wave * (D * VT);
      for (int item = blockIdx.x + G * wave; item < nitem; item += G * MK_WAVES)
        attn_item(a, l, S, chunk, nsplit, item, vt, lane);
    } else {
      // prologue: X rows of this GEMV in LDS (down reads its X, the SwiGLU
      // output, from global memory)
      int ld_s = a.H + 8;
      if (st == ST_QKV || st == ST_HEAD) {
        stage_norm(a, l, 0, st == ST_QKV ? L->w_in : a.w_final, s_x, ld_s, s_ss, wave, lane);
      } else if (st == ST_GU) {
        stage_norm(a, l, 1, L->w_post, s_x, ld_s, s_ss, wave, lane);
      } else if (st == ST_O) {
        ld_s = QD + 8;
        for (int c = tid; c < a.B * (QD / 8); c += MK_THREADS) {
          const int m = c / (QD / 8), k = 8 * (c - m * (QD / 8));
          *reinterpret_cast<uint4*>(s_x + m * ld_s + k) = attn_merge8(a, l, nsplit, m, k);
        }
      }
      if (st != ST_DOWN) __syncthreads();
      MK_TRACE_SUB(step, 0);
      const uint16_t* xps = s_x + xrow * ld_s + 8 * g;
      const uint16_t* xpg = a.act + (static_cast<int64_t>(l) * a.B + xrow) * a.I + 8 * g;

      if (wg_tiles(st)) {
        // ---- workgroup tiles: round j of wave w covers K blocks
        // kb0 + w + 8 (RB j + b); two rounds of weights in flight
        const int items = gv.ntiles * splits;
        for (int i = blockIdx.x; i < items; i += G) {
          const int t = i / splits, sp = i - t * splits;
          const int kb0 = sp * bps, kb1 = min(nkb, kb0 + bps);
          const int row = t * 16 + (lane & 15);
          const bool wok = row < gv.N;
          const uint16_t* wp = gv.W + static_cast<int64_t>(wok ? row : 0) * gv.ldw + 8 * g;
          const int nround = (kb1 - kb0 - wave + RB * MK_WAVES - 1) / (RB * MK_WAVES);
#define MK_WG_LOAD(R_, J_)                                                                           \
  _Pragma("unroll") for (int b_ = 0; b_ < RB; ++b_) {                                               \
    const int kk_ = kb0 + wave + MK_WAVES * (RB * (J_) + b_);                                       \
    if (kk_ < kb1) {                                                                                \
      _Pragma("unroll") for (int u_ = 0; u_ < 4; ++u_) {                                            \
        const int k_ = kk_ * KB + 32 * u_ + 8 * g;                                                  \
        R_[b_][u_] = ld16(wp + ((wok && k_ < K) ? static_cast<int64_t>(kk_) * KB + 32 * u_ : 0));   \
      }                                                                                             \
    }                                                                                               \
  }
#define MK_WG_MMA(R_, J_, XP_, XOFF_)                                                                \
  _Pragma("unroll") for (int b_ = 0; b_ < RB; ++b_) {                                               \
    const int kk_ = kb0 + wave + MK_WAVES * (RB * (J_) + b_);                                       \
    if (kk_ < kb1) {                                                                                \
      _Pragma("unroll") for (int u_ = 0; u_ < 4; ++u_) {                                            \
        const int k_ = kk_ * KB + 32 * u_ + 8 * g;                                                  \
        const bool kin_ = k_ < K;                                                                   \
        uint4 xv_ = lds16((XP_) + ((xok && kin_) ? kk_ * KB + 32 * u_ - (XOFF_) : -8 * g));         \
        if (!(xok && kin_)) xv_ = z4;                                                               \
        const uint4 wv_ = (wok && kin_) ? R_[b_][u_] : z4;                                          \
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv_), as_bf16x8(xv_), acc, 0, 0, 0); \
      }                                                                                             \
    }                                                                                               \
  }
          if (!pre) MK_WG_LOAD(r0, 0)
          pre = false;
          if (nround > 1) MK_WG_LOAD(r1, 1)
          // down: this item's K range of the SwiGLU rows into LDS (when it fits)
          const uint16_t* xp = xps;
          int xoff = 0;
          bool xlds = st != ST_DOWN;
          if (st == ST_DOWN) {
            const int k_lo = kb0 * KB, k_hi = min(kb1 * KB, K);
            const int ldr = k_hi - k_lo + 8;
            xlds = static_cast<size_t>(a.B) * ldr * 2 <= static_cast<size_t>(a.lds_x_bytes);
            if (xlds) {
              const int cpr = (k_hi - k_lo) / 8;
              for (int c = tid; c < a.B * cpr; c += MK_THREADS) {
                const int m = c / cpr, k = k_lo + 8 * (c - m * cpr);
                *reinterpret_cast<uint4*>(s_x + m * ldr + (k - k_lo)) =
                    ld16(a.act + (static_cast<int64_t>(l) * a.B + m) * a.I + k);
              }
              __syncthreads();
              xp = s_x + xrow * ldr + 8 * g;
              xoff = k_lo;
            }
          }
          floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
          if (xlds) {
            for (int j = 0; j < nround; j += 2) {
              MK_WG_MMA(r0, j, xp, xoff)
              if (j + 1 >= nround) break;
              if (j + 2 < nround) MK_WG_LOAD(r0, j + 2)
              MK_WG_MMA(r1, j + 1, xp, xoff)
              if (j + 3 < nround) MK_WG_LOAD(r1, j + 3)
            }
          } else {
            // SwiGLU rows read straight from global memory (large batches)
            for (int j = 0; j < nround; ++j) {
              if (j > 0) MK_WG_LOAD(r0, j)
#pragma unroll
              for (int b_ = 0; b_ < RB; ++b_) {
                const int kk_ = kb0 + wave + MK_WAVES * (RB * j + b_);
                if (kk_ < kb1) {
#pragma unroll
                  for (int u_ = 0; u_ < 4; ++u_) {
                    const int k_ = kk_ * KB + 32 * u_ + 8 * g;
                    const bool kin_ = k_ < K;
                    uint4 xv_ = ld16(xpg + ((xok && kin_) ? static_cast<int64_t>(kk_) * KB + 32 * u_ : 0));
                    if (!(xok && kin_)) xv_ = z4;
                    const uint4 wv_ = (wok && kin_) ? r0[b_][u_] : z4;
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv_), as_bf16x8(xv_), acc, 0, 0, 0);
                  }
                }
              }
            }
          }
#undef MK_WG_LOAD
#undef MK_WG_MMA
          pre = false;
          MK_TRACE_SUB(step, 1);
          // fixed-order sum of the waves' partial tiles; wave 0 applies the epilogue
          red[wave * 64 + lane] = acc;
          __syncthreads();
          if (wave == 0) {
            floatx4_t sum = red[lane];
#pragma unroll
            for (int w = 1; w < MK_WAVES; ++w) {
              const floatx4_t o = red[w * 64 + lane];
              sum[0] += o[0];
              sum[1] += o[1];
              sum[2] += o[2];
              sum[3] += o[3];
            }
            const int m = lane & 15;
            const int n = t * 16 + 4 * g;
            if (m < a.B && n < gv.N) {
              if (st == ST_QKV) {
                epi_qkv_pair(a, l, pos, m, n, sum[0], sum[1]);
                epi_qkv_pair(a, l, pos, m, n + 2, sum[2], sum[3]);
              } else if (st == ST_O) {
                epi_resid_pair(a, l, m, n, sum[0], sum[1]);
                epi_resid_pair(a, l, m, n + 2, sum[2], sum[3]);
              } else {
                float* dst = a.down_part + ((static_cast<int64_t>(l) * splits + sp) * a.B + m) * a.H + n;
#pragma unroll
                for (int r = 0; r < 4; ++r) co_stf(dst + r, sum[r]);
              }
            }
          }
          __syncthreads();
        }
      } else {
        // ---- wave tiles (gate/up, LM head): one wave per 16-row tile, full K
        for (int t = wave_g; t < gv.ntiles; t += G * MK_WAVES) {
          const int n0 = t * 16;
          const int row = n0 + (lane & 15);
          const bool wok = row < gv.N;
          const uint16_t* wp = gv.W + static_cast<int64_t>(wok ? row : 0) * gv.ldw + 8 * g;
          if (!pre) MK_LOAD(r0, wp, wok, 0)
          pre = false;
          floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
          for (int kb = 0; kb < nkb; kb += 2 * RB) {
            if (kb + RB < nkb) MK_LOAD(r1, wp, wok, kb + RB)
            MK_MMA_LDS(r0, wok, kb)
            if (kb + RB >= nkb) break;
            if (kb + 2 * RB < nkb) MK_LOAD(r0, wp, wok, kb + 2 * RB)
            MK_MMA_LDS(r1, wok, kb + RB)
          }
          // next tile's first round in flight during the epilogue
          const int tn = t + G * MK_WAVES;
          if (tn < gv.ntiles) {
            const int rown = tn * 16 + (lane & 15);
            const bool wokn = rown < gv.N;
            const uint16_t* wpn = gv.W + static_cast<int64_t>(wokn ? rown : 0) * gv.ldw + 8 * g;
            MK_LOAD(r0, wpn, wokn, 0)
            pre = true;
          }
          const int m = lane & 15;
          const int n = n0 + 4 * g;
          if (st == ST_HEAD) {
            unsigned long long key = 0;
            if (m < a.B) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                if (n + r < a.V) {
                  if (a.logits) a.logits[static_cast<int64_t>(m) * a.V + n + r] = acc[r];
                  const unsigned long long k = argmax_key(acc[r], n + r);
                  key = k > key ? k : key;
                }
              }
            }
            unsigned long long o = __shfl_xor(key, 16, 64);
            key = o > key ? o : key;
            o = __shfl_xor(key, 32, 64);
            key = o > key ? o : key;
            if (g == 0 && m < a.B) atomicMax(a.keys + m * KEY_ROW + (t % KEY_SLOTS) * KEY_STRIDE, key);
          } else if (m < a.B && n < gv.N) {
            epi_swiglu_pair(a, l, m, n, acc[0], acc[1]);
            epi_swiglu_pair(a, l, m, n + 2, acc[2], acc[3]);
          }
        }
      }
    }
    MK_TRACE_POINT(2 * step);
    // arrive, issue the next stage's first weight loads, then wait
    grid_arrive(a, epoch);
    MK_TRACE_SUB(step, 2);
    pre = false;
    if (step + 1 < nstage) {
      const int l2 = (step + 1) / 5;
      const int st2 = step + 1 == nstage - 1 ? ST_HEAD : step + 1 - 5 * l2;
      if (st2 != ST_ATTN) MK_PREFETCH(l2, st2)
    }
    grid_wait(a, epoch, dead);
    MK_TRACE_POINT(2 * step + 1);
  }
#undef MK_PREFETCH

  // ---- next token of each sequence (one wave)
  if (blockIdx.x == 0 && wave == 0) {
    for (int b = 0; b < a.B; ++b) {
      unsigned long long best = 0;
      unsigned long long* slot = a.keys + b * KEY_ROW + lane * KEY_STRIDE;
      if (lane < KEY_SLOTS) {
        best = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long k = __shfl_xor(best, o, 64);
        best = k > best ? k : best;
      }
      if (lane == 0) {
        const int64_t id = static_cast<int64_t>(argmax_key_index(best));
        a.ids_buf[b] = id;
        a.hist[b * a.hist_ld + S] = id;
      }
    }
    if (lane == 0) *a.d_len = S;
  }
}

#undef MK_LOAD
#undef MK_MMA_LDS

}  // namespace

size_t mk_lds_x_bytes(int B, int H, int QD) {
  // B staged rows (+ the norm weights after them)
  const size_t x = (static_cast<size_t>(B) * (std::max(H, QD) + 8) + H + 8) * sizeof(uint16_t);
  const size_t att = static_cast<size_t>(MK_WAVES) * D * VT * sizeof(uint16_t);
  return (std::max(x, att) + 15) / 16 * 16;
}

size_t mk_lds_bytes(int B, int H, int QD) {
  return mk_lds_x_bytes(B, H, QD) + MK_WAVES * 64 * sizeof(floatx4_t) + 16 * 17 * sizeof(float) +
         16 * MK_WAVES * sizeof(float);
}

int mk_barriers(int L) { return 5 * L + 1; }

q2_status mk_launch(const MkArgs& a, int grid, hipStream_t s) {
  MkArgs args = a;
  void* params[] = {&args};
  const size_t lds = mk_lds_bytes(a.B, a.H, a.nh * D);
  hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<void*>(decode_mk_kernel), dim3(grid), dim3(MK_THREADS),
                                            params, static_cast<unsigned>(lds), s);
  if (e != hipSuccess) return fail(Q2_EHIP, "persistent decode launch failed: %s", hipGetErrorString(e));
  return Q2_OK;
}

q2_status mk_max_grid(int B, int H, int QD, int* grid) {
  int dev = 0;
  Q2_HIP(hipGetDevice(&dev));
  int cus = 0, coop = 0;
  Q2_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  Q2_HIP(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev));
  const size_t lds = mk_lds_bytes(B, H, QD);
  if (!coop) {
    *grid = 0;
    return Q2_OK;
  }
  if (lds > 64 * 1024) {
    Q2_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(decode_mk_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)));
  }
  int per_cu = 0;
  Q2_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(decode_mk_kernel),
                                                      MK_THREADS, lds));
  *grid = per_cu >= 1 ? cus : 0;
  return Q2_OK;
}

}  // namespace q2
