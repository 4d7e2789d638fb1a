// Decode-path linear layers: Y[M, N] = X[M, K] W[N, K]^T for M <= 64 rows.
//
// Bound by reading W once from HBM.  A workgroup owns a tile of 16 weight
// rows; its waves (12 or 16) share that tile's K range, each taking 128-wide
// K blocks in turn.  A lane (row r = lane % 16, group g = lane / 16) loads four
// 16-byte pieces of row r per block (all issued before any math); load u of
// the four lane groups covers 64 contiguous bytes of each of the 16 rows.
// They feed four 16x16x32 bf16 MFMAs with the weight rows as the A operand;
// the token rows ride in the B operand (up to 16 per MFMA, 1-4 MFMA column
// tiles).  MFMA u of lane group g covers k = 32 u + 8 g .. + 7 on both
// operands.
//
// When the tiles alone would not give every CU work (one CU streams only
// about 20 GB/s), K is split over several workgroups that write float32
// partials; a small second kernel sums them in a fixed order and applies the
// epilogue, so results are deterministic.  (A last-arriving-workgroup
// reduction needs device-scope fences, which write back the L2 and cost far
// more than the extra launch on this chip.)
//
// Prologue: when it fits, the workgroup first stages the rows of X it needs
// (its K range) in LDS, built from one of three sources: the plain rows; the
// raw residual stream with RMSNorm applied (from per-16-feature sums of
// squares written by the producer of X, so no normalisation kernel runs); or
// the merge of split-KV attention partials (so no merge kernel runs).
#include <algorithm>

#include "epilogue.hpp"

namespace q2 {

namespace {

constexpr int KB = 128;  // K per block
constexpr int GEMV_WGS = 256;  // workgroups the tile loops aim at (one 12- or 16-wave workgroup per CU)

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// rnd(x * inv * w) for 8 bf16 lanes of a 16-byte vector.
__device__ __forceinline__ uint4 norm8(uint4 x, uint4 w, float inv) {
  uint4 r;
  const uint32_t* xs = &x.x;
  const uint32_t* ws = &w.x;
  uint32_t* rs = &r.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = (bf_lo(xs[i]) * inv) * bf_lo(ws[i]);
    const float b = (bf_hi(xs[i]) * inv) * bf_hi(ws[i]);
    rs[i] = pack_bf2(a, b);
  }
  return r;
}

enum XSrc : int { XSRC_RAW = 0, XSRC_NORM = 1, XSRC_ATTN = 2, XSRC_NORMR = 3 };

struct GemvSrc {
  const uint16_t* w;   // NORM
  const float* sq;
  int64_t sq_ld;
  float eps;
  const float* att_o;  // ATTN
  const float2* att_ml;
  int att_nsplit, att_group, att_nkv;
  const float* rp;     // NORMR: pending split-K partials [split][M][K]
  int rsplits;
  uint16_t* x_out;     // NORMR: the new residual rows (written by workgroup 0)
};

// 8 consecutive features (h * 128 + d0 .. + 7) of the merged attention output
// of sequence m, rounded to bf16.
__device__ __forceinline__ uint4 attn_merge8(const GemvSrc& src, int m, int k) {
  const int h = k >> 7;
  const int d0 = k & 127;
  const int g = h / src.att_group;
  const int r = h - g * src.att_group;
  const int64_t base = (static_cast<int64_t>(m) * src.att_nkv + g) * src.att_nsplit * 16 + r;
  // with up to 4 splits every load (max/sum and output of each split) is
  // issued before any is used: one memory round trip
  float mx = -__builtin_huge_valf();
  float l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (src.att_nsplit <= 4) {
    float2 ml[4];
    float4 pa[4], pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sp = min(i, src.att_nsplit - 1);
      ml[i] = src.att_ml[base + sp * 16];
      const float4* po = reinterpret_cast<const float4*>(src.att_o + (base + sp * 16) * 128 + d0);
      pa[i] = po[0];
      pb[i] = po[1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < src.att_nsplit) mx = fmaxf(mx, ml[i].x);
    const float bse = mx == -__builtin_huge_valf() ? 0.f : mx;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < src.att_nsplit && ml[i].x != -__builtin_huge_valf()) {
        const float f = __expf(ml[i].x - bse);
        l += f * ml[i].y;
        o[0] += f * pa[i].x; o[1] += f * pa[i].y; o[2] += f * pa[i].z; o[3] += f * pa[i].w;
        o[4] += f * pb[i].x; o[5] += f * pb[i].y; o[6] += f * pb[i].z; o[7] += f * pb[i].w;
      }
    }
  } else {
    for (int sp = 0; sp < src.att_nsplit; ++sp) mx = fmaxf(mx, src.att_ml[base + sp * 16].x);
    const float bse = mx == -__builtin_huge_valf() ? 0.f : mx;
    for (int sp = 0; sp < src.att_nsplit; ++sp) {
      const float2 ml = src.att_ml[base + sp * 16];
      if (ml.x == -__builtin_huge_valf()) continue;
      const float f = __expf(ml.x - bse);
      l += f * ml.y;
      const float4* po = reinterpret_cast<const float4*>(src.att_o + (base + sp * 16) * 128 + d0);
      const float4 a = po[0], b = po[1];
      o[0] += f * a.x; o[1] += f * a.y; o[2] += f * a.z; o[3] += f * a.w;
      o[4] += f * b.x; o[5] += f * b.y; o[6] += f * b.z; o[7] += f * b.w;
    }
  }
  const float inv = 1.f / l;
  uint4 r4;
  r4.x = pack_bf2(o[0] * inv, o[1] * inv);
  r4.y = pack_bf2(o[2] * inv, o[3] * inv);
  r4.z = pack_bf2(o[4] * inv, o[5] * inv);
  r4.w = pack_bf2(o[6] * inv, o[7] * inv);
  return r4;
}

// Operands an epilogue thread reads besides the product, loaded before the
// tile's weights arrive so that the epilogue issues no load of its own (a
// load there would also wait for the next tile's weights, issued earlier):
// the residual pair (RESID), the bias pair and RoPE cos/sin (QKV).
struct EpiPre {
  uint32_t x01;
  float b0, b1;
  float2 cs;
  int pos;
};

template <int EK>
__device__ __forceinline__ void epi_preload(const Epi& e, int M, int N, int n0, int m, int p, EpiPre& pre) {
  const int n = n0 + 2 * p;
  if (m >= M || n >= N) return;
  if constexpr (EK == EPI_RESID) {
    const uint16_t* o = static_cast<const uint16_t*>(e.out) + static_cast<int64_t>(m) * e.ldo + n;
    pre.x01 = static_cast<uint32_t>(o[0]) | (n + 1 < N ? static_cast<uint32_t>(o[1]) << 16 : 0u);
  } else if constexpr (EK == EPI_QKV) {
    const uint16_t* b = static_cast<const uint16_t*>(e.bias);
    pre.b0 = bf2f(b[n]);
    pre.b1 = bf2f(b[n + 1]);
    const int head = n / e.dh;
    const int t = m % e.T;
    pre.pos = (e.lens ? e.lens[m / e.T] : e.d_len ? *e.d_len : e.len0) + t;
    if (head < e.nh + e.nkv) pre.cs = e.rope[static_cast<int64_t>(pre.pos) * (e.dh >> 1) + ((n - head * e.dh) >> 1)];
  }
}

// Epilogue of a 16-feature tile for token row m: thread p (0..7 within an
// aligned group of 8 lanes) owns features n0 + 2p, n0 + 2p + 1.
template <int EK>
__device__ __forceinline__ void gemv_epilogue(const Epi& epi, int M, int N, int n0, int tile, int m, int p, float v0,
                                              float v1, const EpiPre* pre = nullptr) {
  const int n = n0 + 2 * p;
  const bool valid = m < M && n < N;
  const bool has1 = n + 1 < N;
  if constexpr (EK == EPI_ARGMAX) {
    unsigned long long key = 0;
    if (valid) {
      if (epi.out) {
        float* o = static_cast<float*>(epi.out) + static_cast<int64_t>(m) * epi.ldo + n;
        o[0] = v0;
        if (has1) o[1] = v1;
      }
      key = argmax_key(v0, n);
      if (has1) {
        const unsigned long long k1 = argmax_key(v1, n + 1);
        key = k1 > key ? k1 : key;
      }
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const unsigned long long k = __shfl_xor(key, o, 64);
      key = k > key ? k : key;
    }
    if (valid && p == 0) atomicMax(epi.keys + m * KEY_ROW + (tile % KEY_SLOTS) * KEY_STRIDE, key);
  } else if constexpr (EK == EPI_RESID) {
    float sq = 0.f;
    if (valid) {
      uint16_t* o = static_cast<uint16_t*>(epi.out) + static_cast<int64_t>(m) * epi.ldo + n;
      const float x0 = pre ? bf_lo(pre->x01) : bf2f(o[0]);
      const float a = round_bf(x0 + round_bf(v0));
      o[0] = f2bf(a);
      sq = a * a;
      if (has1) {
        const float x1 = pre ? bf_hi(pre->x01) : bf2f(o[1]);
        const float b = round_bf(x1 + round_bf(v1));
        o[1] = f2bf(b);
        sq += b * b;
      }
    }
    sq += __shfl_xor(sq, 1, 64);
    sq += __shfl_xor(sq, 2, 64);
    sq += __shfl_xor(sq, 4, 64);
    if (valid && p == 0 && epi.sq_out) epi.sq_out[m * epi.sq_ld + tile] = sq;
  } else if constexpr (EK == EPI_QKV) {
    if (!valid) return;
    if (!pre) {
      epi_pair<uint16_t, EK>(epi, m, n, v0, v1, has1);
      return;
    }
    // as epi_pair's QKV case, with the preloaded bias, position and cos/sin
    const float a = round_bf(v0 + pre->b0);
    const float c = round_bf(v1 + pre->b1);
    const int d = epi.dh;
    const int head = n / d;
    const int r = n - head * d;
    const int bt = m / epi.T;
    const int64_t row = epi.kv_rel ? m - bt * epi.T : pre->pos;
    if (head < epi.nh + epi.nkv) {
      const int q = r >> 1;
      const float ra = round_bf(a * pre->cs.x - c * pre->cs.y);
      const float rb = round_bf(c * pre->cs.x + a * pre->cs.y);
      uint16_t* dst;
      if (head < epi.nh)
        dst = static_cast<uint16_t*>(epi.out) + static_cast<int64_t>(m) * epi.ldo + head * d;
      else
        dst = static_cast<uint16_t*>(epi.kc) + bt * epi.kv_bstride + (head - epi.nh) * epi.kv_hstride + row * d;
      dst[q] = f2bf(ra);
      dst[q + (d >> 1)] = f2bf(rb);
    } else {
      uint16_t* dst = static_cast<uint16_t*>(epi.vc) + bt * epi.kv_bstride + (head - epi.nh - epi.nkv) * epi.kv_hstride +
                      row * d + r;
      dst[0] = f2bf(a);
      dst[1] = f2bf(c);
    }
  } else {
    if (valid) epi_pair<uint16_t, EK>(epi, m, n, v0, v1, has1);
  }
}

// gridDim.x = workgroups along N, gridDim.y = K splits.  With SPLIT the float32
// partial tile goes to partial[split][m][n] and gemv_reduce_kernel applies the
// epilogue; otherwise the epilogue runs here.
// With STAGE the X rows of this workgroup's K range are built in dynamic
// LDS first (required for the NORM and ATTN sources).  Every wave streams
// weights: handing the staging to a few dedicated waves lowers the loads in
// flight more than it saves.  The occupancy bound keeps two 12- or 16-wave
// workgroups resident per CU (at most 64 VGPRs): one more register halves the
// workgroups in flight and costs a third of the bandwidth on the long
// LM-head pass.
template <int MT, int NW, int EK, int SRC, bool STAGE, bool SPLIT>
__global__ __launch_bounds__(NW * 64, 1) void gemv_kernel(const uint16_t* __restrict__ W, int64_t ldw,
                                                       const uint16_t* __restrict__ X, int64_t ldx, int N, int M, int K,
                                                       int blocks_per_split, GemvSrc src, float* __restrict__ partial,
                                                       Epi epi) {
  constexpr int WW = NW;
  __shared__ float s_inv[16 * MT];
  __shared__ float s_ssw[NW];
  __shared__ floatx4_t red[NW][MT][64];
  __shared__ float tile[16 * MT][17];
  extern __shared__ __attribute__((aligned(16))) uint16_t s_x[];
  constexpr bool NORM = SRC == XSRC_NORM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane & 15;
  const int g = lane >> 4;
  // This workgroup's tiles: blockIdx.x, + gridDim.x, ... over the whole
  // rounds of the grid (adjacent workgroups stream adjacent tiles); the rows
  // left over after them, which would give a last round to only some
  // workgroups, are shared out evenly instead (an even number of rows each,
  // the rest of the tile masked: its clamped loads hit L2).  The residual
  // epilogue keeps whole tiles (it stores per-tile sums of squares).
  const int ntile = (N + 15) >> 4;
  const int G = gridDim.x;
  const int nround = EK == EPI_RESID ? (ntile - blockIdx.x + G - 1) / G : ntile / G;
  const int r_rest = nround * G * 16;  // first row of the shared-out rest (non-residual epilogues)
  const int rest = N - r_rest;
  const int rest_rows = EK == EPI_RESID || rest <= 0 ? 0 : ((rest + G - 1) / G + 1) & ~1;
  int k_tile = 0;  // index of the current tile among this workgroup's
  int n0 = blockIdx.x * 16;
  int nlim = N;    // rows of the current tile at or past nlim are not stored
  if (nround == 0) {
    n0 = r_rest + blockIdx.x * rest_rows;
    nlim = min(n0 + rest_rows, N);
  }
  const int nkb = (K + KB - 1) / KB;
  const int kb0 = blockIdx.y * blocks_per_split;
  const int kb1 = min(kb0 + blocks_per_split, nkb);
  const int k_lo = kb0 * KB;
  const int k_hi = min(kb1 * KB, K);
  const int ld_s = k_hi - k_lo + 8;  // LDS row stride of the staged X (+16 bytes of padding)

  // the weight loads do not depend on X: the first batch goes out before the
  // prologue so that its latency overlaps the staging of X.  Loads are
  // unconditional within the block range (out-of-range rows and the K tail
  // read a clamped in-range address of real weights) so the compiler issues
  // them back to back.  The X operand is zero past K, so a clamped weight
  // adds nothing; results of out-of-range rows are never stored.
  bool wrow_ok = n0 + row < nlim;
  const uint16_t* __restrict__ wp = W + static_cast<int64_t>(wrow_ok ? n0 + row : 0) * ldw + 8 * g;
  const uint4 z = {0, 0, 0, 0};
  constexpr int BATCH = 2;  // blocks whose weights are in flight at once per wave
  uint4 wv[BATCH][4];
#define Q2_GEMV_LOAD_BATCH(KB_)                                                              \
  _Pragma("unroll") for (int b = 0; b < BATCH; ++b) {                                       \
    const int kk = (KB_) + NW * b;                                                          \
    if (kk < kb1) { /* wave-uniform: no loads for blocks past the range */                  \
      _Pragma("unroll") for (int u = 0; u < 4; ++u) {                                       \
        const int k = kk * KB + 32 * u + 8 * g;                                             \
        wv[b][u] = ld16(wp + (k < K ? static_cast<int64_t>(kk) * KB + 32 * u : 0));          \
      }                                                                                     \
    }                                                                                       \
  }
  Q2_GEMV_LOAD_BATCH(kb0 + wave)
  // the epilogue thread of (row tid / 8, pair tid % 8) loads its operands now
  constexpr bool PRE = !SPLIT && (EK == EPI_RESID || EK == EPI_QKV);
  EpiPre pre{};
  if (PRE && tid < 16 * MT * 8) epi_preload<EK>(epi, M, nlim, n0, tid >> 3, tid & 7, pre);

  if constexpr (SRC == XSRC_NORMR) {
    // The pending residual add, then RMSNorm, row by row (one pass of the
    // threads covers a row: K / 8 <= 64 NW).  Rounding as the split
    // reduction's epilogue: rnd(x + rnd(sum of partials in split order)).
    const int chunks = K >> 3;
    const bool writer = blockIdx.x == 0 && blockIdx.y == 0;
    for (int m = 0; m < M; ++m) {
      const int k = 8 * tid;
      uint4 xn = {0, 0, 0, 0};
      float ss = 0.f;
      if (tid < chunks) {
        const uint4 xv = ld16(X + static_cast<int64_t>(m) * ldx + k);
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        // four splits' partials are loaded before any is summed (one memory
        // round trip per four splits); the sums still run in split order
        for (int s0 = 0; s0 < src.rsplits; s0 += 4) {
          float4 p0[4], p1[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int sp = min(s0 + i, src.rsplits - 1);
            const float4* q = reinterpret_cast<const float4*>(src.rp + (static_cast<int64_t>(sp) * M + m) * K + k);
            p0[i] = q[0];
            p1[i] = q[1];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (s0 + i < src.rsplits) {
              a[0] += p0[i].x; a[1] += p0[i].y; a[2] += p0[i].z; a[3] += p0[i].w;
              a[4] += p1[i].x; a[5] += p1[i].y; a[6] += p1[i].z; a[7] += p1[i].w;
            }
          }
        }
        const uint32_t* xs = &xv.x;
        uint32_t* ns = &xn.x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = round_bf(bf_lo(xs[i]) + round_bf(a[2 * i]));
          const float hi = round_bf(bf_hi(xs[i]) + round_bf(a[2 * i + 1]));
          ns[i] = pack_bf2(lo, hi);
          ss += lo * lo + hi * hi;
        }
        if (writer) *reinterpret_cast<uint4*>(src.x_out + static_cast<int64_t>(m) * ldx + k) = xn;
      }
      ss = wave_sum(ss);
      if (lane == 0) s_ssw[wave] = ss;
      __syncthreads();
      if (tid == 0) {
        float t = 0.f;
        for (int w = 0; w < NW; ++w) t += s_ssw[w];
        s_inv[m] = 1.0f / sqrtf(t / static_cast<float>(K) + src.eps);
      }
      __syncthreads();
      if (tid < chunks) *reinterpret_cast<uint4*>(s_x + m * ld_s + k) = norm8(xn, ld16(src.w + k), s_inv[m]);
    }
    __syncthreads();
  }
  if constexpr (NORM) {
    const int ntiles = K >> 4;
    for (int m = wave; m < M; m += NW) {
      float ss = 0.f;
      for (int t = lane; t < ntiles; t += 64) ss += src.sq[m * src.sq_ld + t];
      ss = wave_sum(ss);
      if (lane == 0) s_inv[m] = 1.0f / sqrtf(ss / static_cast<float>(K) + src.eps);
    }
    __syncthreads();
  }
  if constexpr (STAGE && SRC != XSRC_NORMR) {
    // X[:, k_lo .. k_hi) into LDS
    const int chunks = (k_hi - k_lo) >> 3;
    for (int idx = tid; idx < M * chunks; idx += NW * 64) {
      const int m = idx / chunks;
      const int k = k_lo + 8 * (idx - m * chunks);
      uint4 v;
      if constexpr (SRC == XSRC_ATTN) {
        v = attn_merge8(src, m, k);
      } else {
        v = ld16(X + static_cast<int64_t>(m) * ldx + k);
        if constexpr (NORM) v = norm8(v, ld16(src.w + k), s_inv[m]);
      }
      *reinterpret_cast<uint4*>(s_x + m * ld_s + (k - k_lo)) = v;
    }
    __syncthreads();
  }

  const uint16_t* xp[MT];
  bool xok[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int tok = 16 * j + row;
    xok[j] = tok < M;
    if constexpr (STAGE)
      xp[j] = s_x + (xok[j] ? tok : 0) * ld_s + 8 * g - k_lo;
    else
      xp[j] = X + static_cast<int64_t>(xok[j] ? tok : 0) * ldx + 8 * g;
  }

  for (;;) {
  floatx4_t acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) acc[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  for (int kb = kb0 + wave; kb < kb1; kb += NW * BATCH) {
    if (kb != kb0 + wave) Q2_GEMV_LOAD_BATCH(kb)
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int kk = kb + NW * b;
      if (kk >= kb1) break;
#pragma unroll
      for (int j = 0; j < MT; ++j) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = kk * KB + 32 * u + 8 * g;
          const bool ok = xok[j] && k < K;
          uint4 xv = ld16(xp[j] + (ok ? static_cast<int64_t>(kk) * KB + 32 * u : k_lo - 8 * g));
          if (!ok) xv = z;
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[b][u]), as_bf16x8(xv), acc[j], 0, 0, 0);
        }
      }
    }
  }

  // the next tile's first weight batch goes out before this tile's
  // reduction and epilogue (the X rows in LDS serve every tile)
  const int c0 = n0, cur = n0 >> 4, clim = nlim;
  const EpiPre pc = pre;
  ++k_tile;
  bool more;
  if (k_tile < nround) {
    n0 = (blockIdx.x + k_tile * G) * 16;
    nlim = N;
    more = true;
  } else {
    n0 = r_rest + blockIdx.x * rest_rows;
    nlim = min(n0 + rest_rows, N);
    more = k_tile == nround && n0 < nlim;
  }
  if (more) {
    wrow_ok = n0 + row < nlim;
    wp = W + static_cast<int64_t>(wrow_ok ? n0 + row : 0) * ldw + 8 * g;
    Q2_GEMV_LOAD_BATCH(kb0 + wave)
    if (PRE && tid < 16 * MT * 8) epi_preload<EK>(epi, M, nlim, n0, tid >> 3, tid & 7, pre);
  }

  // sum the weight waves' partial tiles (fixed order)
  if (wave < WW) {
#pragma unroll
    for (int j = 0; j < MT; ++j) red[wave][j][lane] = acc[j];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      floatx4_t s = red[0][j][lane];
#pragma unroll
      for (int w = 1; w < WW; ++w) {
        const floatx4_t t = red[w][j][lane];
        s[0] += t[0]; s[1] += t[1]; s[2] += t[2]; s[3] += t[3];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) tile[16 * j + row][4 * g + r] = s[r];
    }
  }
  __syncthreads();

  if constexpr (SPLIT) {
    for (int t = tid; t < M * 16; t += NW * 64) {
      const int m = t >> 4, f = t & 15;
      if (c0 + f < clim) partial[(static_cast<int64_t>(blockIdx.y) * M + m) * N + c0 + f] = tile[m][f];
    }
  } else {
    const int Mp = 16 * MT;
    for (int base = 0; base < Mp * 8; base += NW * 64) {
      const int t = base + tid;
      const int m = t >> 3;
      const int p = t & 7;
      const float v0 = m < Mp ? tile[m][2 * p] : 0.f;
      const float v1 = m < Mp ? tile[m][2 * p + 1] : 0.f;
      gemv_epilogue<EK>(epi, M, clim, c0, cur, m, p, v0, v1, PRE ? &pc : nullptr);
    }
  }
  // the next tile's reduction writes red only after every wave has passed
  // the barriers above, and tile only after the barrier that follows it
  if (!more) break;
  }
#undef Q2_GEMV_LOAD_BATCH
}

// Sums the split-K partials of 32 (row, tile) pairs per workgroup, in split
// order, and applies the epilogue.
template <int EK>
__global__ __launch_bounds__(256) void gemv_reduce_kernel(const float* __restrict__ partial, int splits, int M, int N,
                                                          Epi epi) {
  const int ntiles = (N + 15) >> 4;
  const int pair = blockIdx.x * 32 + (threadIdx.x >> 3);
  const int p = threadIdx.x & 7;
  const int m = pair / ntiles;
  const int tl = pair - m * ntiles;
  const int n = tl * 16 + 2 * p;
  float v0 = 0.f, v1 = 0.f;
  if (m < M && n < N) {
    const bool has1 = n + 1 < N;
    if (has1 && (N & 1) == 0) {
      // n is even: one 8-byte load per split, unrolled so that several
      // splits' loads are in flight together; sums in split order
#pragma unroll 8
      for (int sp = 0; sp < splits; ++sp) {
        const float2 q = *reinterpret_cast<const float2*>(partial + (static_cast<int64_t>(sp) * M + m) * N + n);
        v0 += q.x;
        v1 += q.y;
      }
    } else {
      for (int sp = 0; sp < splits; ++sp) {
        const float* q = partial + (static_cast<int64_t>(sp) * M + m) * N + n;
        v0 += q[0];
        if (has1) v1 += q[1];
      }
    }
  }
  gemv_epilogue<EK>(epi, M, N, tl * 16, tl, m < M ? m : M, p, v0, v1);
}

// Split-K reduction of a residual product fused with the RMSNorm of the new
// residual rows.  One workgroup per row m: each thread sums the partials of
// its 8-feature chunks in split order and forms x = rnd(x + rnd(sum)) (the
// residual epilogue's rounding), written back and kept in LDS; wave 0 then
// takes the sum of squares in rmsnorm_vec_kernel's order (lane l: chunks l,
// l + 64, ..., then the wave sum), and every thread writes
// rnd((x * inv) * w) for its chunks -- the RMSNorm operator's result, bit for
// bit.  N % 8 == 0.
__global__ __launch_bounds__(256) void reduce_resid_norm_kernel(const float* __restrict__ partial, int splits, int M,
                                                                int N, uint16_t* __restrict__ x, int64_t ldx,
                                                                uint16_t* __restrict__ out,
                                                                const uint16_t* __restrict__ w, float eps) {
  extern __shared__ uint4 s_row[];  // the new row, N / 8 chunks
  __shared__ float s_inv;
  const int m = blockIdx.x;
  const int nch = N >> 3;
  uint16_t* xr = x + static_cast<int64_t>(m) * ldx;
  for (int i = threadIdx.x; i < nch; i += 256) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint4 xv = *reinterpret_cast<const uint4*>(xr + 8 * i);  // with the first partials
    // sixteen splits' loads in flight at a time
    for (int s0 = 0; s0 < splits; s0 += 16) {
      float4 p0[16], p1[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int sp = min(s0 + j, splits - 1);
        const float4* q = reinterpret_cast<const float4*>(partial + (static_cast<int64_t>(sp) * M + m) * N + 8 * i);
        p0[j] = q[0];
        p1[j] = q[1];
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (s0 + j < splits) {
          a[0] += p0[j].x; a[1] += p0[j].y; a[2] += p0[j].z; a[3] += p0[j].w;
          a[4] += p1[j].x; a[5] += p1[j].y; a[6] += p1[j].z; a[7] += p1[j].w;
        }
      }
    }
    const uint32_t* xs = &xv.x;
    uint4 xn;
    uint32_t* ns = &xn.x;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      ns[k] = pack_bf2(round_bf(bf_lo(xs[k]) + round_bf(a[2 * k])), round_bf(bf_hi(xs[k]) + round_bf(a[2 * k + 1])));
    *reinterpret_cast<uint4*>(xr + 8 * i) = xn;
    s_row[i] = xn;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float ss = 0.f;
    for (int i = lane; i < nch; i += 64) {
      const uint32_t* e = &s_row[i].x;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = bf_lo(e[k]), hi = bf_hi(e[k]);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) s_inv = 1.0f / sqrtf(ss / static_cast<float>(N) + eps);
  }
  __syncthreads();
  const float inv = s_inv;
  uint16_t* y = out + static_cast<int64_t>(m) * N;
  for (int i = threadIdx.x; i < nch; i += 256) {
    const uint4 xv = s_row[i];
    const uint4 wv = *reinterpret_cast<const uint4*>(w + 8 * i);
    const uint32_t* e = &xv.x;
    const uint32_t* we = &wv.x;
    uint4 r;
    uint32_t* re = &r.x;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      re[k] = pack_bf2((bf_lo(e[k]) * inv) * bf_lo(we[k]), (bf_hi(e[k]) * inv) * bf_hi(we[k]));
    *reinterpret_cast<uint4*>(y + 8 * i) = r;
  }
}

struct GemvPlan {
  int mt, nw, splits, bps;
};

GemvPlan plan_gemv(int M, int N, int K) {
  GemvPlan p;
  p.mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  p.nw = p.mt == 4 ? 8 : 16;
  const int tiles = cdiv(N, 16);
  const int nkb = cdiv(K, KB);
  // every CU needs work (a CU alone streams only ~20 GB/s): split K until
  // there are about 512 workgroups while each keeps at least NW/2 K blocks;
  // with many token rows keep the partials well below the weight bytes
  const int cap = p.mt == 1 ? 64 : max(1, K / (8 * M));
  int splits = 1;
  while (tiles * splits < 512 && nkb / (splits + 1) >= p.nw / 2 && splits + 1 <= cap) ++splits;
  // the X rows of a split's K range must fit the LDS stage: reading them from
  // L2 inside the block loop puts a dependent load behind every weight batch
  const int bps_fit = std::max(1, static_cast<int>((GEMV_STAGE_BYTES / (2 * M) - 8) / KB));
  auto fit = [&](int sp, int* bps, int* spl) {
    *bps = std::min(cdiv(nkb, sp), bps_fit);
    *spl = cdiv(nkb, *bps);
  };
  fit(splits, &p.bps, &p.splits);
  if (p.splits > 1) {
    // Each workgroup loops over ceil(tiles / grid) tiles of bps blocks: among
    // up to twice as many splits, take the one whose busiest workgroup has
    // the fewest blocks (whole tile rounds per workgroup, no idle tail).
    auto work = [&](int spl, int bps) {
      const int grid = std::min(tiles, std::max(1, GEMV_WGS / spl));
      return static_cast<int64_t>(cdiv(tiles, grid)) * bps;
    };
    int64_t best = work(p.splits, p.bps);
    for (int sp = p.splits + 1; sp <= 2 * p.splits && sp <= cap && sp <= nkb; ++sp) {
      int b, spl;
      fit(sp, &b, &spl);
      const int64_t w = work(spl, b);
      if (w < best) {
        best = w;
        p.bps = b;
        p.splits = spl;
      }
    }
    // A split costs a reduction kernel, about as long as streaming 24 more
    // blocks per workgroup: keep one split when that is no slower (7B
    // products at batch 8: 224-288 tiles already occupy the chip).
    int b1, s1;
    fit(1, &b1, &s1);
    if (s1 == 1 && work(1, b1) <= best + 24) {
      p.bps = b1;
      p.splits = 1;
    }
  }
  return p;
}

size_t stage_bytes(int M, int bps, int K) {
  const int klen = std::min(bps * KB, K);
  return static_cast<size_t>(M) * (klen + 8) * sizeof(uint16_t);
}

template <int MT, int NW, int EK, int SRC, bool STAGE>
q2_status launch_gemv2(const GemmArgs& a, const GemvPlan& p, size_t lds, hipStream_t s) {
  const GemvSrc src{static_cast<const uint16_t*>(a.norm_w), a.norm_sq, a.norm_sq_ld, a.norm_eps, a.att_o, a.att_ml,
                    a.att_nsplit, a.att_group, a.att_nkv, a.resid_part, a.resid_splits,
                    static_cast<uint16_t*>(a.resid_out)};
  // at most two rounds of 12- or 16-wave workgroups on the chip; each loops over
  // its tiles with the next tile's weights in flight
  // (the residual epilogue needs whole 16-row tiles; the others may give a
  // workgroup fewer rows, down to 8, when there are fewer tiles than slots)
  const int wgs = std::max(1, GEMV_WGS / p.splits);
  const int gx = EK == EPI_RESID ? std::min(cdiv(a.N, 16), wgs) : std::max(std::min(cdiv(a.N, 16), wgs), std::min(wgs, a.N / 8));
  const dim3 grid(gx, p.splits);
  if (p.splits == 1) {
    hipLaunchKernelGGL((gemv_kernel<MT, NW, EK, SRC, STAGE, false>), grid, dim3(NW * 64), lds, s,
                       static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M,
                       a.K, p.bps, src, nullptr, a.epi);
    return check_launch("gemv");
  }
  hipLaunchKernelGGL((gemv_kernel<MT, NW, EK, SRC, STAGE, true>), grid, dim3(NW * 64), lds, s,
                     static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M, a.K,
                     p.bps, src, static_cast<float*>(a.scratch), a.epi);
  return check_launch("gemv");
}

template <int MT, int NW, int EK, int SRC>
q2_status launch_gemv(const GemmArgs& a, const GemvPlan& p, hipStream_t s) {
  const size_t sb = stage_bytes(a.M, p.bps, a.K);
  if constexpr (SRC != XSRC_RAW) {
    Q2_CHECK(sb <= GEMV_STAGE_BYTES, Q2_ESHAPE, "gemv: fused source does not fit in LDS");
    Q2_TRY((launch_gemv2<MT, NW, EK, SRC, true>(a, p, sb, s)));
  } else {
    if (sb <= GEMV_STAGE_BYTES)
      Q2_TRY((launch_gemv2<MT, NW, EK, SRC, true>(a, p, sb, s)));
    else
      Q2_TRY((launch_gemv2<MT, NW, EK, SRC, false>(a, p, 0, s)));
  }
  if (p.splits == 1 || a.defer_reduce) return Q2_OK;
  if (EK == EPI_QKV && a.qkv_cache) return split_reduce(a, p.splits, s);
  const int pairs = a.M * cdiv(a.N, 16);
  hipLaunchKernelGGL((gemv_reduce_kernel<EK>), dim3(cdiv(pairs, 32)), dim3(256), 0, s,
                     static_cast<const float*>(a.scratch), p.splits, a.M, a.N, a.epi);
  return check_launch("gemv_reduce");
}

// Waves per workgroup for up to 16 token rows: 12 when a split's K range is
// at most 12 blocks (hidden 1536: every wave streams one block of each tile
// and none waits idle at the cross-wave reduction; batch-1 decode +1 %), 16
// otherwise (the 7B products' 28 blocks: 12 waves would leave a third of
// them with a second round of loads).  The pending-residual prologue covers
// a row with one pass of the threads, so there 12 waves also need
// K <= 8 x 768.  The LM head (argmax epilogue, 37 rounds of tiles at
// batch 1) keeps 16 waves: about 2 us per token faster there.
constexpr int GEMV_NW_SHORT = 12;

template <int EK, int SRC>
q2_status gemv_mt1(const GemmArgs& a, const GemvPlan& p, hipStream_t s) {
  if (EK != EPI_ARGMAX && p.bps <= GEMV_NW_SHORT && (SRC != XSRC_NORMR || a.K <= 8 * 64 * GEMV_NW_SHORT))
    return launch_gemv<1, GEMV_NW_SHORT, EK, SRC>(a, p, s);
  return launch_gemv<1, 16, EK, SRC>(a, p, s);
}

template <int EK>
q2_status gemv_ek(const GemmArgs& a, const GemvPlan& p, hipStream_t s) {
  if (a.norm_w && a.resid_part) return gemv_mt1<EK, XSRC_NORMR>(a, p, s);
  if (a.norm_w) return gemv_mt1<EK, XSRC_NORM>(a, p, s);
  if (a.att_o) return gemv_mt1<EK, XSRC_ATTN>(a, p, s);
  if (p.mt == 1) return gemv_mt1<EK, XSRC_RAW>(a, p, s);
  if (p.mt == 2) return launch_gemv<2, 16, EK, XSRC_RAW>(a, p, s);
  return launch_gemv<4, 8, EK, XSRC_RAW>(a, p, s);
}

}  // namespace

bool gemv_can_fuse(int M, int K) {
  // The fused prologues rebuild X once per workgroup (each loops over its
  // tiles), so they pay while X fits the LDS stage.  (The staged K range is
  // largest without splits.)
  return M <= GEMV_NORM_MAX_M && stage_bytes(M, cdiv(K, KB), K) <= GEMV_STAGE_BYTES;
}

bool gemv_can_defer(int M, int K) {
  // the deferred residual add normalises row by row, one pass of the
  // workgroup's threads per row: only for a few short rows
  return gemv_can_fuse(M, K) && M <= 2 && K / 8 <= 16 * 64;
}

namespace {

// Split-K reduction of the QKV product straight into a staged-layout cache
// (paged and/or FP8): one wave per (token row m, head).  Lane l owns features
// 2l, 2l + 1 of the head -- for q and k heads the rotate-half pair (l, l + 64),
// as the packed weight rows put them -- and sums their partials in split order
// (as gemv_reduce_kernel), then applies the QKV epilogue (bias, RoPE,
// rounding).  q rows go to e.out; k and v rows go to the cache rows of their
// positions: bf16 values, or FP8 codes quantised as whole 128-element blocks
// (kv_store_kernel's quantisation, so the same codes and scales).
template <bool FP8>
__global__ __launch_bounds__(256) void qkv_reduce_cache_kernel(const float* __restrict__ partial, int splits, int M,
                                                               int N, Epi e, KvLayout c) {
  const int nht = e.nh + 2 * e.nkv;
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= M * nht) return;  // whole waves leave together
  const int lane = threadIdx.x & 63;
  const int m = idx / nht;
  const int head = idx - m * nht;
  const int n = head * 128 + 2 * lane;
  float v0 = 0.f, v1 = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < splits; ++sp) {
    const float2 q = *reinterpret_cast<const float2*>(partial + (static_cast<int64_t>(sp) * M + m) * N + n);
    v0 += q.x;
    v1 += q.y;
  }
  const uint16_t* bias = static_cast<const uint16_t*>(e.bias);
  const float a = round_bf(v0 + bf2f(bias[n]));
  const float b = round_bf(v1 + bf2f(bias[n + 1]));
  const int bt = m / e.T;
  const int t = m - bt * e.T;
  const int pos = (e.lens ? e.lens[bt] : e.d_len ? *e.d_len : e.len0) + t;
  float x0 = a, x1 = b;  // the block elements this lane holds
  if (head < e.nh + e.nkv) {
    const float2 cs = e.rope[static_cast<int64_t>(pos) * 64 + lane];
    x0 = round_bf(a * cs.x - b * cs.y);  // element lane
    x1 = round_bf(b * cs.x + a * cs.y);  // element lane + 64
    if (head < e.nh) {
      uint16_t* dst = static_cast<uint16_t*>(e.out) + static_cast<int64_t>(m) * e.ldo + head * 128;
      dst[lane] = f2bf(x0);
      dst[lane + 64] = f2bf(x1);
      return;
    }
  }
  if (!kv_mapped(c, bt, pos)) return;  // whole waves leave together
  const bool isv = head >= e.nh + e.nkv;
  const bool rot = !isv;  // k: elements lane, lane + 64; v: 2 lane, 2 lane + 1
  const int hh = isv ? head - e.nh - e.nkv : head - e.nh;
  const int64_t row = kv_row(c, bt, hh, pos);
  if constexpr (FP8) {
    const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    const float scale = amax / 448.0f;
    const uint32_t c0 = e4m3_encode(amax == 0.f ? x0 : x0 / scale);
    const uint32_t c1 = e4m3_encode(amax == 0.f ? x1 : x1 / scale);
    uint8_t* dst = static_cast<uint8_t*>(isv ? c.vc : c.kc) + row * KV_BLOCK;
    if (rot) {
      dst[lane] = static_cast<uint8_t>(c0);
      dst[lane + 64] = static_cast<uint8_t>(c1);
    } else {
      *reinterpret_cast<uint16_t*>(dst + 2 * lane) = static_cast<uint16_t>(c0 | (c1 << 8));
    }
    if (lane == 0) (isv ? c.vs : c.ks)[row] = amax == 0.f ? 0.f : scale;
  } else {
    uint16_t* dst = static_cast<uint16_t*>(isv ? c.vc : c.kc) + row * KV_BLOCK;
    if (rot) {
      dst[lane] = f2bf(x0);
      dst[lane + 64] = f2bf(x1);
    } else {
      *reinterpret_cast<uint32_t*>(dst + 2 * lane) = pack_bf2(x0, x1);
    }
  }
}

}  // namespace

q2_status split_reduce(const GemmArgs& a, int splits, hipStream_t s) {
  if (a.epi.kind == EPI_QKV && a.qkv_cache) {
    Q2_CHECK(a.epi.dh == 128 && a.N == (a.epi.nh + 2 * a.epi.nkv) * 128 && a.epi.bias, Q2_EINVAL,
             "split reduce: the fused cache store needs head_dim 128 and a bias");
    const int waves = a.M * (a.epi.nh + 2 * a.epi.nkv);
    if (a.qkv_cache->fp8)
      hipLaunchKernelGGL(qkv_reduce_cache_kernel<true>, dim3(cdiv(waves, 4)), dim3(256), 0, s,
                         static_cast<const float*>(a.scratch), splits, a.M, a.N, a.epi, *a.qkv_cache);
    else
      hipLaunchKernelGGL(qkv_reduce_cache_kernel<false>, dim3(cdiv(waves, 4)), dim3(256), 0, s,
                         static_cast<const float*>(a.scratch), splits, a.M, a.N, a.epi, *a.qkv_cache);
    Q2_TRY(check_launch("split_reduce_qkv_cache"));
    if (a.qkv_cache_done) *a.qkv_cache_done = true;
    return Q2_OK;
  }
  if (a.epi.kind == EPI_RESID && a.post_out) {
    Q2_CHECK(a.N % 8 == 0 && a.epi.ldo % 8 == 0, Q2_EINVAL, "split reduce: fused norm needs N %% 8 == 0");
    hipLaunchKernelGGL(reduce_resid_norm_kernel, dim3(a.M), dim3(256), static_cast<size_t>(a.N) * 2, s,
                       static_cast<const float*>(a.scratch), splits, a.M, a.N, static_cast<uint16_t*>(a.epi.out),
                       a.epi.ldo, static_cast<uint16_t*>(a.post_out), static_cast<const uint16_t*>(a.post_w),
                       a.post_eps);
    return check_launch("split_reduce_norm");
  }
  const int pairs = a.M * cdiv(a.N, 16);
  switch (a.epi.kind) {
#define Q2_REDUCE_CASE(EK_)                                                                                     \
  case EK_:                                                                                                     \
    hipLaunchKernelGGL((gemv_reduce_kernel<EK_>), dim3(cdiv(pairs, 32)), dim3(256), 0, s,                        \
                       static_cast<const float*>(a.scratch), splits, a.M, a.N, a.epi);                          \
    return check_launch("split_reduce");
    Q2_REDUCE_CASE(EPI_STORE)
    Q2_REDUCE_CASE(EPI_RESID)
    Q2_REDUCE_CASE(EPI_SWIGLU)
    Q2_REDUCE_CASE(EPI_QKV)
#undef Q2_REDUCE_CASE
  }
  return fail(Q2_EINVAL, "split reduce: unsupported epilogue %d", a.epi.kind);
}

int gemv_splits(int M, int N, int K) { return plan_gemv(M, N, K).splits; }

size_t gemv_scratch_bytes(int M, int N, int K) {
  if (M > GEMV_MAX_M) return 0;
  GemvPlan p = plan_gemv(M, N, K);
  return p.splits > 1 ? static_cast<size_t>(p.splits) * M * N * sizeof(float) : 0;
}

q2_status gemv_bf16(const GemmArgs& a, hipStream_t s) {
  Q2_CHECK(a.M >= 1 && a.M <= GEMV_MAX_M, Q2_ESHAPE, "gemv: M=%d not in [1, %d]", a.M, GEMV_MAX_M);
  Q2_CHECK(a.K % 8 == 0, Q2_ESHAPE, "gemv: K must be a multiple of 8");
  GemvPlan p = plan_gemv(a.M, a.N, a.K);
  if (a.norm_w) {
    Q2_CHECK(a.M <= GEMV_NORM_MAX_M && a.norm_sq && a.K % 16 == 0, Q2_EINVAL, "gemv: bad fused-norm arguments");
  }
  if (a.att_o) {
    Q2_CHECK(!a.norm_w && a.M <= GEMV_NORM_MAX_M && a.att_ml && a.att_nsplit >= 1 && a.K % 128 == 0, Q2_EINVAL,
             "gemv: bad fused attention-merge arguments");
  }
  if (a.resid_part) {
    Q2_CHECK(a.norm_w && a.resid_out && a.resid_out != a.X && a.resid_splits >= 1 && a.K % 8 == 0 &&
                 a.K / 8 <= 16 * 64 && !a.defer_reduce,
             Q2_EINVAL, "gemv: bad deferred-residual arguments");
  }
  if (a.epi.kind == EPI_ARGMAX || a.resid_part) {
    // the argmax needs whole sums; the deferred residual add needs whole rows
    p.splits = 1;
    p.bps = cdiv(a.K, KB);
  }
  Q2_CHECK(!a.defer_reduce || a.epi.kind != EPI_ARGMAX, Q2_EINVAL, "gemv: argmax cannot defer its reduction");
  if (p.splits > 1) {
    const size_t need = static_cast<size_t>(p.splits) * a.M * a.N * sizeof(float);
    if (a.unsplit_if_short && (!a.scratch || a.scratch_bytes < need)) {
      p.splits = 1;
      p.bps = cdiv(a.K, KB);
    }
    Q2_CHECK(p.splits == 1 || (a.scratch && a.scratch_bytes >= need), Q2_EINVAL, "gemv: split-K scratch too small");
  }
  switch (a.epi.kind) {
    case EPI_STORE: return gemv_ek<EPI_STORE>(a, p, s);
    case EPI_RESID: return gemv_ek<EPI_RESID>(a, p, s);
    case EPI_SWIGLU: return gemv_ek<EPI_SWIGLU>(a, p, s);
    case EPI_QKV: return gemv_ek<EPI_QKV>(a, p, s);
    case EPI_ARGMAX: return gemv_ek<EPI_ARGMAX>(a, p, s);
  }
  return fail(Q2_EINVAL, "unknown epilogue %d", a.epi.kind);
}

}  // namespace q2
