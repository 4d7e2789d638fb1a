// Linear layers: Y = X W^T with fused epilogues.
//
// Kernels sharing one epilogue interface (epilogue.hpp):
//  * gemm_dtl     bf16, 32x32x16 MFMA, operands loaded straight into a
//                 four-stage LDS ring, epilogue staged through LDS for
//                 row-contiguous stores (prefill; K % 128 == 0).
//  * gemm_big     bf16, 16x16x32 MFMA, register-staged double-buffered LDS
//                 (prefill shapes the first kernel does not take).
//  * gemm_f32     float32 FMA (the fp32 model), one output pair per thread.
// Up to 64 token rows go to the weight-streaming GEMV kernel (gemv.hip).
//
// MFMA orientation: weights are the A operand (rows = output features) and
// tokens the B operand, so a lane's accumulators hold runs of four
// consecutive features of one token -- the adjacent feature pairs the QKV
// (rotate-half) and SwiGLU epilogues need are in the same lane.
#include <algorithm>
#include <type_traits>

#include "epilogue.hpp"

namespace q2 {

namespace {

// ------------------------------------------------------------------ large-tile kernel
//
// BN features x BM tokens per workgroup, WN x WM waves, each wave a
// (BN/WN) x (BM/WM) block of 16x16 MFMA tiles.  K moves in 64-wide slices
// through two LDS stages: the next slice's global loads are issued before the
// current slice's MFMAs and written to LDS after them, one barrier per slice.
//
// LDS rows are 128 bytes (64 bf16) with the eight 16-byte chunks of row r
// stored at chunk c ^ ((r ^ (r >> 1)) & 7): the fragment reads (16 rows, one
// chunk column, per 16 lanes) and the slice writes (one row per 8 lanes)
// both touch distinct banks, for 32 or 64 four-byte banks.
//
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2); the tile order gives each XCD a contiguous band of tiles, token tiles
// fastest, so the workgroups resident on one XCD share their weight tiles.

__device__ __forceinline__ int lds_swz(int r, int c) { return c ^ ((r ^ (r >> 1)) & 7); }

template <int BN, int BM, int WN, int WM>
struct BigTile {
  static constexpr int NT = WN * WM * 64;
  static constexpr int TN = BN / WN, TM = BM / WM;
  static constexpr int FN = TN / 16, FM = TM / 16;
  static constexpr int BK = 64;
  static constexpr int A_LD = BN * 8 / NT;   // 16-byte weight chunks per thread per slice
  static constexpr int B_LD = BM * 8 / NT;   // 16-byte token chunks per thread per slice
  static constexpr int STAGE = (BN + BM) * 8;  // uint4 per LDS stage
  static constexpr size_t LDS_BYTES = size_t(2) * STAGE * 16;
  static_assert(A_LD * NT == BN * 8 && B_LD * NT == BM * 8, "tile does not split over the threads");
};

template <typename T, int EK, int BN, int BM, int WN, int WM, int PF>
__global__ __launch_bounds__(WN * WM * 64) void gemm_big_kernel(const uint16_t* __restrict__ W, int64_t ldw,
                                                               const uint16_t* __restrict__ X, int64_t ldx, int N,
                                                               int M, int K, int tiles_m, int tiles, int per_xcd,
                                                               Epi epi) {
  using C = BigTile<BN, BM, WN, WM>;
  extern __shared__ uint4 smem[];

  // XCD-aware tile order (per_xcd == 0: plain order)
  const int id = blockIdx.x;
  const int t = per_xcd ? (id & 7) * per_xcd + (id >> 3) : id;
  if (t >= tiles) return;
  const int tn = t / tiles_m;
  const int tm = t - tn * tiles_m;
  const int n0 = tn * BN;
  const int m0 = tm * BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave / WM;
  const int wm = wave - wn * WM;

  // Slice loads: chunk q = tid + NT * i covers row q / 8, 16-byte chunk q % 8.
  // Every load is issued (out-of-range rows and the K tail read a clamped
  // in-range address and are zeroed afterwards) so that the compiler keeps
  // the staging registers in VGPRs and leaves the loads in flight across the
  // MFMAs of the current slice.
  const uint16_t* __restrict__ pa[C::A_LD];
  const uint16_t* __restrict__ pb[C::B_LD];
  bool oka[C::A_LD], okb[C::B_LD];
  int sa_off[C::A_LD], sb_off[C::B_LD], kq[C::A_LD > C::B_LD ? C::A_LD : C::B_LD];
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    const int q = tid + C::NT * i;
    const int r = q >> 3;
    oka[i] = n0 + r < N;
    pa[i] = W + static_cast<int64_t>(oka[i] ? n0 + r : 0) * ldw + 8 * (q & 7);
    sa_off[i] = r * 8 + lds_swz(r, q & 7);
  }
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) {
    const int q = tid + C::NT * i;
    const int r = q >> 3;
    okb[i] = m0 + r < M;
    pb[i] = X + static_cast<int64_t>(okb[i] ? m0 + r : 0) * ldx + 8 * (q & 7);
    sb_off[i] = BN * 8 + r * 8 + lds_swz(r, q & 7);
  }
  (void)kq;
  const int kc = 8 * (tid & 7);  // k offset of this thread's chunk inside a slice (same for every i)
  // two register sets: slices kt+1 and kt+2 are in flight while slice kt is
  // multiplied out of LDS
  uint4 ra0[C::A_LD], rb0[C::B_LD];
  uint4 ra1[PF == 2 ? C::A_LD : 1], rb1[PF == 2 ? C::B_LD : 1];
  const uint4 z = {0, 0, 0, 0};
#define Q2_BIG_LOAD(RA_, RB_, K0_)                                                                \
  {                                                                                               \
    const int k0_ = (K0_);                                                                        \
    const bool kin_ = k0_ + kc < K;                                                               \
    const int64_t ko_ = kin_ ? k0_ : 0;                                                           \
    _Pragma("unroll") for (int i = 0; i < C::A_LD; ++i) RA_[i] = *reinterpret_cast<const uint4*>(pa[i] + ko_); \
    _Pragma("unroll") for (int i = 0; i < C::B_LD; ++i) RB_[i] = *reinterpret_cast<const uint4*>(pb[i] + ko_); \
    _Pragma("unroll") for (int i = 0; i < C::A_LD; ++i) if (!(kin_ && oka[i])) RA_[i] = z;             \
    _Pragma("unroll") for (int i = 0; i < C::B_LD; ++i) if (!(kin_ && okb[i])) RB_[i] = z;             \
  }
#define Q2_BIG_STORE(RA_, RB_, S_)                                                                \
  {                                                                                               \
    uint4* st_ = smem + (S_) * C::STAGE;                                                          \
    _Pragma("unroll") for (int i = 0; i < C::A_LD; ++i) st_[sa_off[i]] = RA_[i];                  \
    _Pragma("unroll") for (int i = 0; i < C::B_LD; ++i) st_[sb_off[i]] = RB_[i];                  \
  }

  floatx4_t acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fch = lane >> 4;
#define Q2_BIG_MMA(S_)                                                                            \
  {                                                                                               \
    const uint4* sa_ = smem + (S_) * C::STAGE;                                                    \
    const uint4* sb_ = sa_ + BN * 8;                                                              \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                                            \
      const int c = 4 * kk + fch;                                                                 \
      bf16x8_t a[C::FN], b[C::FM];                                                                \
      _Pragma("unroll") for (int i = 0; i < C::FN; ++i) {                                         \
        const int r = wn * C::TN + 16 * i + frow;                                                 \
        a[i] = as_bf16x8(sa_[r * 8 + lds_swz(r, c)]);                                             \
      }                                                                                           \
      _Pragma("unroll") for (int j = 0; j < C::FM; ++j) {                                         \
        const int r = wm * C::TM + 16 * j + frow;                                                 \
        b[j] = as_bf16x8(sb_[r * 8 + lds_swz(r, c)]);                                             \
      }                                                                                           \
      _Pragma("unroll") for (int i = 0; i < C::FN; ++i)                                           \
        _Pragma("unroll") for (int j = 0; j < C::FM; ++j)                                         \
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);    \
    }                                                                                             \
  }

  // Slices past the end load a zeroed dummy (keeps every load unconditional)
  // and are never stored or multiplied.
  const int nk = (K + C::BK - 1) / C::BK;
  Q2_BIG_LOAD(ra0, rb0, 0)
  Q2_BIG_STORE(ra0, rb0, 0)
  __syncthreads();
  if constexpr (PF == 1) {
    for (int kt = 0; kt < nk; ++kt) {
      const int s = kt & 1;
      Q2_BIG_LOAD(ra0, rb0, (kt + 1) * C::BK)
      Q2_BIG_MMA(s)
      if (kt + 1 < nk) Q2_BIG_STORE(ra0, rb0, s ^ 1)
      __syncthreads();
    }
  } else {
    Q2_BIG_LOAD(ra0, rb0, 1 * C::BK)
    Q2_BIG_LOAD(ra1, rb1, 2 * C::BK)
    for (int kt = 0; kt < nk; kt += 2) {
      // even slice kt: LDS stage 0; set 0 holds slice kt+1, set 1 slice kt+2
      Q2_BIG_MMA(0)
      if (kt + 1 >= nk) break;
      Q2_BIG_STORE(ra0, rb0, 1)
      __syncthreads();
      Q2_BIG_LOAD(ra0, rb0, (kt + 3) * C::BK)
      // odd slice kt+1: LDS stage 1; set 1 holds slice kt+2, set 0 slice kt+3
      Q2_BIG_MMA(1)
      if (kt + 2 >= nk) break;
      Q2_BIG_STORE(ra1, rb1, 0)
      __syncthreads();
      Q2_BIG_LOAD(ra1, rb1, (kt + 4) * C::BK)
    }
  }
#undef Q2_BIG_LOAD
#undef Q2_BIG_STORE
#undef Q2_BIG_MMA


  // epilogue: lane holds features 4*(lane/16)+r of token lane%16 in each 16x16 tile
#pragma unroll
  for (int i = 0; i < C::FN; ++i) {
    const int f = n0 + wn * C::TN + i * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const int m = m0 + wm * C::TM + j * 16 + (lane & 15);
      if (m >= M) continue;
      if (f < N) epi_pair<T, EK>(epi, m, f, acc[i][j][0], acc[i][j][1], f + 1 < N);
      if (f + 2 < N) epi_pair<T, EK>(epi, m, f + 2, acc[i][j][2], acc[i][j][3], f + 3 < N);
    }
  }
}

template <int EK, int BN, int BM, int WN, int WM, int PF = 1>
q2_status launch_big(const GemmArgs& a, hipStream_t s, bool xcd_order = true) {
  using C = BigTile<BN, BM, WN, WM>;
  const int tiles_m = cdiv(a.M, BM), tiles = tiles_m * cdiv(a.N, BN);
  const int per = xcd_order ? cdiv(tiles, 8) : 0;
  const int grid = xcd_order ? 8 * per : tiles;
  hipLaunchKernelGGL((gemm_big_kernel<uint16_t, EK, BN, BM, WN, WM, PF>), dim3(grid), dim3(C::NT), C::LDS_BYTES, s,
                     static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M,
                     a.K, tiles_m, tiles, per, a.epi);
  return check_launch("gemm_big");
}

// ------------------------------------------------------------------ direct-to-LDS kernel
//
// BN features x BM tokens per workgroup, WN x WM waves of (BN/WN) x (BM/WM),
// 32x32x16 bf16 MFMAs (on gfx950 twice the rate of 16x16x32).  K moves in
// 32-wide slices through a ring of four LDS stages that the global loads
// write directly (global_load_lds_dwordx4: no staging registers), so three
// slices are in flight while one is multiplied.  The wait for a stage is
// explicit: a wave waits until at most two stages of its own loads are
// outstanding (loads complete in issue order), then the workgroup barrier
// publishes every wave's part.  The two k16 steps of a slice are software-
// pipelined: the fragments of the next step are read while the MFMAs of the
// current one run.
//
// LDS rows are 64 bytes (32 bf16); chunk c of row r sits at c ^ (((r >> 1) ^
// (r >> 2)) & 3), which keeps the 32-lane fragment reads on distinct banks
// (for 32 or 64 banks).  A load instruction fills 64 consecutive 16-byte
// slots, so each lane fetches the global chunk that belongs in its slot.
// Requires K % 128 == 0 (whole trips of the four-stage ring) and 16-byte
// aligned rows; rows beyond M or N read a clamped valid row and their results
// are discarded.

__device__ __forceinline__ int dtl_swz(int r, int c) { return c ^ (((r >> 1) ^ (r >> 2)) & 3); }

// One global_load_lds_dwordx4: each lane's 16 bytes at g go to LDS at
// lds + 16 * lane (lds is the wave's base).  Written as asm so that the
// compiler does not track these LDS writes (it would otherwise wait for every
// load in flight before reading any stage); the kernel waits for them
// explicitly.  The instruction has no destination register; it reads its
// address operands when it issues.
__device__ __forceinline__ void dtl16(const void* g, const uint4* lds) {
  const uint32_t la =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint4*)lds));
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(la)) : "memory");
}

template <int BN, int BM, int WN, int WM>
struct Dtl {
  static constexpr int NT = WN * WM * 64;
  static constexpr int TN = BN / WN, TM = BM / WM;  // wave tile
  static constexpr int FN = TN / 32, FM = TM / 32;  // 32x32 MFMA tiles per wave
  static constexpr int BK = 32;
  static constexpr int SLOTS = (BN + BM) * 4;       // 16-byte slots per stage
  static constexpr int LD = SLOTS / NT;             // load instructions per wave per stage
  static constexpr size_t LDS_BYTES = size_t(4) * SLOTS * 16;
  // s_waitcnt vmcnt(2 * LD) expcnt(7) lgkmcnt(0) (gfx9 encoding)
  static constexpr int WAIT = ((2 * LD) & 15) | (((2 * LD) >> 4) << 14) | (7 << 4);
  static_assert(LD * NT == SLOTS, "stage does not split over the threads");
  static_assert(TN == 128, "the staged epilogue writes 128-feature rows");
};

// Staged epilogue (bf16): each wave applies the epilogue math to its
// 128-feature block in registers (where the feature pairs are), writes the
// results into LDS (16-byte chunk c of row r at c ^ (r & 15), 256 bytes per
// row) and then stores whole 16-byte chunks along output rows, so a store
// instruction covers four contiguous 256-byte row segments instead of 32
// scattered 8-byte pieces.
__device__ __forceinline__ int stg_idx(int r, int col) {
  return r * 128 + ((((col >> 3) ^ (r & 15)) << 3) | (col & 7));
}

// len0: position of token 0 of each sequence (QKV), read once per tile.
// The four features fb0 + nl .. + 3 (nl % 4 == 0) take their bias as one
// 8-byte load and the two RoPE (cos, sin) pairs as one 16-byte load.
template <int EK>
__device__ __forceinline__ void stg_put(uint16_t* sh, const Epi& e, int M, int fb0, int tb0, int r, int nl,
                                        int len0, float x0, float x1, float x2, float x3,
                                        const uint2* pre_bias = nullptr, const float4* pre_cs = nullptr) {
  const uint16_t* bias = static_cast<const uint16_t*>(e.bias);
  if constexpr (EK == EPI_STORE || EK == EPI_RESID) {
    if (EK == EPI_STORE && bias) {
      const uint2 bb = *reinterpret_cast<const uint2*>(bias + fb0 + nl);
      x0 += bf_lo(bb.x);
      x1 += bf_hi(bb.x);
      x2 += bf_lo(bb.y);
      x3 += bf_hi(bb.y);
    }
    const uint2 v = {pack_bf2(x0, x1), pack_bf2(x2, x3)};
    *reinterpret_cast<uint2*>(sh + stg_idx(r, nl)) = v;
  } else if constexpr (EK == EPI_SWIGLU) {
    const float y0 = silu_f(round_bf(x0)) * round_bf(x1);
    const float y1 = silu_f(round_bf(x2)) * round_bf(x3);
    *reinterpret_cast<uint32_t*>(sh + stg_idx(r, nl >> 1)) = pack_bf2(y0, y1);
  } else if constexpr (EK == EPI_QKV) {
    // the block is one head (d = 128); q and k heads hold rotate-half pairs
    // in adjacent rows (2p: original p, 2p+1: original p + 64)
    const uint2 bb = pre_bias ? *pre_bias : *reinterpret_cast<const uint2*>(bias + fb0 + nl);
    const float a0 = round_bf(x0 + bf_lo(bb.x)), a1 = round_bf(x1 + bf_hi(bb.x));
    const float a2 = round_bf(x2 + bf_lo(bb.y)), a3 = round_bf(x3 + bf_hi(bb.y));
    const int head = fb0 >> 7;
    if (head < e.nh + e.nkv) {
      const int m = tb0 + r;
      const int p = nl >> 1;
      float2 c0 = make_float2(1.f, 0.f), c1 = c0;
      if (pre_cs) {
        c0 = make_float2(pre_cs->x, pre_cs->y);
        c1 = make_float2(pre_cs->z, pre_cs->w);
      } else if (m < M) {
        const int64_t pos = (e.lens ? e.lens[m / e.T] : len0) + m % e.T;
        const float4 cs = *reinterpret_cast<const float4*>(e.rope + pos * 64 + p);
        c0 = make_float2(cs.x, cs.y);
        c1 = make_float2(cs.z, cs.w);
      }
      const float ra0 = a0 * c0.x - a1 * c0.y, rb0 = a1 * c0.x + a0 * c0.y;
      const float ra1 = a2 * c1.x - a3 * c1.y, rb1 = a3 * c1.x + a2 * c1.y;
      *reinterpret_cast<uint32_t*>(sh + stg_idx(r, p)) = pack_bf2(ra0, ra1);
      *reinterpret_cast<uint32_t*>(sh + stg_idx(r, p + 64)) = pack_bf2(rb0, rb1);
    } else {
      const uint2 v = {pack_bf2(a0, a1), pack_bf2(a2, a3)};
      *reinterpret_cast<uint2*>(sh + stg_idx(r, nl)) = v;
    }
  }
}

// Residual chunks a lane adds in stg_copy_out, loaded before the epilogue's
// LDS staging (up to RES_PRE per lane; iterations past them load their own).
constexpr int RES_PRE = 8;

template <int ROWS>
__device__ __forceinline__ void res_preload(const Epi& e, int M, int N, int fb0, int tb0, int lane,
                                            uint4 (&pre)[RES_PRE]) {
#pragma unroll
  for (int it = 0; it < RES_PRE && it < ROWS * 16 / 64; ++it) {
    // unconditional loads at a clamped in-range address (chunks outside the
    // product are never stored), so none of them waits for another
    const int q = it * 64 + lane;
    const int r = q / 16, c = q % 16;
    const int m = min(tb0 + r, M - 1);
    const int f = min(fb0 + c * 8, N - 8);
    pre[it] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(e.out) + static_cast<int64_t>(m) * e.ldo + f);
  }
}

template <int EK, int ROWS>
__device__ __forceinline__ void stg_copy_out(const uint16_t* sh, const Epi& e, int M, int N, int fb0, int tb0,
                                             int lane, int len0, const uint4 (&res)[RES_PRE]) {
  constexpr int CPR = EK == EPI_SWIGLU ? 8 : 16;  // 16-byte chunks per row of the block
  // fully unrolled, so that res[] stays in registers
#pragma unroll
  for (int it = 0; it < ROWS * CPR / 64; ++it) {
    const int q = it * 64 + lane;
    const int r = q / CPR, c = q % CPR;
    const int m = tb0 + r;
    if (m >= M) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(sh + stg_idx(r, c * 8));
    if constexpr (EK == EPI_STORE) {
      if (fb0 + c * 8 >= N) continue;
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(e.out) + static_cast<int64_t>(m) * e.ldo + fb0 + c * 8) = v;
    } else if constexpr (EK == EPI_RESID) {
      if (fb0 + c * 8 >= N) continue;
      uint4* dst =
          reinterpret_cast<uint4*>(static_cast<uint16_t*>(e.out) + static_cast<int64_t>(m) * e.ldo + fb0 + c * 8);
      const uint4 o = it < RES_PRE ? res[it] : *dst;
      const uint32_t* os = &o.x;
      const uint32_t* vs = &v.x;
      uint4 w;
      uint32_t* ws = &w.x;
#pragma unroll
      for (int k = 0; k < 4; ++k) ws[k] = pack_bf2(bf_lo(os[k]) + bf_lo(vs[k]), bf_hi(os[k]) + bf_hi(vs[k]));
      *dst = w;
    } else if constexpr (EK == EPI_SWIGLU) {
      if ((fb0 >> 1) + c * 8 >= (N >> 1)) continue;
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(e.out) + static_cast<int64_t>(m) * e.ldo + (fb0 >> 1) +
                                c * 8) = v;
    } else if constexpr (EK == EPI_QKV) {
      const int head = fb0 >> 7;
      uint16_t* dst;
      if (head < e.nh) {
        dst = static_cast<uint16_t*>(e.out) + static_cast<int64_t>(m) * e.ldo + head * 128;
      } else {
        const int bt = m / e.T;
        const int t = m - bt * e.T;
        const int64_t pos = e.kv_rel ? t : len0 + t;
        const bool isk = head < e.nh + e.nkv;
        uint16_t* base = static_cast<uint16_t*>(isk ? e.kc : e.vc);
        const int hh = isk ? head - e.nh : head - e.nh - e.nkv;
        dst = base + bt * e.kv_bstride + hh * e.kv_hstride + pos * 128;
      }
      *reinterpret_cast<uint4*>(dst + c * 8) = v;
    }
  }
}

// Tile order.  Workgroups are dealt to the 8 XCDs in turn, each with its own
// L2: logical tile L = (t % 8) * (T / 8) + t / 8 makes a run of consecutive
// tiles live on one XCD, and walking them in groups of 4 token tiles x all
// weight tiles keeps the ~32 tiles resident on an XCD within 4 token panels
// and 8 weight panels, which its L2 then serves.  t: this workgroup's index
// among the T tiles (tiles_m token tiles per weight panel).
__device__ __forceinline__ void xcd_tile(int t, int T, int tiles_m, int& tn, int& tm) {
  const int L = T % 8 == 0 ? (t % 8) * (T / 8) + t / 8 : t;
  const int tiles_n = T / tiles_m;
  constexpr int GM = 4;
  const int per_group = GM * tiles_n;
  const int fm = L / per_group * GM;
  const int gs = min(tiles_m - fm, GM);
  const int r = L - fm * tiles_n;
  tm = fm + r % gs;
  tn = r / gs;
}

// Stream-K hand-over between the two workgroups that share a tile: the
// partial tile and the flag are written and read at agent scope (the L2s of
// the XCDs are not coherent with each other), the flag only after every
// store of the partial has completed.
__device__ __forceinline__ void sk_st64(float* p, float x, float y) {
  const uint64_t v = static_cast<uint64_t>(__float_as_uint(x)) | (static_cast<uint64_t>(__float_as_uint(y)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 sk_ld64(const float* p) {
  const uint64_t v =
      __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}
__device__ __forceinline__ void sk_st32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned sk_ld32(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// polls of a stream-K flag before the finisher gives up and reports it
constexpr long SK_SPIN_MAX = 1L << 22;

// Stream-K roles of dtl_tile (template argument SK):
enum SkRole : int { SK_NONE = 0, SK_PRODUCE = 1, SK_FINISH = 2 };
struct SkPart {
  int kt0, nkt;       // K slices [kt0, kt0 + nkt) of the tile
  float* part;        // the tile's float32 hand-over buffer (NT x 64 floats, thread-major)
  unsigned* flag;     // 0: empty, 1: written; the finisher resets it
  unsigned* err;      // set when a finisher's wait times out
};

// One BN x BM output tile at features n0.., tokens m0...
// With SPLIT, blockIdx.y takes slices [y * kt_split, (y + 1) * kt_split) of
// K and the float32 tile goes to partial[y][m][n] (a second kernel sums the
// splits in order and applies the epilogue).
// With SK, the K slices are sk.kt0 .. + sk.nkt: SK_PRODUCE hands its float32
// tile over to the finisher and returns; SK_FINISH adds the hand-over
// (earlier slices first: p + acc) and applies the epilogue.
template <int EK, int BN, int BM, int WN, int WM, bool STAGED, bool SPLIT, int SK = SK_NONE>
__device__ __forceinline__ void dtl_tile(const uint16_t* __restrict__ W, int64_t ldw, const uint16_t* __restrict__ X,
                                         int64_t ldx, int N, int M, int K, int n0, int m0, int kt_split,
                                         float* __restrict__ partial, const Epi& epi, const SkPart& sk = SkPart{}) {
  using C = Dtl<BN, BM, WN, WM>;
  constexpr int FN = C::FN, FM = C::FM, TN = C::TN, TM = C::TM, NT = C::NT, LD = C::LD;
  extern __shared__ uint4 dsm[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave / WM;
  const int wm = wave - wn * WM;

  // the global chunk behind each of this lane's slots (slot = i * NT + tid;
  // slots [0, 4 BN) hold weight rows, the rest token rows)
  const uint16_t* src[LD];
#pragma unroll
  for (int i = 0; i < LD; ++i) {
    const int slot = i * NT + tid;
    const bool isw = slot < BN * 4;
    const int ls = isw ? slot : slot - BN * 4;
    const int r = ls >> 2;
    const int c = dtl_swz(r, ls & 3) +
                  (SPLIT ? blockIdx.y * kt_split * (C::BK / 8) : SK != SK_NONE ? sk.kt0 * (C::BK / 8) : 0);
    if (isw) {
      const int row = min(n0 + r, N - 1);
      src[i] = W + static_cast<int64_t>(row) * ldw + 8 * c;
    } else {
      const int row = min(m0 + r, M - 1);
      src[i] = X + static_cast<int64_t>(row) * ldx + 8 * c;
    }
  }
  const int nk = SPLIT ? min(kt_split, K / C::BK - static_cast<int>(blockIdx.y) * kt_split)
                 : SK != SK_NONE ? sk.nkt : K / C::BK;
#define Q2_DTL_ISSUE(S_, KT_)                                                                        \
  {                                                                                                  \
    const int kt_ = (KT_);                                                                           \
    const int64_t ko_ = kt_ < nk ? static_cast<int64_t>(kt_) * C::BK : 0; /* past the end: dummy */  \
    const uint4* st_ = dsm + (S_) * C::SLOTS;                                                        \
    _Pragma("unroll") for (int i = 0; i < LD; ++i) dtl16(src[i] + ko_, st_ + i * NT + wave * 64);    \
  }

  floatx16_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragment slots: row lane % 32, 8-element chunk 2 * kk + lane / 32
  const int frow = lane & 31;
  const int fch = lane >> 5;
  int a_off[2][FN], b_off[2][FM];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int r = wn * TN + 32 * i + frow;
      a_off[kk][i] = r * 4 + dtl_swz(r, 2 * kk + fch);
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int r = wm * TM + 32 * j + frow;
      b_off[kk][j] = BN * 4 + r * 4 + dtl_swz(r, 2 * kk + fch);
    }
  }

  // Slice kt lives in stage kt % 4.  The fragments of the next k16 step are
  // read while the MFMAs of the current one run; slice kt+1's barrier comes
  // before the second step of slice kt is multiplied, and by then every wave
  // has read all of slice kt, whose stage the loads issued after that barrier
  // (slice kt+4) overwrite.
  bf16x8_t fa[2][FN], fb[2][FM];
#define Q2_DTL_WAIT_BARRIER()                                                                        \
  __builtin_amdgcn_s_waitcnt(C::WAIT);                                                               \
  __builtin_amdgcn_s_barrier();                                                                      \
  asm volatile("" ::: "memory");
#define Q2_DTL_READ(SET_, S_, KK_)                                                                   \
  {                                                                                                  \
    const uint4* st_ = dsm + (S_) * C::SLOTS;                                                        \
    _Pragma("unroll") for (int i = 0; i < FN; ++i) fa[SET_][i] = as_bf16x8(st_[a_off[KK_][i]]);      \
    _Pragma("unroll") for (int j = 0; j < FM; ++j) fb[SET_][j] = as_bf16x8(st_[b_off[KK_][j]]);      \
  }
#define Q2_DTL_MMA(SET_)                                                                             \
  _Pragma("unroll") for (int i = 0; i < FN; ++i)                                                     \
    _Pragma("unroll") for (int j = 0; j < FM; ++j)                                                   \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SET_][i], fb[SET_][j], acc[i][j], 0, 0, 0);
#define Q2_DTL_SLICE(S_)                                                                             \
  {                                                                                                  \
    Q2_DTL_READ(1, S_, 1)                                                                            \
    Q2_DTL_MMA(0)                                                                                    \
    Q2_DTL_WAIT_BARRIER()                                                                            \
    Q2_DTL_ISSUE(S_, kt + S_ + 4)                                                                    \
    Q2_DTL_READ(0, (S_ + 1) & 3, 0)                                                                  \
    Q2_DTL_MMA(1)                                                                                    \
    __builtin_amdgcn_sched_barrier(0);                                                               \
  }
  Q2_DTL_ISSUE(0, 0)
  Q2_DTL_ISSUE(1, 1)
  Q2_DTL_ISSUE(2, 2)
  Q2_DTL_WAIT_BARRIER()
  Q2_DTL_ISSUE(3, 3)
  Q2_DTL_READ(0, 0, 0)
  for (int kt = 0; kt < nk; kt += 4) {
    Q2_DTL_SLICE(0)
    Q2_DTL_SLICE(1)
    Q2_DTL_SLICE(2)
    Q2_DTL_SLICE(3)
  }
  // no load into LDS may still be in flight when the stages are reused or
  // the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (SK == SK_PRODUCE) {
    // hand the float32 tile over (thread-major: a store instruction covers
    // 512 contiguous bytes per wave), then raise the flag once every
    // thread's stores have completed
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sk_st64(sk.part + 2 * (static_cast<int64_t>((i * FM + j) * 8 + e) * NT + tid), acc[i][j][2 * e],
                  acc[i][j][2 * e + 1]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) sk_st32(sk.flag, 1u);
    return;
  }
  if constexpr (SK == SK_FINISH) {
    if (tid == 0) {
      long spins = 0;
      while (sk_ld32(sk.flag) == 0u) {
        if (++spins > SK_SPIN_MAX) {
          sk_st32(sk.err, 1u);
          break;
        }
      }
      sk_st32(sk.flag, 0u);  // ready for the next launch
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 q = sk_ld64(sk.part + 2 * (static_cast<int64_t>((i * FM + j) * 8 + e) * NT + tid));
          acc[i][j][2 * e] = q.x + acc[i][j][2 * e];
          acc[i][j][2 * e + 1] = q.y + acc[i][j][2 * e + 1];
        }
  }
#undef Q2_DTL_ISSUE
#undef Q2_DTL_WAIT_BARRIER
#undef Q2_DTL_READ
#undef Q2_DTL_MMA
#undef Q2_DTL_SLICE

  // epilogue: element 4v+e of a 32x32 tile is feature 8v + 4*(lane/32) + e of
  // token lane%32
  const int fb0 = n0 + wn * TN;
  const int tb0 = m0 + wm * TM;
  if constexpr (SPLIT) {
    // N % 4 == 0: the four features of a lane's group are stored together
    float* pp = partial + static_cast<int64_t>(blockIdx.y) * M * N;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = tb0 + 32 * j + (lane & 31);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int f = fb0 + 32 * i + 8 * v + 4 * (lane >> 5);
          if (m < M && f < N)
            *reinterpret_cast<float4*>(pp + static_cast<int64_t>(m) * N + f) =
                make_float4(acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2], acc[i][j][4 * v + 3]);
        }
      }
  } else if constexpr (EK == EPI_ARGMAX) {
    // logits (optional) and the row's best (value, index) key over this
    // lane's 64 features; lanes l and l + 32 share a token row
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = tb0 + 32 * j + (lane & 31);
      unsigned long long key = 0;
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int f = fb0 + 32 * i + 8 * v + 4 * (lane >> 5) + e;
            if (m < M && f < N) {
              if (epi.out) static_cast<float*>(epi.out)[static_cast<int64_t>(m) * epi.ldo + f] = acc[i][j][4 * v + e];
              const unsigned long long k = argmax_key(acc[i][j][4 * v + e], f);
              key = k > key ? k : key;
            }
          }
      const unsigned long long k2 = __shfl_xor(key, 32, 64);
      key = k2 > key ? k2 : key;
      if (lane < 32 && m < M) atomicMax(epi.keys + m * KEY_ROW + (blockIdx.x % KEY_SLOTS) * KEY_STRIDE, key);
    }
  } else if constexpr (STAGED) {
    // the residual rows this lane adds are loaded before the staging, so
    // their latency overlaps it
    uint4 res[RES_PRE];
    if constexpr (EK == EPI_RESID) res_preload<TM>(epi, M, N, fb0, tb0, lane, res);
    // QKV (one token row per lane): every bias quad and RoPE (cos, sin) pair
    // pair of the lane's features, loaded together at clamped in-range
    // addresses (rows past M and value heads ignore theirs)
    constexpr bool QPRE = EK == EPI_QKV && FM == 1;
    uint2 qb[QPRE ? FN : 1][4];
    float4 qcs[QPRE ? FN : 1][4];
    if constexpr (QPRE) {
      // the position first (its load, if any, is then the only one waited
      // for), then all the loads that need it
      const int m = min(tb0 + (lane & 31), M - 1);
      const int len0q = epi.d_len ? *epi.d_len : epi.len0;
      const int64_t pos = (epi.lens ? epi.lens[m / epi.T] : len0q) + m % epi.T;
      const uint16_t* bias = static_cast<const uint16_t*>(epi.bias);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int nl = 32 * i + 8 * v + 4 * (lane >> 5);
          qcs[i][v] = *reinterpret_cast<const float4*>(epi.rope + pos * 64 + (nl >> 1));
          qb[i][v] = *reinterpret_cast<const uint2*>(bias + fb0 + nl);
        }
    }
    // every wave has finished reading the stages reused below (an LDS-only
    // barrier: the residual loads stay in flight across it)
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    uint16_t* sh = reinterpret_cast<uint16_t*>(dsm) + wave * (TM * 128);
    const int len0 = EK == EPI_QKV ? (epi.d_len ? *epi.d_len : epi.len0) : 0;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          stg_put<EK>(sh, epi, M, fb0, tb0, 32 * j + (lane & 31), 32 * i + 8 * v + 4 * (lane >> 5), len0,
                      acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2], acc[i][j][4 * v + 3],
                      QPRE ? &qb[QPRE ? i : 0][v] : nullptr, QPRE ? &qcs[QPRE ? i : 0][v] : nullptr);
    stg_copy_out<EK, TM>(sh, epi, M, N, fb0, tb0, lane, len0, res);
  } else {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = tb0 + 32 * j + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int f = fb0 + 32 * i + 8 * v + 4 * (lane >> 5);
          if (f < N) epi_pair<uint16_t, EK>(epi, m, f, acc[i][j][4 * v], acc[i][j][4 * v + 1], f + 1 < N);
          if (f + 2 < N)
            epi_pair<uint16_t, EK>(epi, m, f + 2, acc[i][j][4 * v + 2], acc[i][j][4 * v + 3], f + 3 < N);
        }
      }
    }
  }
}


template <int EK, int BN, int BM, int WN, int WM, bool STAGED, bool SPLIT>
__global__ __launch_bounds__(WN * WM * 64) void gemm_dtl_kernel(const uint16_t* __restrict__ W, int64_t ldw,
                                                                const uint16_t* __restrict__ X, int64_t ldx, int N,
                                                                int M, int K, int tiles_m, int kt_split,
                                                                float* __restrict__ partial, Epi epi) {
  int tn, tm;
  xcd_tile(blockIdx.x, gridDim.x, tiles_m, tn, tm);
  dtl_tile<EK, BN, BM, WN, WM, STAGED, SPLIT>(W, ldw, X, ldx, N, M, K, tn * BN, tm * BM, kt_split, partial, epi);
}

// Products whose 256 x 256 tiles leave the last round mostly idle: the
// first main_tiles workgroups take 256 x 256 tiles over features [0, n_main)
// (whole rounds of the chip), the rest 128-feature x 256-token tiles over the
// remaining features, which take a little over half the time of a square
// tile.  Both are 8-wave shapes; the launch gives the larger LDS ring.
template <int EK, bool STAGED>
__global__ __launch_bounds__(512) void gemm_dtl_mix_kernel(const uint16_t* __restrict__ W, int64_t ldw,
                                                           const uint16_t* __restrict__ X, int64_t ldx, int N, int M,
                                                           int K, int tiles_m, int main_tiles, Epi epi) {
  const int t = blockIdx.x;
  if (t < main_tiles) {
    int tn, tm;
    xcd_tile(t, main_tiles, tiles_m, tn, tm);
    dtl_tile<EK, 256, 256, 2, 4, STAGED, false>(W, ldw, X, ldx, N, M, K, tn * 256, tm * 256, 0, nullptr, epi);
  } else {
    const int n_main = main_tiles / tiles_m * 256;
    int tn, tm;
    xcd_tile(t - main_tiles, gridDim.x - main_tiles, tiles_m, tn, tm);
    dtl_tile<EK, 128, 256, 1, 8, STAGED, false>(W, ldw, X, ldx, N, M, K, n_main + tn * 128, tm * 256, 0, nullptr,
                                               epi);
  }
}

// Stream-K for long-K products with fewer 128-feature x 256-token tiles than
// CUs (down at hidden 1536 and 4096 tokens: 192 tiles, K = 8960): each
// tile's K is cut into four quarters (whole 128-wide groups) and every
// workgroup takes three consecutive quarters, so 4/3 as many workgroups as
// tiles (256 for 192) each do three quarters of a tile.  A tile is then shared by at most two workgroups: the
// one with its first quarters hands its float32 partial over (SK_PRODUCE),
// the one with its last quarters adds it and applies the epilogue
// (SK_FINISH).  Every workgroup produces before it finishes, so the hand-over
// it waits for was (nearly always) written long before.  All workgroups must
// be resident together (one per CU; the host launches this only when the
// grid fits the CUs); a wait that times out sets the error word instead of
// hanging.  Workgroups are numbered XCD-major, so that consecutive ones (which
// share tiles) sit on one XCD.
// sk: [flags: SK_MAX_TILES words][err word, padded to 1 KB][partials].
constexpr int SK_MAX_TILES = 256;
constexpr size_t SK_PART_OFF = SK_MAX_TILES * sizeof(unsigned) + 1024;
constexpr size_t SK_TILE_FLOATS = 128 * 256;

template <int EK, bool STAGED, int SK>
__device__ __forceinline__ void sk_segment(const uint16_t* __restrict__ W, int64_t ldw,
                                           const uint16_t* __restrict__ X, int64_t ldx, int N, int M, int K,
                                           int tiles_m, int tiles, int t, int q0, int q1, unsigned char* skw,
                                           const Epi& epi) {
  // tile t: groups of 4 token tiles x all weight tiles (as xcd_tile)
  const int tiles_n = tiles / tiles_m;
  const int fm = t / (4 * tiles_n) * 4;
  const int gs = min(tiles_m - fm, 4);
  const int r = t - fm * tiles_n;
  const int tm = fm + r % gs, tn = r / gs;
  // quarter q starts at K group round(q * G4 / 4) of G4 128-wide groups: the
  // main loop takes 32-wide slices four at a time, so a segment must be
  // whole groups (quarters of 280 slices: 72, 68, 72, 68)
  const int G4 = K / 128;
  const int g0 = (2 * q0 * G4 + 4) / 8, g1 = (2 * q1 * G4 + 4) / 8;
  unsigned* flags = reinterpret_cast<unsigned*>(skw);
  SkPart sk;
  sk.kt0 = 4 * g0;
  sk.nkt = 4 * (g1 - g0);
  sk.part = reinterpret_cast<float*>(skw + SK_PART_OFF) + static_cast<int64_t>(t) * SK_TILE_FLOATS;
  sk.flag = flags + t;
  sk.err = flags + SK_MAX_TILES;
  dtl_tile<EK, 128, 256, 1, 8, STAGED, false, SK>(W, ldw, X, ldx, N, M, K, tn * 128, tm * 256, 0, nullptr, epi, sk);
}

template <int EK, bool STAGED>
__global__ __launch_bounds__(512) void gemm_dtl_sk_kernel(const uint16_t* __restrict__ W, int64_t ldw,
                                                          const uint16_t* __restrict__ X, int64_t ldx, int N, int M,
                                                          int K, int tiles_m, int tiles, unsigned char* skw, Epi epi) {
  const int G = gridDim.x;
  const int L = G % 8 == 0 ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  const int s0 = 3 * L, s1 = s0 + 3;  // quarters [s0, s1) of the tile sequence
  const int t0 = s0 >> 2, t1 = (s1 - 1) >> 2;
  if (t1 > t0) {
    // the first quarters of tile t1, handed over
    sk_segment<EK, STAGED, SK_PRODUCE>(W, ldw, X, ldx, N, M, K, tiles_m, tiles, t1, 0, s1 - 4 * t1, skw, epi);
    __syncthreads();  // every wave is done with the LDS ring before it is refilled
  }
  const int a = s0 - 4 * t0, b = min(s1, 4 * t0 + 4) - 4 * t0;
  if (a == 0)
    sk_segment<EK, STAGED, SK_PRODUCE>(W, ldw, X, ldx, N, M, K, tiles_m, tiles, t0, 0, b, skw, epi);
  else
    sk_segment<EK, STAGED, SK_FINISH>(W, ldw, X, ldx, N, M, K, tiles_m, tiles, t0, a, 4, skw, epi);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The direct-to-LDS kernel's operand requirements.
bool dtl_ok(const GemmArgs& a) {
  return a.K % 128 == 0 && a.ldw % 8 == 0 && a.ldx % 8 == 0 && aligned16(a.W) && aligned16(a.X);
}

// The staged epilogue's output requirements (16-byte row chunks).
bool staged_ok(const GemmArgs& a) {
  const Epi& e = a.epi;
  if (a.N % 8 != 0 || e.ldo % 8 != 0 || !aligned16(e.out)) return false;
  if (e.bias && (reinterpret_cast<uintptr_t>(e.bias) & 7) != 0) return false;  // 8-byte bias loads
  switch (e.kind) {
    case EPI_STORE: return !e.out_f32;
    case EPI_RESID: return true;
    case EPI_SWIGLU: return (a.N / 2) % 8 == 0;
    case EPI_QKV:
      return e.dh == 128 && aligned16(e.kc) && aligned16(e.vc) && e.kv_bstride % 8 == 0 && e.kv_hstride % 8 == 0;
    default: return false;
  }
}

template <int EK, int BN, int BM, int WN, int WM>
q2_status launch_dtl_cfg(const GemmArgs& a, hipStream_t s) {
  using C = Dtl<BN, BM, WN, WM>;
  const int tiles_m = cdiv(a.M, BM), tiles = tiles_m * cdiv(a.N, BN);
  const bool staged = EK != EPI_ARGMAX && staged_ok(a);
  if (staged)
    hipLaunchKernelGGL((gemm_dtl_kernel<EK, BN, BM, WN, WM, true, false>), dim3(tiles), dim3(C::NT), C::LDS_BYTES, s,
                       static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M,
                       a.K, tiles_m, 0, nullptr, a.epi);
  else
    hipLaunchKernelGGL((gemm_dtl_kernel<EK, BN, BM, WN, WM, false, false>), dim3(tiles), dim3(C::NT), C::LDS_BYTES,
                       s, static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M,
                       a.K, tiles_m, 0, nullptr, a.epi);
  return check_launch("gemm_dtl");
}

// ------------------------------------------------------------------ skinny products (decode batches)
//
// 17..64 token rows: too many for the GEMV (whose workgroups own 16 weight
// rows each, so every workgroup would re-read all of X from L2) and too few
// for the big tiles.  The direct-to-LDS kernel with 256 weight rows (128 when
// that gives fewer than 32 tiles: twice the workgroups for the products with
// few output features, QKV, o_proj and down at hidden 1536) and all token
// rows (32 or 64) per tile streams W once; K is split over workgroups until
// the chip has work, as long as the float32 partials stay below a quarter of
// the weight bytes (or 8 MB, which the L2 and MALL absorb).  The LM head
// (argmax epilogue) needs no split.

struct SkinnyPlan {
  int bm, splits, kt_split;  // kt_split: 32-wide K slices per split (a multiple of 4)
  int bn = 256;               // weight rows per tile: 256 or 128
};

SkinnyPlan plan_skinny(int M, int N, int K) {
  SkinnyPlan p;
  p.bm = M <= 32 ? 32 : 64;
  p.bn = cdiv(N, 256) < 32 ? 128 : 256;
  const int tiles = cdiv(N, p.bn);
  const int nblk = K / 128;
  const double wbytes = 2.0 * N * K, per_split = 4.0 * M * N;
  const double cap = std::max(wbytes / 4, 8.0 * (1 << 20));
  int splits = 1;
  while (splits + 1 <= nblk && tiles * (splits + 1) <= 512 && per_split * (splits + 1) <= cap) ++splits;
  const int bps = cdiv(nblk, splits);
  p.splits = cdiv(nblk, bps);
  p.kt_split = 4 * bps;
  return p;
}

bool skinny_shape(int M, int N, int K) { return M > 16 && M <= 64 && K % 128 == 0 && N % 8 == 0; }

// 64-token tiles run 2 x 2 waves of 128 x 32 (256 weight rows; 1 x 2 for
// 128): about a quarter faster than 2 waves of 128 x 64 (more loads in
// flight per workgroup); 32-token tiles have one 32-row MFMA block per wave
// column.
template <int EK, int BM, int BN>
q2_status launch_skinny_cfg(const GemmArgs& a, const SkinnyPlan& p, hipStream_t s) {
  constexpr int WM = BM == 64 ? 2 : 1;
  constexpr int WN = BN / 128;
  using C = Dtl<BN, BM, WN, WM>;
  const int tiles = cdiv(a.N, BN);
  if constexpr (EK == EPI_ARGMAX) {
    hipLaunchKernelGGL((gemm_dtl_kernel<EK, BN, BM, WN, WM, false, false>), dim3(tiles), dim3(C::NT), C::LDS_BYTES, s,
                       static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M,
                       a.K, 1, 0, nullptr, a.epi);
    return check_launch("gemm_skinny");
  } else {
    if (p.splits == 1) {
      if (staged_ok(a))
        hipLaunchKernelGGL((gemm_dtl_kernel<EK, BN, BM, WN, WM, true, false>), dim3(tiles), dim3(C::NT), C::LDS_BYTES,
                           s, static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N,
                           a.M, a.K, 1, 0, nullptr, a.epi);
      else
        hipLaunchKernelGGL((gemm_dtl_kernel<EK, BN, BM, WN, WM, false, false>), dim3(tiles), dim3(C::NT),
                           C::LDS_BYTES, s, static_cast<const uint16_t*>(a.W), a.ldw,
                           static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M, a.K, 1, 0, nullptr, a.epi);
      return check_launch("gemm_skinny");
    }
    hipLaunchKernelGGL((gemm_dtl_kernel<EK, BN, BM, WN, WM, false, true>), dim3(tiles, p.splits), dim3(C::NT),
                       C::LDS_BYTES, s, static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.X),
                       a.ldx, a.N, a.M, a.K, 1, p.kt_split, static_cast<float*>(a.scratch), a.epi);
    Q2_TRY(check_launch("gemm_skinny"));
    return split_reduce(a, p.splits, s);
  }
}

template <int EK>
q2_status launch_skinny(const GemmArgs& a, hipStream_t s) {
  SkinnyPlan p = plan_skinny(a.M, a.N, a.K);
  if (EK == EPI_ARGMAX) p.splits = 1;
  if (p.splits > 1) {
    const size_t need = static_cast<size_t>(p.splits) * a.M * a.N * sizeof(float);
    if (a.unsplit_if_short && (!a.scratch || a.scratch_bytes < need)) p.splits = 1;
    Q2_CHECK(p.splits == 1 || (a.scratch && a.scratch_bytes >= need), Q2_EINVAL,
             "skinny linear: split-K scratch too small");
  }
  if (p.bn == 128) {
    if (p.bm == 32) return launch_skinny_cfg<EK, 32, 128>(a, p, s);
    return launch_skinny_cfg<EK, 64, 128>(a, p, s);
  }
  if (p.bm == 32) return launch_skinny_cfg<EK, 32, 256>(a, p, s);
  return launch_skinny_cfg<EK, 64, 256>(a, p, s);
}

// Tile shape by how many tiles the product has for 256 CUs:
//  * 256 x 256 (8 waves of 128 x 64, 128 KB LDS, one workgroup per CU) when
//    that gives at least ~1.5 rounds of work, with a 128 x 256 tail when the
//    last round would be mostly idle (gemm_dtl_mix_kernel);
//  * otherwise, with at least 512 token rows, 128 features x 256 tokens
//    (8 waves of 128 x 32, 96 KB): twice the tiles of the square shape, so
//    products with few output features (o_proj and down at hidden 1536: 96
//    square tiles) spread over most CUs instead of a third of them;
//  * otherwise 128 x 128 tiles (4 waves, 64 KB, two per CU).
// Main/tail split for gemm_dtl_mix_kernel: the number of 256 x 256 tiles,
// over leading weight panels and in whole rounds of 256 CUs, whose remainder
// as 128 x 256 tiles (about 0.6 of a square tile's time each) ends well
// before the plain grid's partly idle last round would.  0: no split.
int mix_main_tiles(int M, int N) {
  const int tiles_m = cdiv(M, 256), tiles_n = cdiv(N, 256);
  constexpr double kTail = 0.6;
  double best_cost = cdiv(tiles_m * tiles_n, 256);
  int best = 0;
  for (int tn = tiles_n - 1; tn >= 1; --tn) {
    const int main_tiles = tiles_m * tn;
    if (main_tiles % 256 != 0) continue;
    const int tail = tiles_m * cdiv(N - tn * 256, 128);
    const double cost = main_tiles / 256 + kTail * cdiv(tail, 256);
    if (cost < best_cost - 0.25) {
      best = main_tiles;
      best_cost = cost;
    }
  }
  return best;
}

template <int EK>
q2_status launch_dtl_mix(const GemmArgs& a, int main_tiles, hipStream_t s) {
  const int tiles_m = cdiv(a.M, 256);
  const int n_main = main_tiles / tiles_m * 256;
  const int tiles = main_tiles + tiles_m * cdiv(a.N - n_main, 128);
  const size_t lds = Dtl<256, 256, 2, 4>::LDS_BYTES;
  if (staged_ok(a))
    hipLaunchKernelGGL((gemm_dtl_mix_kernel<EK, true>), dim3(tiles), dim3(512), lds, s,
                       static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M,
                       a.K, tiles_m, main_tiles, a.epi);
  else
    hipLaunchKernelGGL((gemm_dtl_mix_kernel<EK, false>), dim3(tiles), dim3(512), lds, s,
                       static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M,
                       a.K, tiles_m, main_tiles, a.epi);
  return check_launch("gemm_dtl_mix");
}

// Stream-K applies to a 128 x 256 tiling of `tiles` tiles when its 4/3 as
// many workgroups fit the CUs at once (one each) and the workspace holds the
// hand-over tiles.
bool sk_fits(const GemmArgs& a, int tiles) {
  if (!a.sk_ws || a.epi.kind == EPI_ARGMAX || tiles % 3 != 0 || tiles > SK_MAX_TILES) return false;
  // long K only: the hand-over (a 128 KB partial tile written and read back)
  // costs a short product more than its idle CUs do (o_proj at K = 1536:
  // 30 -> 38 us); every quarter is at least one 128-wide group
  if (a.K % 128 != 0 || a.K < 4096) return false;
  const int grid = tiles / 3 * 4;
  if (grid > a.sk_cus) return false;
  return a.sk_ws_bytes >= SK_PART_OFF + static_cast<size_t>(tiles) * SK_TILE_FLOATS * sizeof(float);
}

template <int EK>
q2_status launch_dtl_sk(const GemmArgs& a, int tiles, hipStream_t s) {
  const int tiles_m = cdiv(a.M, 256);
  const size_t lds = Dtl<128, 256, 1, 8>::LDS_BYTES;
  unsigned char* skw = static_cast<unsigned char*>(a.sk_ws);
  const dim3 grid(tiles / 3 * 4);
  if (staged_ok(a))
    hipLaunchKernelGGL((gemm_dtl_sk_kernel<EK, true>), grid, dim3(512), lds, s, static_cast<const uint16_t*>(a.W),
                       a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M, a.K, tiles_m, tiles, skw, a.epi);
  else
    hipLaunchKernelGGL((gemm_dtl_sk_kernel<EK, false>), grid, dim3(512), lds, s, static_cast<const uint16_t*>(a.W),
                       a.ldw, static_cast<const uint16_t*>(a.X), a.ldx, a.N, a.M, a.K, tiles_m, tiles, skw, a.epi);
  return check_launch("gemm_dtl_sk");
}

template <int EK>
q2_status launch_dtl(const GemmArgs& a, hipStream_t s) {
  const int big_tiles = cdiv(a.M, 256) * cdiv(a.N, 256);
  if (big_tiles >= 384) {
    const int main_tiles = mix_main_tiles(a.M, a.N);
    if (main_tiles > 0) return launch_dtl_mix<EK>(a, main_tiles, s);
    return launch_dtl_cfg<EK, 256, 256, 2, 4>(a, s);
  }
  if (a.M >= 512) {
    if constexpr (EK != EPI_ARGMAX) {
      const int tiles = cdiv(a.M, 256) * cdiv(a.N, 128);
      if (sk_fits(a, tiles)) return launch_dtl_sk<EK>(a, tiles, s);
    }
    return launch_dtl_cfg<EK, 128, 256, 1, 8>(a, s);
  }
  return launch_dtl_cfg<EK, 128, 128, 1, 4>(a, s);
}

// ------------------------------------------------------------------ float32 kernel

template <int EK>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ W, int64_t ldw,
                                                       const float* __restrict__ X, int64_t ldx, int N, int M,
                                                       int K, Epi epi) {
  const int npairs = (N + 1) >> 1;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(npairs) * M) return;
  const int m = static_cast<int>(idx / npairs);
  const int n = static_cast<int>(idx - static_cast<int64_t>(m) * npairs) * 2;
  const bool has1 = n + 1 < N;
  const float* x = X + static_cast<int64_t>(m) * ldx;
  const float* w0 = W + static_cast<int64_t>(n) * ldw;
  const float* w1 = W + static_cast<int64_t>(has1 ? n + 1 : n) * ldw;
  float v0 = 0.f, v1 = 0.f;
  for (int k = 0; k < K; ++k) {
    const float xv = x[k];
    v0 = fmaf(xv, w0[k], v0);
    v1 = fmaf(xv, w1[k], v1);
  }
  if (EK == EPI_ARGMAX) {
    if (epi.out) {
      float* o = static_cast<float*>(epi.out) + static_cast<int64_t>(m) * epi.ldo + n;
      o[0] = v0;
      if (has1) o[1] = v1;
    }
    unsigned long long key = argmax_key(v0, n);
    if (has1) {
      unsigned long long k1 = argmax_key(v1, n + 1);
      key = k1 > key ? k1 : key;
    }
    atomicMax(epi.keys + m * KEY_ROW + ((n >> 1) % KEY_SLOTS) * KEY_STRIDE, key);
    return;
  }
  epi_pair<float, EK>(epi, m, n, v0, v1, has1);
}

template <int EK>
q2_status gemm_bf16_ek(const GemmArgs& a, hipStream_t s) {
  if constexpr (EK == EPI_ARGMAX) {
    return fail(Q2_ESHAPE, "argmax epilogue supports at most 64 rows");
  } else {
    if (dtl_ok(a)) return launch_dtl<EK>(a, s);
    return launch_big<EK, 128, 128, 2, 2>(a, s);
  }
}

template <int EK>
q2_status gemm_f32_ek(const GemmArgs& a, hipStream_t s) {
  const int64_t work = static_cast<int64_t>((a.N + 1) / 2) * a.M;
  hipLaunchKernelGGL(gemm_f32_kernel<EK>, dim3(cdiv(work, 256)), dim3(256), 0, s, static_cast<const float*>(a.W),
                     a.ldw, static_cast<const float*>(a.X), a.ldx, a.N, a.M, a.K, a.epi);
  return check_launch("gemm_f32");
}

}  // namespace

size_t gemm_scratch_bytes(int M, int N, int K) {
  size_t b = gemv_scratch_bytes(M, N, K);
  if (skinny_shape(M, N, K)) {
    const SkinnyPlan p = plan_skinny(M, N, K);
    if (p.splits > 1) b = std::max(b, static_cast<size_t>(p.splits) * M * N * sizeof(float));
  }
  return b;
}

int device_cus(int device) {
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
  return n;
}

size_t stream_k_bytes(int cus) {
  const int tiles = std::min(SK_MAX_TILES, cus / 4 * 3);
  return tiles > 0 ? SK_PART_OFF + static_cast<size_t>(tiles) * SK_TILE_FLOATS * sizeof(float) : 0;
}

size_t stream_k_err_offset() { return SK_MAX_TILES * sizeof(unsigned); }

bool gemm_post_norm(const GemmArgs& a) {
  // the skinny path's split-K reduction of a residual product (rows of 16-byte
  // chunks, row-contiguous output)
  return a.post_out && a.post_w && a.epi.kind == EPI_RESID && a.M > 0 && skinny_shape(a.M, a.N, a.K) &&
         dtl_ok(a) && !a.norm_w && !a.att_o && a.epi.ldo % 8 == 0 && aligned16(a.epi.out) &&
         aligned16(a.post_out) && aligned16(a.post_w) && plan_skinny(a.M, a.N, a.K).splits > 1;
}

q2_status gemm_bf16(const GemmArgs& a_in, hipStream_t s) {
  // the fused norm applies only where gemm_post_norm says so
  GemmArgs a = a_in;
  if (!gemm_post_norm(a)) a.post_out = nullptr;
  if (a.M == 0 || a.N == 0) return Q2_OK;
  Q2_CHECK(a.K % 8 == 0, Q2_ESHAPE, "bf16 linear: K=%d must be a multiple of 8", a.K);
  if (skinny_shape(a.M, a.N, a.K) && dtl_ok(a) && !a.norm_w && !a.att_o) {
    switch (a.epi.kind) {
      case EPI_STORE: return launch_skinny<EPI_STORE>(a, s);
      case EPI_RESID: return launch_skinny<EPI_RESID>(a, s);
      case EPI_SWIGLU: return launch_skinny<EPI_SWIGLU>(a, s);
      case EPI_QKV: return launch_skinny<EPI_QKV>(a, s);
      case EPI_ARGMAX: return launch_skinny<EPI_ARGMAX>(a, s);
    }
  }
  if (a.M <= GEMV_MAX_M) return gemv_bf16(a, s);
  Q2_CHECK(a.norm_w == nullptr, Q2_EINVAL, "fused RMSNorm needs M <= %d", GEMV_NORM_MAX_M);
  switch (a.epi.kind) {
    case EPI_STORE: return gemm_bf16_ek<EPI_STORE>(a, s);
    case EPI_RESID: return gemm_bf16_ek<EPI_RESID>(a, s);
    case EPI_SWIGLU: return gemm_bf16_ek<EPI_SWIGLU>(a, s);
    case EPI_QKV: return gemm_bf16_ek<EPI_QKV>(a, s);
    case EPI_ARGMAX: return gemm_bf16_ek<EPI_ARGMAX>(a, s);
  }
  return fail(Q2_EINVAL, "unknown epilogue %d", a.epi.kind);
}

q2_status gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return Q2_OK;
  switch (a.epi.kind) {
    case EPI_STORE: return gemm_f32_ek<EPI_STORE>(a, s);
    case EPI_RESID: return gemm_f32_ek<EPI_RESID>(a, s);
    case EPI_SWIGLU: return gemm_f32_ek<EPI_SWIGLU>(a, s);
    case EPI_QKV: return gemm_f32_ek<EPI_QKV>(a, s);
    case EPI_ARGMAX: return gemm_f32_ek<EPI_ARGMAX>(a, s);
  }
  return fail(Q2_EINVAL, "unknown epilogue %d", a.epi.kind);
}

}  // namespace q2
