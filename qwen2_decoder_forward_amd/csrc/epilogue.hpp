// Fused GEMM epilogues.  Every GEMM kernel of the library hands its float32
// accumulators to one of these, two adjacent output features at a time.
//
// Rounding points follow the operator sequence they replace, so that a fused
// kernel stores exactly what the unfused chain of operators would store:
//   STORE   out = rnd(acc + bias)                          (linear)
//   RESID   x   = rnd(x + rnd(acc))                        (linear, then add)
//   SWIGLU  a   = rnd(silu(rnd(g)) * rnd(u))               (two linears, then swiglu)
//   QKV     q/k = rnd(rope(rnd(acc + bias))), v = rnd(acc + bias), with k and
//           v written straight into the KV cache           (linear, rope, rearrange)
//   ARGMAX  logits (float32, optional) and a per-row packed (value, index) key
//           combined with atomicMax                        (linear, argmax)
//
// Packed weight layouts the epilogues rely on (built by the model loader):
//   QKV rows: q heads, then k heads, then v heads, d rows each.  Inside a q
//   or k head, row 2p holds original row p and row 2p+1 original row p + d/2,
//   so the two halves of a rotate-half pair are adjacent.  v heads keep the
//   original order.
//   gate/up rows: row 2f is gate row f, row 2f+1 is up row f.
#pragma once

#include "common.hpp"
#include "kvcache.hpp"

namespace q2 {

enum EpiKind : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_QKV = 3, EPI_ARGMAX = 4 };

struct Epi {
  int kind;
  int out_f32;            // STORE: output is float32 instead of the storage type
  void* out;              // STORE / RESID / SWIGLU / QKV(q) / ARGMAX(logits, may be null)
  int64_t ldo;            // row stride of out, elements
  const void* bias;       // STORE / QKV: [N] storage type, or null
  // QKV
  void* kc;               // K cache of this layer, [B][nkv][S_max][d]
  void* vc;               // V cache of this layer, same layout
  int64_t kv_bstride;     // elements between batches
  int64_t kv_hstride;     // elements between kv heads (= S_max * d)
  int nh, nkv, dh;
  int T;                  // tokens per sequence in this call (row m = b * T + t)
  const int* d_len;       // device cached length (position of t = 0) or null
  int len0;               // host cached length, used when d_len is null
  // k / v rows go to row t (this call's token index) of kc / vc instead of
  // row len + t: a staging buffer [B][nkv][T][d] that a separate kernel
  // stores into the cache (quantised caches); RoPE still uses len + t
  int kv_rel;
  // per-sequence cached lengths (sequence b's token t sits at lens[b] + t),
  // overriding d_len / len0 when set
  const int* lens;
  const float2* rope;     // [S_max][d/2] (cos, sin)
  // ARGMAX: packed (value, index) keys, KEY_SLOTS per row each on its own
  // 128-byte line (stride KEY_STRIDE), combined with atomicMax: spreading a
  // row's maxima over many lines keeps thousands of workgroups from queueing
  // on one atomic unit.  Zero before the GEMM (the finalize kernel that reads
  // them resets them).
  unsigned long long* keys;
  // RESID, decode path: per-row sums of squares of the new residual stream,
  // one float per 16-feature tile (the next GEMV's fused RMSNorm reads them)
  float* sq_out;
  int64_t sq_ld;
};

constexpr int KEY_SLOTS = 64;
constexpr int KEY_STRIDE = 16;  // 16 x 8 bytes = one 128-byte line per slot
constexpr int KEY_ROW = KEY_SLOTS * KEY_STRIDE;

template <typename T, int EK>
__device__ __forceinline__ void epi_pair(const Epi& e, int m, int n, float v0, float v1, bool has1) {
  using S = St<T>;
  switch (EK) {
    case EPI_STORE: {
      if (e.bias) {
        v0 += S::ld(static_cast<const T*>(e.bias) + n);
        if (has1) v1 += S::ld(static_cast<const T*>(e.bias) + n + 1);
      }
      if (e.out_f32) {
        float* o = static_cast<float*>(e.out) + static_cast<int64_t>(m) * e.ldo + n;
        o[0] = v0;
        if (has1) o[1] = v1;
      } else {
        T* o = static_cast<T*>(e.out) + static_cast<int64_t>(m) * e.ldo + n;
        S::st(o, v0);
        if (has1) S::st(o + 1, v1);
      }
      break;
    }
    case EPI_RESID: {
      T* o = static_cast<T*>(e.out) + static_cast<int64_t>(m) * e.ldo + n;
      S::st(o, S::ld(o) + S::rnd(v0));
      if (has1) S::st(o + 1, S::ld(o + 1) + S::rnd(v1));
      break;
    }
    case EPI_SWIGLU: {
      T* o = static_cast<T*>(e.out) + static_cast<int64_t>(m) * e.ldo + (n >> 1);
      S::st(o, silu_f(S::rnd(v0)) * S::rnd(v1));
      break;
    }
    case EPI_QKV: {
      const T* b = static_cast<const T*>(e.bias);
      float a = S::rnd(v0 + S::ld(b + n));
      float c = S::rnd(v1 + S::ld(b + n + 1));
      const int d = e.dh;
      const int head = n / d;
      const int r = n - head * d;
      const int bt = m / e.T;
      const int t = m - bt * e.T;
      const int pos = (e.lens ? e.lens[bt] : e.d_len ? *e.d_len : e.len0) + t;
      if (head < e.nh + e.nkv) {
        const int p = r >> 1;
        const float2 cs = e.rope[static_cast<int64_t>(pos) * (d >> 1) + p];
        const float ra = S::rnd(a * cs.x - c * cs.y);
        const float rb = S::rnd(c * cs.x + a * cs.y);
        T* dst;
        if (head < e.nh) {
          dst = static_cast<T*>(e.out) + static_cast<int64_t>(m) * e.ldo + head * d;
        } else {
          dst = static_cast<T*>(e.kc) + bt * e.kv_bstride + (head - e.nh) * e.kv_hstride +
                static_cast<int64_t>(e.kv_rel ? t : pos) * d;
        }
        S::st(dst + p, ra);
        S::st(dst + p + (d >> 1), rb);
      } else {
        T* dst = static_cast<T*>(e.vc) + bt * e.kv_bstride + (head - e.nh - e.nkv) * e.kv_hstride +
                 static_cast<int64_t>(e.kv_rel ? t : pos) * d + r;
        S::st(dst, a);
        S::st(dst + 1, c);
      }
      break;
    }
    default:
      break;
  }
}

// Host-side launch descriptors for the GEMM family (gemm.hip).
// Y[m, n] = sum_k X[m, k] W[n, k], epilogue `epi`; W [N, K], X [M, K] with
// row strides ldw, ldx.  `scratch` (float32) is needed for split-K runs of
// the skinny kernel; `scratch_bytes` bounds it.
struct GemmArgs {
  const void* W;
  int64_t ldw;
  const void* X;
  int64_t ldx;
  int M, N, K;
  Epi epi;
  void* scratch;             // float32 split-K partials (GEMV path)
  size_t scratch_bytes;
  // a split plan whose partials exceed scratch_bytes runs unsplit instead of
  // failing (operator calls with a caller-sized workspace)
  bool unsplit_if_short;
  // fused RMSNorm of X's rows (GEMV path, M <= 16): X is the raw residual
  // stream, the kernel multiplies it by 1/sqrt(sum(norm_sq row)/K + eps) and
  // norm_w, rounded to the storage type, before the product
  const void* norm_w;
  const float* norm_sq;
  int64_t norm_sq_ld;
  float norm_eps;
  // fused split-KV merge (GEMV path, M <= 16, one query token per sequence):
  // X[m][h * 128 + d] is the attention output of sequence m, head h, merged
  // from att_nsplit partial results (unnormalised output, running max and sum)
  // laid out [m][kv head][split][16 rows][128] and [m][kv head][split][16]
  const float* att_o;
  const float2* att_ml;
  int att_nsplit, att_group, att_nkv;
  // deferred residual add (GEMV path with norm_w, M <= 16): X is the residual
  // stream before the previous layer's down projection, whose split-K
  // partials (resid_splits of them, [split][M][K] float32) are still pending.
  // The kernel forms rnd(X + rnd(sum of partials)) (what the split reduction
  // would have stored), normalises that row itself (norm_sq unused) and one
  // workgroup writes the new residual row to resid_out (not X).
  const float* resid_part;
  int resid_splits;
  void* resid_out;
  // split-K GEMV: leave the float32 partials in scratch and skip the
  // reduction kernel (a later product's prologue consumes them)
  bool defer_reduce;
  // RESID product followed by an RMSNorm of the new residual rows: where the
  // product's split-K reduction runs as a kernel of its own
  // (gemm_post_norm), that kernel also writes RMSNorm(rows) * post_w to
  // post_out (ld = N), exactly as the RMSNorm operator would
  void* post_out;
  const void* post_w;
  float post_eps;
  // QKV product (bf16, d = 128) whose split-K reduction runs as a kernel of
  // its own: with qkv_cache set (a paged and/or FP8 cache), that kernel also
  // writes the k and v rows straight into the cache (positions as the
  // epilogue's; FP8 rows quantised) and sets *qkv_cache_done, so that no
  // separate store of the staged rows is needed.  Without a split-K
  // reduction the epilogue writes epi.kc / epi.vc as usual and
  // *qkv_cache_done stays false.
  const KvLayout* qkv_cache;
  bool* qkv_cache_done;
  // Stream-K workspace (stream_k_bytes, zeroed once before its first use;
  // the kernels leave it zeroed): prefill products with fewer tiles than CUs
  // then share tiles between workgroups instead of leaving CUs idle.  Null:
  // plain tiles.
  void* sk_ws;
  size_t sk_ws_bytes;
  int sk_cus;  // compute units of the device the product runs on
};

q2_status gemm_bf16(const GemmArgs& a, hipStream_t s);
q2_status gemm_f32(const GemmArgs& a, hipStream_t s);
// GEMV path (M <= 64, bf16): gemv.hip.
constexpr int GEMV_MAX_M = 64;
constexpr int GEMV_NORM_MAX_M = 16;
// bytes of X the GEMV path stages in LDS (fused sources need it to fit)
constexpr size_t GEMV_STAGE_BYTES = size_t(64) << 10;
bool gemv_can_fuse(int M, int K);
// Whether a split-K residual add may be left to the next normalising GEMV.
bool gemv_can_defer(int M, int K);
q2_status gemv_bf16(const GemmArgs& a, hipStream_t s);
// Split-K partial bytes the GEMV path needs for this shape (0 if unsplit).
size_t gemv_scratch_bytes(int M, int N, int K);
// Number of K splits the GEMV path uses for this shape.
int gemv_splits(int M, int N, int K);
// Split-K partial bytes any bf16 decode-size product of this shape may need.
size_t gemm_scratch_bytes(int M, int N, int K);
// Sums split-K float32 partials partial[split][m][n] (a.scratch) in split
// order and applies a.epi (not the argmax epilogue); with a.post_out and the
// residual epilogue, also the RMSNorm of the new rows.
q2_status split_reduce(const GemmArgs& a, int splits, hipStream_t s);
// Whether gemm_bf16(a) writes a.post_out itself (else the caller norms).
bool gemm_post_norm(const GemmArgs& a);
// Compute units of device `device` (0 if unknown); bytes of the stream-K
// workspace for a device of `cus` compute units (GemmArgs::sk_ws), and the
// offset of its error word (non-zero after a hand-over wait timed out).
int device_cus(int device);
size_t stream_k_bytes(int cus);
size_t stream_k_err_offset();

}  // namespace q2
