// Qwen2 decoder model driver: packed weights, KV cache, activation arena,
// prefill in token chunks, single-token decode replayed from a HIP graph,
// and greedy generation with the next token fed back on the device.
//
// Per layer (x is the residual stream, stored in the model dtype):
//   h = rmsnorm(x, w_in)                         rmsnorm kernel
//   q, K/V cache <- rope(h Wqkv^T + b)           GEMM, QKV epilogue
//   att = attention(q, K, V)                     attention kernels
//   x = x + att Wo^T                             GEMM, residual epilogue
//   h = rmsnorm(x, w_post)                       rmsnorm kernel
//   act = silu(h Wg^T) * (h Wu^T)                GEMM, SwiGLU epilogue
//   x = x + act Wd^T                             GEMM, residual epilogue
// then rmsnorm of each sequence's last row, the LM head GEMM with a fused
// argmax epilogue, and a finalize kernel that turns the packed argmax keys
// into token ids, stores them for the next step and resets the keys.
//
// Decode steps of up to 16 sequences can also run as one persistent
// cooperative kernel per step (decode_mk.hip) that performs the same chain
// with grid barriers between the stages (q2_model_set_decode_path); the graph
// of per-operator kernels is the default and serves larger batches and the
// float32 model.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "attention.hpp"
#include "decode_mk.hpp"
#include "epilogue.hpp"
#include "kvcache.hpp"
#include "simple.hpp"

using namespace q2;

struct q2_model {
  q2_config cfg{};
  int device = 0;
  int esize = 2;
  int qkv_out = 0;
  int max_tok = 0;   // tokens per forward chunk
  // device memory
  char* wmem = nullptr;
  char* kvmem = nullptr;
  char* amem = nullptr;
  size_t wbytes = 0, kvbytes = 0, abytes = 0;
  // weights
  void* embed = nullptr;
  void* lm_head = nullptr;
  void* w_final = nullptr;
  struct Layer {
    void *w_in, *w_post, *w_qkv, *b_qkv, *w_o, *w_gu, *w_d;
  };
  std::vector<Layer> layers;
  // KV cache [L][Bmax][nkv][S][d]
  void* kc = nullptr;
  void* vc = nullptr;
  int64_t kv_lstride = 0, kv_bstride = 0, kv_hstride = 0;
  // FP8 cache (cfg.kv_fp8): kc / vc hold E4M3 codes (same layout, 1 byte per
  // element) and ks / vs one float32 scale per (layer, sequence, head,
  // position).  FP8 and paged caches stage new k / v rows as bf16 in kstage /
  // vstage [B][nkv][T][d], which kv_store writes (or quantises) into the
  // cache; their prefill attention reads the positions it needs expanded to
  // contiguous bf16 in kexp / vexp [B][nkv][S][d]
  bool fp8 = false;
  float* ks = nullptr;
  float* vs = nullptr;
  int64_t ks_lstride = 0;
  // paged cache (cfg.page_size > 0): each layer's K and V pools hold
  // pages_total pages of [nkv][page][d]; sequence b's positions
  // [p * page, (p + 1) * page) live in page d_table[b][p] (all layers);
  // d_lens[b] is sequence b's cached length (sequences may differ).  The host
  // keeps copies (h_table, h_lens) and the free list; pages are taken as
  // positions are reached and given back when a sequence is released.
  int page = 0;
  int pages_total = 0;
  int pages_per_seq = 0;
  int* d_table = nullptr;
  int* d_lens = nullptr;
  std::vector<int> h_table;
  std::vector<int> h_lens;
  std::vector<int> free_pages;
  int slot0 = 0;            // first slot of the rows of the current call (paged)
  void* kstage = nullptr;
  void* vstage = nullptr;
  void* kexp = nullptr;
  void* vexp = nullptr;
  float2* rope = nullptr;
  // arena
  void *x = nullptr, *h = nullptr, *q = nullptr, *att = nullptr, *act = nullptr, *xl = nullptr;
  // the buffer that holds the residual stream after the last forward: x, or
  // h when the fused decode path ping-pongs between the two
  void* xcur = nullptr;
  float* logits_buf = nullptr;
  unsigned long long* keys = nullptr;
  int64_t* ids_buf = nullptr;
  int64_t* hist = nullptr;
  int* d_len = nullptr;
  void* gscratch = nullptr;
  size_t gscratch_bytes = 0;
  // stream-K workspace of the prefill products (zeroed with the arena)
  void* skws = nullptr;
  size_t sk_bytes = 0;
  int cus = 0;
  void* ascratch = nullptr;
  size_t ascratch_bytes = 0;
  float* sq = nullptr;            // [max_tok][hidden / 16] row sums of squares (decode path)
  int64_t sq_ld = 0;
  // host state
  int len = 0;
  int cur_batch = 0;
  int last_rows = 0;      // rows of x written by the last chunk / step
  bool len_dirty = true;
  hipStream_t cap = nullptr;
  std::map<std::pair<int, int>, hipGraphExec_t> graphs;
  // persistent decode kernel (decode_mk.hip)
  bool mk_ok = false;      // buffers exist and a cooperative grid fits
  bool mk_on = false;      // use it when eligible (q2_model_set_decode_path)
  int mk_grid = 0;
  unsigned mk_epoch = 0;
  char* mkmem = nullptr;
  MkArgs mk{};             // everything but B, logits, epoch0
};

namespace {

__global__ void set_len_kernel(int* d_len, int v) { *d_len = v; }
// The device length, and with lens each of the B sequences' lengths, move on by t.
__global__ void advance_len_kernel(int* d_len, int t, int* lens, int B) {
  if (threadIdx.x == 0) *d_len += t;
  if (lens && static_cast<int>(threadIdx.x) < B) lens[threadIdx.x] += t;
}

// Paged cache: table[slot * stride + page_idx[i]] = page[i] for i < n, and
// lens[slot_len] = len_val when slot_len >= 0 (host-side page allocation and
// sequence release, applied in stream order).
struct TableEdits {
  int n;
  int slot[64], idx[64], page[64];
};
__global__ void table_edit_kernel(int* table, int64_t stride, TableEdits e, int* lens, int slot_len, int len_val) {
  const int i = threadIdx.x;
  if (i < e.n) table[static_cast<int64_t>(e.slot[i]) * stride + e.idx[i]] = e.page[i];
  if (i == 0 && slot_len >= 0) lens[slot_len] = len_val;
}

__global__ void copy_ids_kernel(int64_t* dst, int64_t dst_stride, const int64_t* src, int64_t src_stride, int B) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b < B) dst[b * dst_stride] = src[b * src_stride];
}

// Next token of each sequence from its KEY_SLOTS packed argmax keys: stores it
// for the next step (ids_buf), in the history at its position (len + pending),
// optionally in `next`; resets the keys; then moves the device length on by
// `pending` (the positions of this forward not yet counted).  One workgroup.
__global__ __launch_bounds__(1024) void finalize_kernel(unsigned long long* keys, int64_t* ids_buf, int64_t* hist,
                                                        int64_t hist_ld, int* d_len, int pending, int64_t* next,
                                                        int64_t next_stride, int B, int* lens) {
  // one wave per row, FIN_ROWS rows per wave at a time with their slot loads
  // in flight together; lane i takes key slot i
  static_assert(KEY_SLOTS == 64, "one key slot per lane");
  constexpr int FIN_ROWS = 4;
  const int pos = *d_len + pending;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  for (int b0 = wave * FIN_ROWS; b0 < B; b0 += nw * FIN_ROWS) {
    unsigned long long best[FIN_ROWS];
#pragma unroll
    for (int r = 0; r < FIN_ROWS; ++r)
      best[r] = b0 + r < B ? keys[static_cast<int64_t>(b0 + r) * KEY_ROW + lane * KEY_STRIDE] : 0ull;
#pragma unroll
    for (int r = 0; r < FIN_ROWS; ++r)
      if (b0 + r < B) keys[static_cast<int64_t>(b0 + r) * KEY_ROW + lane * KEY_STRIDE] = 0ull;
#pragma unroll
    for (int r = 0; r < FIN_ROWS; ++r)
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long k = __shfl_xor(best[r], o, 64);
        best[r] = k > best[r] ? k : best[r];
      }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < FIN_ROWS; ++r) {
        const int b = b0 + r;
        if (b >= B) break;
        const int64_t id = static_cast<int64_t>(argmax_key_index(best[r]));
        ids_buf[b] = id;
        if (lens) {
          // per-sequence position; this lane alone reads and moves lens[b]
          hist[b * hist_ld + lens[b] + pending] = id;
          lens[b] += pending;
        } else {
          hist[b * hist_ld + pos] = id;
        }
        if (next) next[b * next_stride] = id;
      }
    }
  }
  __syncthreads();  // every wave has read *d_len
  if (threadIdx.x == 0 && pending) *d_len += pending;
}

// out[b][c] = hist[b][start + c]; with lens, start = lens[b] - back (per
// sequence, after the steps moved lens on).
__global__ void copy_hist_kernel(int64_t* out, int64_t ld_out, const int64_t* hist, int64_t hist_ld, int start, int n,
                                 int B, const int* lens, int back) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n * B) return;
  const int b = i / n;
  const int c = i - b * n;
  out[b * ld_out + c] = hist[b * hist_ld + (lens ? lens[b] - back : start) + c];
}

__global__ void copy_logits_kernel(float* out, int64_t ld_out, const float* src, int64_t ld_src, int V, int B) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(V) * B) return;
  const int b = static_cast<int>(i / V);
  const int v = static_cast<int>(i - static_cast<int64_t>(b) * V);
  out[b * ld_out + v] = src[b * ld_src + v];
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

bool staged_kv(const q2_model* m) { return m->fp8 || m->page > 0; }

// Layer l's cache as KvLayout, for the rows of the current call (slot0 on).
KvLayout cache_layout(const q2_model* m, int l) {
  KvLayout c{};
  const int kv_es = m->fp8 ? 1 : m->esize;
  c.kc = static_cast<char*>(m->kc) + l * m->kv_lstride * kv_es;
  c.vc = static_cast<char*>(m->vc) + l * m->kv_lstride * kv_es;
  c.fp8 = m->fp8 ? 1 : 0;
  if (m->fp8) {
    c.ks = m->ks + l * m->ks_lstride;
    c.vs = m->vs + l * m->ks_lstride;
  }
  c.nkv = m->cfg.nkv;
  if (m->page > 0) {
    c.table = m->d_table + static_cast<int64_t>(m->slot0) * m->pages_per_seq;
    c.tstride = m->pages_per_seq;
    c.P = m->page;
  } else {
    c.hs = m->cfg.max_seq;
    c.bs = int64_t(m->cfg.max_seq) * m->cfg.nkv;
  }
  return c;
}

// Per-sequence lengths of the current call's rows (paged), else null.
const int* call_lens(const q2_model* m) { return m->page > 0 ? m->d_lens + m->slot0 : nullptr; }

q2_status gemm(const q2_model* m, const GemmArgs& a, hipStream_t s) {
  return m->cfg.dtype == Q2_BF16 ? gemm_bf16(a, s) : gemm_f32(a, s);
}

GemmArgs gemm_args(const q2_model* m, const void* W, int64_t ldw, const void* X, int64_t ldx, int M, int N, int K) {
  GemmArgs a{};
  a.W = W;
  a.ldw = ldw;
  a.X = X;
  a.ldx = ldx;
  a.M = M;
  a.N = N;
  a.K = K;
  a.scratch = m->gscratch;
  a.scratch_bytes = m->gscratch_bytes;
  a.sk_ws = m->skws;
  a.sk_ws_bytes = m->sk_bytes;
  a.sk_cus = m->cus;
  return a;
}

// Which kernels a forward of M token rows uses: up to 64 rows of a bf16 model
// go through the weight-streaming GEMV; up to 16 rows also fuse each RMSNorm
// into the GEMV that consumes it (fed by per-tile sums of squares).
struct Path {
  bool gemv;
  bool fused_norm;
  bool defer;  // split-K residual adds left to the next normalising GEMV
};
Path path_for(const q2_model* m, int M) {
  Path p;
  p.gemv = m->cfg.dtype == Q2_BF16 && M <= GEMV_MAX_M;
  p.fused_norm = p.gemv && gemv_can_fuse(M, m->cfg.hidden) && gemv_can_fuse(M, m->cfg.nh * m->cfg.dh);
  p.defer = p.fused_norm && gemv_can_defer(M, m->cfg.hidden);
  return p;
}

// Transformer layers for B sequences x Tc new tokens whose ids are already
// embedded in x.  Positions start at the device length; with `advance` the
// device length moves on by Tc at the end.
// Products of a layer, for measurement (q2_model_replay_stage).
// STAGE_ATTN_CORE: the attention kernel alone, leaving its split-KV partials
// unmerged (the merge launch, or o_proj's merging prologue, is left out).
enum Stage : int { STAGE_QKV = 0, STAGE_ATTN = 1, STAGE_O = 2, STAGE_GATE_UP = 3, STAGE_DOWN = 4, STAGE_ATTN_CORE = 5 };

// only_stage >= 0: launch nothing but that stage of layer only_layer (the
// launch decisions of every other stage are still taken, so the launched
// kernels and their arguments are those of the full forward).
template <typename T>
q2_status run_layers(q2_model* m, int B, int Tc, bool advance, hipStream_t s, int only_stage = -1,
                     int only_layer = -1) {
  const q2_config& c = m->cfg;
  const int M = B * Tc;
  const int H = c.hidden, d = c.dh, qd = c.nh * c.dh;
  const Path path = path_for(m, M);
  // With the fused norms the down projection's split-K reduction is folded
  // into the next layer's QKV prologue, which writes the completed residual
  // rows to the other of x / h (the reduction's in-place add would race with
  // the other workgroups reading the old rows).  The last layer reduces as
  // usual, for the head.
  void* cur = m->x;
  int pend_splits = 0;  // > 0: down-projection partials of the previous layer pending in gscratch
  // without the fused norms: h already holds the RMSNorm of the residual rows
  // (written by the previous residual product's split-K reduction)
  bool h_ready = false;
  for (int l = 0; l < c.nlayer; ++l) {
    auto want = [&](int st) {
      if (only_stage == STAGE_ATTN_CORE && st == STAGE_ATTN) st = STAGE_ATTN_CORE;
      return only_stage < 0 || (only_stage == st && only_layer == l);
    };
    const q2_model::Layer& L = m->layers[l];
    const int kv_es = m->fp8 ? 1 : m->esize;
    void* kc = static_cast<char*>(m->kc) + l * m->kv_lstride * kv_es;
    void* vc = static_cast<char*>(m->vc) + l * m->kv_lstride * kv_es;
    if (!path.fused_norm && !h_ready && want(STAGE_QKV))
      Q2_TRY(launch_rmsnorm<T>(static_cast<T*>(m->h), H, static_cast<const T*>(m->x), H,
                               static_cast<const T*>(L.w_in), M, H, c.eps, s));
    h_ready = false;
    {
      GemmArgs a = gemm_args(m, L.w_qkv, H, path.fused_norm ? cur : m->h, H, M, m->qkv_out, H);
      void* nxt = cur;
      if (path.fused_norm) {
        a.norm_w = L.w_in;
        a.norm_sq = m->sq;
        a.norm_sq_ld = m->sq_ld;
        a.norm_eps = c.eps;
        if (pend_splits > 0) {
          nxt = cur == m->x ? m->h : m->x;
          a.resid_part = static_cast<const float*>(m->gscratch);
          a.resid_splits = pend_splits;
          a.resid_out = nxt;
        }
      }
      a.epi.kind = EPI_QKV;
      a.epi.out = m->q;
      a.epi.ldo = qd;
      a.epi.bias = L.b_qkv;
      const bool stg = staged_kv(m);
      a.epi.kc = stg ? m->kstage : kc;
      a.epi.vc = stg ? m->vstage : vc;
      a.epi.kv_bstride = stg ? int64_t(c.nkv) * Tc * d : m->kv_bstride;
      a.epi.kv_hstride = stg ? int64_t(Tc) * d : m->kv_hstride;
      a.epi.kv_rel = stg ? 1 : 0;
      a.epi.lens = call_lens(m);
      a.epi.nh = c.nh;
      a.epi.nkv = c.nkv;
      a.epi.dh = d;
      a.epi.T = Tc;
      a.epi.d_len = m->d_len;
      a.epi.rope = m->rope;
      // a paged and/or FP8 cache: a split-K reduction of this product stores
      // the k / v rows itself, else kv_store does from the staged rows
      const KvLayout lay = cache_layout(m, l);
      bool stored = false;
      if (stg && m->cfg.dtype == Q2_BF16) {
        a.qkv_cache = &lay;
        a.qkv_cache_done = &stored;
      }
      if (want(STAGE_QKV)) Q2_TRY(gemm(m, a, s));
      cur = nxt;
      pend_splits = 0;
      if (staged_kv(m) && !stored && want(STAGE_QKV))
        Q2_TRY(launch_kv_store(lay, static_cast<const uint16_t*>(m->kstage),
                               static_cast<const uint16_t*>(m->vstage), B, Tc, call_lens(m), m->d_len, m->len, s));
    }
    // with one query per sequence and split-KV partials, o_proj merges them
    // itself -- when there are few: every o_proj workgroup merges all rows of
    // its heads, so the merge reads grow with rows x splits (8 rows x 10
    // splits cost more than the combine kernel and a plain product)
    const int nsplit = c.dtype == Q2_BF16 ? attention_decode_splits(B, Tc, c.max_seq, c.nh, c.nkv, d) : 0;
    const bool merge_in_o = path.fused_norm && Tc == 1 && nsplit > 1 && B * nsplit <= 16;
    {
      AttnArgs a{};
      a.leave_partials = merge_in_o || only_stage == STAGE_ATTN_CORE;
      a.q = m->q;
      a.q_bs = static_cast<int64_t>(Tc) * qd;
      a.q_ts = qd;
      a.q_hs = d;
      a.o = m->att;
      a.o_bs = a.q_bs;
      a.o_ts = a.q_ts;
      a.o_hs = a.q_hs;
      a.k = kc;
      a.v = vc;
      a.k_bs = a.v_bs = m->kv_bstride;
      a.k_ss = a.v_ss = d;
      a.k_hs = a.v_hs = m->kv_hstride;
      a.B = B;
      a.T = Tc;
      a.S = m->len + Tc;  // unused when d_len is set
      a.nh = c.nh;
      a.nkv = c.nkv;
      a.d = d;
      a.scale = static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
      a.d_len = m->d_len;
      a.s_max = c.max_seq;
      a.scratch = m->ascratch;
      a.scratch_bytes = m->ascratch_bytes;
      if (staged_kv(m)) {
        if (Tc * (c.nh / c.nkv) <= 16) {
          // decode kernel: reads the cache rows itself (per-sequence lengths when paged)
          a.use_cache = true;
          a.cache = cache_layout(m, l);
          a.lens = call_lens(m);
        } else {
          // prefill kernel: positions [0, len + Tc) expanded to contiguous bf16 first
          if (want(STAGE_ATTN))
            Q2_TRY(launch_kv_expand(static_cast<uint16_t*>(m->kexp), static_cast<uint16_t*>(m->vexp), c.max_seq,
                                    cache_layout(m, l), B, m->len + Tc, s));
          a.k = m->kexp;
          a.v = m->vexp;
          a.k_hs = a.v_hs = int64_t(c.max_seq) * d;
          a.k_bs = a.v_bs = a.k_hs * c.nkv;
        }
      }
      if (want(STAGE_ATTN)) Q2_TRY(c.dtype == Q2_BF16 ? attention_bf16(a, s) : attention_f32(a, s));
    }
    {
      GemmArgs a = gemm_args(m, L.w_o, qd, m->att, qd, M, H, qd);
      if (merge_in_o) {
        const size_t slots = static_cast<size_t>(B) * c.nkv * nsplit * 16;
        a.att_o = static_cast<const float*>(m->ascratch);
        a.att_ml = reinterpret_cast<const float2*>(static_cast<const float*>(m->ascratch) + slots * d);
        a.att_nsplit = nsplit;
        a.att_group = c.nh / c.nkv;
        a.att_nkv = c.nkv;
      }
      a.epi.kind = EPI_RESID;
      a.epi.out = cur;
      a.epi.ldo = H;
      a.epi.sq_out = path.fused_norm ? m->sq : nullptr;
      a.epi.sq_ld = m->sq_ld;
      if (!path.fused_norm && c.dtype == Q2_BF16) {
        a.post_out = m->h;
        a.post_w = L.w_post;
        a.post_eps = c.eps;
        h_ready = gemm_post_norm(a);
      }
      if (want(STAGE_O)) Q2_TRY(gemm(m, a, s));
    }
    if (!path.fused_norm && !h_ready && want(STAGE_GATE_UP))
      Q2_TRY(launch_rmsnorm<T>(static_cast<T*>(m->h), H, static_cast<const T*>(m->x), H,
                               static_cast<const T*>(L.w_post), M, H, c.eps, s));
    h_ready = false;
    {
      GemmArgs a = gemm_args(m, L.w_gu, H, path.fused_norm ? cur : m->h, H, M, 2 * c.inter, H);
      if (path.fused_norm) {
        a.norm_w = L.w_post;
        a.norm_sq = m->sq;
        a.norm_sq_ld = m->sq_ld;
        a.norm_eps = c.eps;
      }
      a.epi.kind = EPI_SWIGLU;
      a.epi.out = m->act;
      a.epi.ldo = c.inter;
      if (want(STAGE_GATE_UP)) Q2_TRY(gemm(m, a, s));
    }
    {
      GemmArgs a = gemm_args(m, L.w_d, c.inter, m->act, c.inter, M, H, c.inter);
      a.epi.kind = EPI_RESID;
      a.epi.out = cur;
      a.epi.ldo = H;
      a.epi.sq_out = path.fused_norm ? m->sq : nullptr;
      a.epi.sq_ld = m->sq_ld;
      if (path.defer && l + 1 < c.nlayer) {
        const int sp = gemv_splits(M, H, c.inter);
        if (sp > 1) {
          a.defer_reduce = true;
          pend_splits = sp;
        }
      }
      if (!path.fused_norm && c.dtype == Q2_BF16 && l + 1 < c.nlayer) {
        a.post_out = m->h;
        a.post_w = m->layers[l + 1].w_in;
        a.post_eps = c.eps;
        h_ready = gemm_post_norm(a);
      }
      if (want(STAGE_DOWN)) Q2_TRY(gemm(m, a, s));
    }
  }
  if (only_stage >= 0) return Q2_OK;
  m->xcur = cur;
  if (!advance) return Q2_OK;
  hipLaunchKernelGGL(advance_len_kernel, dim3(1), dim3(64), 0, s, m->d_len, Tc, const_cast<int*>(call_lens(m)), B);
  return check_launch("advance_len");
}

// Final norm of each sequence's last row, LM head with argmax, finalize.
// `pending` is the number of new positions the device length has not been
// advanced by yet (1 for a decode step, whose finalize advances it; 0 after
// a prefill, whose layers already did).
template <typename T>
q2_status run_head(q2_model* m, int B, int Tc, int pending, float* logits, int64_t ld_logits, int64_t* next,
                   int64_t next_stride, hipStream_t s) {
  const q2_config& c = m->cfg;
  const int H = c.hidden;
  const Path path = path_for(m, B * Tc);
  const bool fused = path.fused_norm && Tc == 1;
  if (!fused)
    Q2_TRY(launch_rmsnorm<T>(static_cast<T*>(m->xl), H,
                             static_cast<const T*>(m->xcur) + static_cast<int64_t>(Tc - 1) * H,
                             static_cast<int64_t>(Tc) * H, static_cast<const T*>(m->w_final), B, H, c.eps, s));
  GemmArgs a = gemm_args(m, m->lm_head, H, fused ? m->xcur : m->xl, H, B, c.vocab, H);
  if (fused) {
    a.norm_w = m->w_final;
    a.norm_sq = m->sq;
    a.norm_sq_ld = m->sq_ld;
    a.norm_eps = c.eps;
  }
  a.epi.kind = EPI_ARGMAX;
  a.epi.out = logits;
  a.epi.ldo = ld_logits;
  a.epi.keys = m->keys;
  Q2_TRY(gemm(m, a, s));
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, s, m->keys, m->ids_buf + m->slot0,
                     m->hist + static_cast<int64_t>(m->slot0) * (c.max_seq + 1), static_cast<int64_t>(c.max_seq) + 1,
                     m->d_len, pending, next, next_stride, B, const_cast<int*>(call_lens(m)));
  return check_launch("finalize");
}

// Copy hidden-state rows embeds[b, t0 + t, :] into x[b * tc + t, :].
// (with sq: also each row's sums of squares per 16-feature tile)
template <typename T>
__global__ __launch_bounds__(256) void load_embeds_kernel(T* x, const T* e, int64_t e_bs, int64_t e_ts, int tc, int H,
                                                          float* sq, int64_t sq_ld) {
  const int m = blockIdx.x;
  const int b = m / tc, t = m - b * tc;
  for (int i0 = 0; i0 < H; i0 += 256) {
    const int i = i0 + threadIdx.x;
    float v = 0.f;
    if (i < H) {
      const T xv = e[b * e_bs + t * e_ts + i];
      x[static_cast<int64_t>(m) * H + i] = xv;
      v = St<T>::ld(&xv);
    }
    if (sq) {
      float ss = v * v;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o, 64);
      if (i < H && (threadIdx.x & 15) == 0) sq[m * sq_ld + i / 16] = ss;
    }
  }
}

template <typename T>
q2_status prefill_impl(q2_model* m, const int64_t* ids, int64_t ids_bs, int64_t ids_ts, int B, int Tn, float* logits,
                       int64_t ld_logits, int64_t* next, int64_t next_stride, hipStream_t s,
                       const T* embeds = nullptr, int64_t e_bs = 0, int64_t e_ts = 0) {
  const int Tc_max = m->max_tok / B > 0 ? m->max_tok / B : 1;
  int tc = 0;
  for (int t0 = 0; t0 < Tn; t0 += tc) {
    tc = Tn - t0 < Tc_max ? Tn - t0 : Tc_max;
    float* sq = path_for(m, B * tc).fused_norm ? m->sq : nullptr;
    if (embeds) {
      hipLaunchKernelGGL(load_embeds_kernel<T>, dim3(B * tc), dim3(256), 0, s, static_cast<T*>(m->x),
                         embeds + t0 * e_ts, e_bs, e_ts, tc, m->cfg.hidden, sq, m->sq_ld);
      Q2_TRY(check_launch("load_embeds"));
    } else {
      Q2_TRY(launch_embedding<T>(static_cast<T*>(m->x), m->cfg.hidden, ids + t0 * ids_ts, ids_bs, ids_ts, B, tc,
                                 static_cast<const T*>(m->embed), m->cfg.hidden, m->cfg.vocab, m->cfg.hidden, s, sq,
                                 m->sq_ld));
    }
    Q2_TRY(run_layers<T>(m, B, tc, true, s));
    m->len += tc;
    m->last_rows = B * tc;
  }
  return run_head<T>(m, B, tc, 0, logits, ld_logits, next, next_stride, s);
}

// One decode step from ids_buf (the graph body).
template <typename T>
q2_status decode_body(q2_model* m, int B, bool want_logits, hipStream_t s) {
  float* sq = path_for(m, B).fused_norm ? m->sq : nullptr;
  Q2_TRY(launch_embedding<T>(static_cast<T*>(m->x), m->cfg.hidden, m->ids_buf, 1, 0, B, 1,
                             static_cast<const T*>(m->embed), m->cfg.hidden, m->cfg.vocab, m->cfg.hidden, s, sq,
                             m->sq_ld));
  Q2_TRY(run_layers<T>(m, B, 1, false, s));
  return run_head<T>(m, B, 1, 1, want_logits ? m->logits_buf : nullptr, m->cfg.vocab, nullptr, 0, s);
}

q2_status get_graph(q2_model* m, int B, bool want_logits, hipGraphExec_t* out) {
  auto key = std::make_pair(B, want_logits ? 1 : 0);
  auto it = m->graphs.find(key);
  if (it != m->graphs.end()) {
    *out = it->second;
    return Q2_OK;
  }
  Q2_HIP(hipStreamBeginCapture(m->cap, hipStreamCaptureModeThreadLocal));
  const int saved_len = m->len;
  q2_status st = m->cfg.dtype == Q2_BF16 ? decode_body<uint16_t>(m, B, want_logits, m->cap)
                                         : decode_body<float>(m, B, want_logits, m->cap);
  m->len = saved_len;
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(m->cap, &graph);
  if (st != Q2_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (e != hipSuccess) return fail(Q2_EHIP, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess) return fail(Q2_EHIP, "hipGraphInstantiate failed: %s", hipGetErrorString(e));
  m->graphs[key] = exec;
  *out = exec;
  return Q2_OK;
}

q2_status sync_len(q2_model* m, hipStream_t s) {
  if (!m->len_dirty) return Q2_OK;
  hipLaunchKernelGGL(set_len_kernel, dim3(1), dim3(1), 0, s, m->d_len, m->len);
  Q2_TRY(check_launch("set_len"));
  m->len_dirty = false;
  return Q2_OK;
}

q2_status check_batch(q2_model* m, int B, int add) {
  Q2_CHECK(B >= 1 && B <= m->cfg.max_batch, Q2_ESHAPE, "batch %d not in [1, %d]", B, m->cfg.max_batch);
  Q2_CHECK(m->len == 0 || B == m->cur_batch, Q2_ESTATE, "batch %d differs from the cached batch %d (reset first)", B,
           m->cur_batch);
  Q2_CHECK(static_cast<int64_t>(m->len) + add <= m->cfg.max_seq, Q2_ESTATE,
           "KV cache capacity exceeded: %d cached + %d new > %d", m->len, add, m->cfg.max_seq);
  return Q2_OK;
}

q2_status check_ids_2d(const q2_tensor* ids, int* B, int* Tn, int64_t* bs, int64_t* ts) {
  Q2_TRY(check_desc(ids, "ids"));
  Q2_CHECK(ids->dtype == Q2_I64, Q2_EDTYPE, "ids must be int64");
  Q2_CHECK(ids->ndim == 1 || ids->ndim == 2, Q2_ESHAPE, "ids must be [T] or [B, T]");
  *B = ids->ndim == 2 ? static_cast<int>(ids->shape[0]) : 1;
  *Tn = static_cast<int>(ids->shape[ids->ndim - 1]);
  *bs = ids->ndim == 2 ? ids->stride[0] : 0;
  *ts = ids->stride[ids->ndim - 1];
  return Q2_OK;
}

q2_status check_next(const q2_tensor* next, int B, int64_t* stride) {
  *stride = 0;
  if (!next) return Q2_OK;
  Q2_TRY(check_desc(next, "next"));
  Q2_CHECK(next->dtype == Q2_I64, Q2_EDTYPE, "next must be int64");
  Q2_CHECK(numel(*next) == B && next->ndim == 1, Q2_ESHAPE, "next must be [B]");
  *stride = next->stride[0];
  return Q2_OK;
}

q2_status check_logits(const q2_model* m, const q2_tensor* logits, int B, Rows* r) {
  if (!logits) return Q2_OK;
  Q2_TRY(as_rows(logits, "logits", r));
  Q2_CHECK(r->dtype == Q2_F32, Q2_EDTYPE, "logits must be f32");
  Q2_CHECK(r->rows == B && r->cols == m->cfg.vocab, Q2_ESHAPE, "logits must be [B, V]");
  return Q2_OK;
}

struct WeightSlot {
  void* dst;
  int64_t rows, cols;   // source shape ([rows] for vectors: cols = 1)
  int mode;             // pack_rows mode
  int64_t off;          // destination row offset
  int64_t dst_ld;       // destination row stride (elements)
};

q2_status find_slot(q2_model* m, const std::string& name, int layer, WeightSlot* w) {
  const q2_config& c = m->cfg;
  const int64_t H = c.hidden, d = c.dh, qd = int64_t(c.nh) * c.dh, kd = int64_t(c.nkv) * c.dh, I = c.inter;
  if (layer < 0) {
    Q2_CHECK(layer == -1, Q2_EINVAL, "layer must be -1 for global tensors");
    if (name == "embed_tokens") *w = {m->embed, c.vocab, H, 0, 0, H};
    else if (name == "lm_head") *w = {m->lm_head, c.vocab, H, 0, 0, H};
    else if (name == "norm") *w = {m->w_final, H, 1, 0, 0, 1};
    else return fail(Q2_EINVAL, "unknown global weight '%s'", name.c_str());
    return Q2_OK;
  }
  Q2_CHECK(layer < c.nlayer, Q2_EINVAL, "layer %d out of range", layer);
  const q2_model::Layer& L = m->layers[layer];
  if (name == "input_layernorm") *w = {L.w_in, H, 1, 0, 0, 1};
  else if (name == "post_attention_layernorm") *w = {L.w_post, H, 1, 0, 0, 1};
  else if (name == "q_proj.weight") *w = {L.w_qkv, qd, H, 1, 0, H};
  else if (name == "k_proj.weight") *w = {L.w_qkv, kd, H, 1, qd, H};
  else if (name == "v_proj.weight") *w = {L.w_qkv, kd, H, 0, qd + kd, H};
  else if (name == "q_proj.bias") *w = {L.b_qkv, qd, 1, 1, 0, 1};
  else if (name == "k_proj.bias") *w = {L.b_qkv, kd, 1, 1, qd, 1};
  else if (name == "v_proj.bias") *w = {L.b_qkv, kd, 1, 0, qd + kd, 1};
  else if (name == "o_proj.weight") *w = {L.w_o, H, qd, 0, 0, qd};
  else if (name == "gate_proj.weight") *w = {L.w_gu, I, H, 2, 0, H};
  else if (name == "up_proj.weight") *w = {L.w_gu, I, H, 2, 1, H};
  else if (name == "down_proj.weight") *w = {L.w_d, H, I, 0, 0, I};
  else return fail(Q2_EINVAL, "unknown layer weight '%s'", name.c_str());
  (void)d;
  return Q2_OK;
}

}  // namespace

// Buffers and arguments of the persistent decode kernel, when the model
// qualifies (bf16, head_dim 128, at most MK_MAX_BATCH sequences) and a
// cooperative grid with one workgroup per CU fits.
static q2_status setup_persistent(q2_model* m) {
  const q2_config& c = m->cfg;
  if (c.dtype != Q2_BF16 || c.dh != 128 || c.max_batch > MK_MAX_BATCH || c.hidden % 16 != 0 ||
      c.inter % 16 != 0 || m->fp8 || m->page)
    return Q2_OK;
  // the norm prologue spreads a row over 8 / B waves (one wave per row from
  // batch 8 on), each lane holding at most MK_NORM_CHUNKS 16-byte chunks
  const int wpr = c.max_batch >= 8 ? 1 : 8 / c.max_batch;
  if (c.hidden / 8 > 64 * wpr * MK_NORM_CHUNKS) return Q2_OK;
  const int H = c.hidden, QD = c.nh * c.dh, B = c.max_batch, L = c.nlayer, I = c.inter;
  int grid = 0;
  Q2_TRY(mk_max_grid(B, H, QD, &grid));
  if (grid <= 0) return Q2_OK;
  MkArgs& a = m->mk;
  a.att_nsplit_max = MK_ATT_SPLITS;
  // split the down projection over K so that its (tile, split) work items,
  // one workgroup each, cover most of the grid
  const int tiles = cdiv(H, 16), nkb = cdiv(I, 128);
  const int splits = std::max(1, std::min(std::min(nkb, MK_DOWN_SPLITS), grid / tiles));
  a.down_bps = cdiv(nkb, splits);
  a.down_splits = cdiv(nkb, a.down_bps);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t o_layers = take(sizeof(MkLayer) * L);
  const size_t o_xres = take(size_t(L + 1) * B * H * 2), o_xmid = take(size_t(L) * B * H * 2);
  const size_t o_q = take(size_t(L) * B * QD * 2), o_act = take(size_t(L) * B * I * 2);
  const size_t slots = size_t(L) * B * c.nkv * a.att_nsplit_max * 16;
  const size_t o_atto = take(slots * 128 * sizeof(float)), o_attml = take(slots * sizeof(float2));
  const size_t o_down = take(size_t(L) * a.down_splits * B * H * sizeof(float));
  const size_t o_bar = take((size_t(grid) * 33 + 64) * sizeof(unsigned));
  if (hipMalloc(&m->mkmem, off) != hipSuccess) {
    (void)hipGetLastError();
    return Q2_OK;  // the per-operator path still works
  }
  Q2_HIP(hipMemset(m->mkmem, 0, off));
  std::vector<MkLayer> hl(L);
  for (int l = 0; l < L; ++l) {
    const q2_model::Layer& w = m->layers[l];
    hl[l].w_in = static_cast<const uint16_t*>(w.w_in);
    hl[l].w_post = static_cast<const uint16_t*>(w.w_post);
    hl[l].w_qkv = static_cast<const uint16_t*>(w.w_qkv);
    hl[l].b_qkv = static_cast<const uint16_t*>(w.b_qkv);
    hl[l].w_o = static_cast<const uint16_t*>(w.w_o);
    hl[l].w_gu = static_cast<const uint16_t*>(w.w_gu);
    hl[l].w_d = static_cast<const uint16_t*>(w.w_d);
    hl[l].kc = static_cast<uint16_t*>(m->kc) + int64_t(l) * m->kv_lstride;
    hl[l].vc = static_cast<uint16_t*>(m->vc) + int64_t(l) * m->kv_lstride;
  }
  Q2_HIP(hipMemcpy(m->mkmem + o_layers, hl.data(), sizeof(MkLayer) * L, hipMemcpyHostToDevice));
  a.layers = reinterpret_cast<const MkLayer*>(m->mkmem + o_layers);
  a.L = L;
  a.H = H;
  a.nh = c.nh;
  a.nkv = c.nkv;
  a.I = I;
  a.V = c.vocab;
  a.eps = c.eps;
  a.scale = static_cast<float>(1.0 / sqrt(static_cast<double>(c.dh)));
  a.embed = static_cast<const uint16_t*>(m->embed);
  a.w_final = static_cast<const uint16_t*>(m->w_final);
  a.lm_head = static_cast<const uint16_t*>(m->lm_head);
  a.kv_bstride = m->kv_bstride;
  a.kv_hstride = m->kv_hstride;
  a.rope = m->rope;
  a.d_len = m->d_len;
  a.ids_buf = m->ids_buf;
  a.hist = m->hist;
  a.hist_ld = static_cast<int64_t>(c.max_seq) + 1;
  a.keys = m->keys;
  a.xres = reinterpret_cast<uint16_t*>(m->mkmem + o_xres);
  a.xmid = reinterpret_cast<uint16_t*>(m->mkmem + o_xmid);
  a.qbuf = reinterpret_cast<uint16_t*>(m->mkmem + o_q);
  a.act = reinterpret_cast<uint16_t*>(m->mkmem + o_act);
  a.att_o = reinterpret_cast<float*>(m->mkmem + o_atto);
  a.att_ml = reinterpret_cast<float2*>(m->mkmem + o_attml);
  a.down_part = reinterpret_cast<float*>(m->mkmem + o_down);
  a.bar_flags = reinterpret_cast<unsigned*>(m->mkmem + o_bar);
  a.err = a.bar_flags + grid;
  a.bar_release = a.bar_flags + grid + 32;  // [grid][32]
  m->mk_grid = grid;
  m->mk_ok = true;
  m->abytes += off;
  return Q2_OK;
}

static bool use_persistent(const q2_model* m, int B) { return m->mk_ok && m->mk_on && B <= MK_MAX_BATCH; }

// One decode step on the persistent kernel (ids_buf holds the input tokens).
static q2_status persistent_step(q2_model* m, int B, bool want_logits, hipStream_t s) {
  MkArgs a = m->mk;
  a.B = B;
  a.logits = want_logits ? m->logits_buf : nullptr;
  a.epoch0 = m->mk_epoch;
  a.lds_x_bytes = static_cast<int>(mk_lds_x_bytes(B, a.H, a.nh * 128));
  Q2_TRY(mk_launch(a, m->mk_grid, s));
  m->mk_epoch += static_cast<unsigned>(mk_barriers(a.L));
  return Q2_OK;
}

// ------------------------------------------------------------------ paged cache bookkeeping

// Queue one table entry; flush 64 at a time (and at the end) as a kernel on s.
static q2_status table_flush(q2_model* m, TableEdits& e, hipStream_t s, int slot_len = -1, int len_val = 0) {
  if (e.n == 0 && slot_len < 0) return Q2_OK;
  hipLaunchKernelGGL(table_edit_kernel, dim3(1), dim3(64), 0, s, m->d_table, static_cast<int64_t>(m->pages_per_seq),
                     e, m->d_lens, slot_len, len_val);
  e.n = 0;
  return check_launch("table_edit");
}

static q2_status table_set(q2_model* m, TableEdits& e, int slot, int idx, int page, hipStream_t s) {
  m->h_table[static_cast<size_t>(slot) * m->pages_per_seq + idx] = page;
  e.slot[e.n] = slot;
  e.idx[e.n] = idx;
  e.page[e.n] = page;
  if (++e.n == 64) return table_flush(m, e, s);
  return Q2_OK;
}

// Pages for positions [h_lens[b], h_lens[b] + T) of slots slot0 .. slot0 + B - 1
// (all or nothing: on failure every page taken here goes back and nothing
// is launched).
static q2_status paged_reserve(q2_model* m, int slot0, int B, int T, hipStream_t s) {
  const int P = m->page;
  std::vector<std::pair<int, int>> taken;  // (slot, page index)
  for (int b = slot0; b < slot0 + B; ++b) {
    const int len = m->h_lens[b];
    Q2_CHECK(static_cast<int64_t>(len) + T <= m->cfg.max_seq, Q2_ESTATE,
             "sequence %d: %d cached + %d new positions exceed max_seq %d", b, len, T, m->cfg.max_seq);
    for (int p = len / P; p < cdiv(len + T, P); ++p) {
      int& e = m->h_table[static_cast<size_t>(b) * m->pages_per_seq + p];
      if (e >= 0) continue;
      if (m->free_pages.empty()) {
        for (auto& t : taken) {
          int& r = m->h_table[static_cast<size_t>(t.first) * m->pages_per_seq + t.second];
          m->free_pages.push_back(r);
          r = -1;
        }
        return fail(Q2_ESTATE, "KV cache out of pages (%d pages of %d positions)", m->pages_total, P);
      }
      e = m->free_pages.back();
      m->free_pages.pop_back();
      taken.emplace_back(b, p);
    }
  }
  TableEdits ed{};
  for (auto& t : taken)
    Q2_TRY(table_set(m, ed, t.first, t.second, m->h_table[static_cast<size_t>(t.first) * m->pages_per_seq + t.second],
                     s));
  return table_flush(m, ed, s);
}

// Give slot's pages back and set its length to 0 (host and device).
static q2_status paged_release(q2_model* m, int slot, hipStream_t s) {
  TableEdits ed{};
  for (int p = 0; p < m->pages_per_seq; ++p) {
    int& e = m->h_table[static_cast<size_t>(slot) * m->pages_per_seq + p];
    if (e < 0) continue;
    m->free_pages.push_back(e);
    Q2_TRY(table_set(m, ed, slot, p, -1, s));
  }
  m->h_lens[slot] = 0;
  return table_flush(m, ed, s, slot, 0);
}

// Before a call on slots slot0 .. slot0 + B - 1 that adds T positions each:
// equal lengths when `uniform`, at least `min_len` cached, then the pages.
static q2_status paged_begin(q2_model* m, int slot0, int B, int T, bool uniform, int min_len, hipStream_t s) {
  Q2_CHECK(slot0 >= 0 && B >= 1 && slot0 + B <= m->cfg.max_batch, Q2_ESHAPE, "slots %d .. %d not in [0, %d)", slot0,
           slot0 + B - 1, m->cfg.max_batch);
  for (int b = slot0; b < slot0 + B; ++b) {
    Q2_CHECK(m->h_lens[b] >= min_len, Q2_ESTATE, "sequence %d has %d cached positions (needs %d)", b, m->h_lens[b],
             min_len);
    Q2_CHECK(!uniform || m->h_lens[b] == m->h_lens[slot0], Q2_ESTATE,
             "sequences %d and %d have different lengths: prefill them one at a time (q2_model_seq_prefill)", slot0, b);
  }
  Q2_TRY(paged_reserve(m, slot0, B, T, s));
  m->slot0 = slot0;
  m->len = m->h_lens[slot0];
  m->len_dirty = true;
  return sync_len(m, s);
}

static void paged_end(q2_model* m, int slot0, int B, int T) {
  for (int b = slot0; b < slot0 + B; ++b) m->h_lens[b] += T;
  m->slot0 = 0;
  m->len = m->h_lens[0];
  m->len_dirty = true;
}

// ==================================================================== C ABI

extern "C" q2_status q2_model_create(const q2_config* cfg, int32_t device, q2_model** out) {
  clear_error();
  Q2_CHECK(cfg && out, Q2_EINVAL, "null argument");
  *out = nullptr;
  const q2_config c = *cfg;
  Q2_CHECK(c.dtype == Q2_F32 || c.dtype == Q2_BF16, Q2_EDTYPE, "model dtype must be f32 or bf16");
  Q2_CHECK(c.nlayer >= 1 && c.hidden >= 1 && c.nh >= 1 && c.nkv >= 1 && c.dh >= 2 && c.inter >= 1 && c.vocab >= 1 &&
               c.max_seq >= 1 && c.max_batch >= 1,
           Q2_ESHAPE, "all sizes must be positive");
  Q2_CHECK(c.nh % c.nkv == 0, Q2_ESHAPE, "nh must be a multiple of nkv");
  Q2_CHECK(c.dh % 2 == 0, Q2_ESHAPE, "head dim must be even");
  Q2_CHECK(c.max_batch <= 64, Q2_ESHAPE, "max_batch must be <= 64");
  Q2_CHECK(c.eps >= 0.f && c.theta > 0.f, Q2_EINVAL, "bad eps / theta");
  Q2_CHECK(c.kv_fp8 == 0 || c.kv_fp8 == 1, Q2_EINVAL, "kv_fp8 must be 0 or 1");
  Q2_CHECK(!c.kv_fp8 || c.dtype == Q2_BF16, Q2_EDTYPE, "the FP8 KV cache needs a bf16 model");
  Q2_CHECK(!c.kv_fp8 || c.nh / c.nkv <= 16, Q2_ESHAPE, "the FP8 KV cache needs at most 16 query heads per KV head");
  Q2_CHECK(c.page_size >= 0 && c.page_size % 64 == 0 && c.kv_pages >= 0, Q2_EINVAL,
           "page_size must be a non-negative multiple of 64 and kv_pages non-negative");
  Q2_CHECK(c.page_size == 0 || (c.dtype == Q2_BF16 && c.nh / c.nkv <= 16), Q2_EDTYPE,
           "the paged KV cache needs a bf16 model with at most 16 query heads per KV head");
  if (c.dtype == Q2_BF16) {
    Q2_CHECK(c.dh == 128, Q2_ESHAPE, "bf16 model needs head_dim 128");
    Q2_CHECK(c.hidden % 32 == 0 && c.inter % 32 == 0, Q2_ESHAPE, "bf16 model needs hidden and inter multiples of 32");
  } else {
    Q2_CHECK(c.dh <= 256 && c.max_seq <= 16384, Q2_ESHAPE, "f32 model: head_dim <= 256, max_seq <= 16384");
  }
  int ndev = 0;
  Q2_HIP(hipGetDeviceCount(&ndev));
  Q2_CHECK(device >= 0 && device < ndev, Q2_EINVAL, "device %d not present", device);
  Q2_HIP(hipSetDevice(device));

  q2_model* m = new (std::nothrow) q2_model();
  Q2_CHECK(m, Q2_ENOMEM, "host allocation failed");
  m->cfg = c;
  m->device = device;
  m->esize = c.dtype == Q2_BF16 ? 2 : 4;
  m->fp8 = c.kv_fp8 != 0;
  m->page = c.page_size;
  if (m->page) {
    m->pages_per_seq = cdiv(c.max_seq, m->page);
    m->pages_total = c.kv_pages ? c.kv_pages : c.max_batch * m->pages_per_seq;
  }
  m->qkv_out = (c.nh + 2 * c.nkv) * c.dh;
  const size_t es = m->esize;
  const size_t H = c.hidden, I = c.inter, V = c.vocab, qd = size_t(c.nh) * c.dh;

  // weights
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t o_embed = take(V * H * es), o_lm = take(V * H * es), o_final = take(H * es);
  std::vector<size_t> lo(size_t(c.nlayer) * 7);
  for (int l = 0; l < c.nlayer; ++l) {
    size_t* p = &lo[size_t(l) * 7];
    p[0] = take(H * es);
    p[1] = take(H * es);
    p[2] = take(size_t(m->qkv_out) * H * es);
    p[3] = take(size_t(m->qkv_out) * es);
    p[4] = take(H * qd * es);
    p[5] = take(2 * I * H * es);
    p[6] = take(H * I * es);
  }
  m->wbytes = off;

  // KV cache: [L][Bmax][nkv][S][d], or paged [L][pages][nkv][page][d]
  m->kv_hstride = int64_t(c.max_seq) * c.dh;
  m->kv_bstride = m->kv_hstride * c.nkv;
  m->kv_lstride = m->page ? int64_t(m->pages_total) * c.nkv * m->page * c.dh : m->kv_bstride * c.max_batch;
  const size_t kv_one = size_t(m->kv_lstride) * c.nlayer * (m->fp8 ? 1 : es);
  m->ks_lstride = m->kv_lstride / c.dh;
  const size_t ks_one = m->fp8 ? size_t(m->ks_lstride) * c.nlayer * sizeof(float) : 0;
  m->kvbytes = 2 * align256(kv_one) + 2 * align256(ks_one);

  // arena
  const int64_t bs = int64_t(c.max_batch) * c.max_seq;
  m->max_tok = static_cast<int>(bs < 16384 ? bs : 16384);
  if (m->max_tok < c.max_batch) m->max_tok = c.max_batch;
  const size_t mt = m->max_tok;
  off = 0;
  const size_t a_rope = take(size_t(c.max_seq) * (c.dh / 2) * sizeof(float2));
  const size_t a_x = take(mt * H * es), a_h = take(mt * H * es), a_q = take(mt * qd * es), a_att = take(mt * qd * es);
  const size_t a_act = take(mt * I * es), a_xl = take(size_t(c.max_batch) * H * es);
  const size_t a_logits = take(size_t(c.max_batch) * V * sizeof(float));
  const size_t a_keys = take(size_t(c.max_batch) * KEY_ROW * 8), a_ids = take(size_t(c.max_batch) * 8);
  const size_t a_hist = take(size_t(c.max_batch) * (c.max_seq + 1) * 8), a_len = take(sizeof(int));
  m->sq_ld = c.hidden / 16;
  const size_t a_sq = take(mt * size_t(m->sq_ld) * sizeof(float));
  size_t gs = 0;
  {
    const int shapes[4][2] = {{m->qkv_out, c.hidden}, {c.hidden, int(qd)}, {2 * c.inter, c.hidden}, {c.hidden, c.inter}};
    for (int i = 0; i < 4; ++i)
      for (int mm2 = 1; mm2 <= m->max_tok && mm2 <= GEMV_MAX_M; ++mm2) {
        size_t b = gemm_scratch_bytes(mm2, shapes[i][0], shapes[i][1]);
        gs = b > gs ? b : gs;
      }
  }
  m->gscratch_bytes = gs;
  const size_t a_gs = take(gs);
  m->cus = device_cus(m->device);
  m->sk_bytes = (c.dtype == Q2_BF16 && m->max_tok >= 512) ? stream_k_bytes(m->cus) : 0;
  const size_t a_sk = take(m->sk_bytes);
  size_t as = 0;
  if (c.dtype == Q2_BF16)
    for (int b = 1; b <= c.max_batch; ++b) {
      const int group = c.nh / c.nkv;
      for (int t = 1; t * group <= 16; ++t) {
        size_t x = attention_scratch_bytes(b, t, c.max_seq, c.nh, c.nkv, c.dh);
        as = x > as ? x : as;
      }
      // prefill chunks of up to max_tok / b tokens (split query blocks)
      const int tc = std::max(1, std::min(m->max_tok / b, c.max_seq));
      if (tc * group > 16) {
        const size_t x = attention_scratch_bytes(b, tc, c.max_seq, c.nh, c.nkv, c.dh);
        as = x > as ? x : as;
      }
    }
  m->ascratch_bytes = as;
  const size_t a_as = take(as);
  const bool staged = m->fp8 || m->page > 0;
  const size_t stage_b = staged ? mt * c.nkv * c.dh * es : 0;
  const size_t exp_b = staged ? size_t(c.max_batch) * c.nkv * c.max_seq * c.dh * es : 0;
  const size_t a_ks = take(stage_b), a_vs = take(stage_b), a_ke = take(exp_b), a_ve = take(exp_b);
  const size_t tab_n = m->page ? size_t(c.max_batch) * m->pages_per_seq : 0;
  const size_t a_tab = take(tab_n * sizeof(int)), a_lens = take(m->page ? size_t(c.max_batch) * sizeof(int) : 0);
  m->abytes = off;

  auto cleanup = [&](q2_status st) {
    q2_model_destroy(m);
    return st;
  };
  if (hipMalloc(&m->wmem, m->wbytes) != hipSuccess || hipMalloc(&m->kvmem, m->kvbytes) != hipSuccess ||
      hipMalloc(&m->amem, m->abytes) != hipSuccess) {
    (void)hipGetLastError();
    return cleanup(fail(Q2_ENOMEM, "device allocation of %.2f GB failed",
                        double(m->wbytes + m->kvbytes + m->abytes) / 1e9));
  }
  if (hipMemset(m->wmem, 0, m->wbytes) != hipSuccess || hipMemset(m->kvmem, 0, m->kvbytes) != hipSuccess ||
      hipMemset(m->amem, 0, m->abytes) != hipSuccess)
    return cleanup(fail(Q2_EHIP, "hipMemset failed"));
  m->embed = m->wmem + o_embed;
  m->lm_head = m->wmem + o_lm;
  m->w_final = m->wmem + o_final;
  m->layers.resize(c.nlayer);
  for (int l = 0; l < c.nlayer; ++l) {
    const size_t* p = &lo[size_t(l) * 7];
    m->layers[l] = {m->wmem + p[0], m->wmem + p[1], m->wmem + p[2], m->wmem + p[3],
                    m->wmem + p[4], m->wmem + p[5], m->wmem + p[6]};
  }
  m->kc = m->kvmem;
  m->vc = m->kvmem + align256(kv_one);
  if (m->fp8) {
    m->ks = reinterpret_cast<float*>(m->kvmem + 2 * align256(kv_one));
    m->vs = reinterpret_cast<float*>(m->kvmem + 2 * align256(kv_one) + align256(ks_one));
  }
  if (staged) {
    m->kstage = m->amem + a_ks;
    m->vstage = m->amem + a_vs;
    m->kexp = m->amem + a_ke;
    m->vexp = m->amem + a_ve;
  }
  if (m->page) {
    m->d_table = reinterpret_cast<int*>(m->amem + a_tab);
    m->d_lens = reinterpret_cast<int*>(m->amem + a_lens);
    if (hipMemset(m->d_table, 0xFF, tab_n * sizeof(int)) != hipSuccess)  // every entry -1: no page
      return cleanup(fail(Q2_EHIP, "hipMemset failed"));
    m->h_table.assign(tab_n, -1);
    m->h_lens.assign(c.max_batch, 0);
    m->free_pages.resize(m->pages_total);
    for (int i = 0; i < m->pages_total; ++i) m->free_pages[i] = m->pages_total - 1 - i;
  }
  m->rope = reinterpret_cast<float2*>(m->amem + a_rope);
  m->x = m->amem + a_x;
  m->h = m->amem + a_h;
  m->xcur = m->x;
  m->q = m->amem + a_q;
  m->att = m->amem + a_att;
  m->act = m->amem + a_act;
  m->xl = m->amem + a_xl;
  m->logits_buf = reinterpret_cast<float*>(m->amem + a_logits);
  m->keys = reinterpret_cast<unsigned long long*>(m->amem + a_keys);
  m->ids_buf = reinterpret_cast<int64_t*>(m->amem + a_ids);
  m->hist = reinterpret_cast<int64_t*>(m->amem + a_hist);
  m->d_len = reinterpret_cast<int*>(m->amem + a_len);
  m->gscratch = gs ? m->amem + a_gs : nullptr;
  m->skws = m->sk_bytes ? m->amem + a_sk : nullptr;
  m->ascratch = as ? m->amem + a_as : nullptr;
  m->sq = reinterpret_cast<float*>(m->amem + a_sq);
  if (hipStreamCreateWithFlags(&m->cap, hipStreamNonBlocking) != hipSuccess)
    return cleanup(fail(Q2_EHIP, "stream creation failed"));
  q2_status st = launch_rope_table(m->rope, c.max_seq, c.dh, c.theta, nullptr);
  if (st != Q2_OK) return cleanup(st);
  st = setup_persistent(m);
  if (st != Q2_OK) return cleanup(st);
  if (hipDeviceSynchronize() != hipSuccess) return cleanup(fail(Q2_EHIP, "device synchronize failed"));
  *out = m;
  return Q2_OK;
}

extern "C" q2_status q2_model_device_bytes(const q2_model* m, size_t* bytes) {
  clear_error();
  Q2_CHECK(m && bytes, Q2_EINVAL, "null argument");
  *bytes = m->wbytes + m->kvbytes + m->abytes;
  return Q2_OK;
}

extern "C" q2_status q2_model_load_weight(q2_model* m, const char* name, int32_t layer, const q2_tensor* src,
                                          void* stream) {
  clear_error();
  Q2_CHECK(m && name, Q2_EINVAL, "null argument");
  Q2_TRY(check_desc(src, "src"));
  WeightSlot w{};
  Q2_TRY(find_slot(m, name, layer, &w));
  Q2_CHECK(src->dtype == m->cfg.dtype, Q2_EDTYPE, "weight '%s' dtype differs from the model dtype", name);
  Q2_CHECK(is_contiguous(*src), Q2_ESTRIDE, "weight '%s' must be contiguous", name);
  const bool vec = w.cols == 1;
  if (vec) {
    Q2_CHECK(src->ndim == 1 && src->shape[0] == w.rows, Q2_ESHAPE, "weight '%s' must be [%lld]", name,
             (long long)w.rows);
  } else {
    Q2_CHECK(src->ndim == 2 && src->shape[0] == w.rows && src->shape[1] == w.cols, Q2_ESHAPE,
             "weight '%s' must be [%lld, %lld]", name, (long long)w.rows, (long long)w.cols);
  }
  return launch_pack_rows(w.dst, w.dst_ld, src->data, vec ? 1 : w.cols, w.rows, w.cols, m->esize, w.mode, m->cfg.dh,
                          w.off, static_cast<hipStream_t>(stream));
}

extern "C" q2_status q2_model_prefill(q2_model* m, const q2_tensor* ids, const q2_tensor* next,
                                      const q2_tensor* logits, void* stream) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  int B = 0, Tn = 0;
  int64_t bs = 0, ts = 0, ns = 0;
  Q2_TRY(check_ids_2d(ids, &B, &Tn, &bs, &ts));
  Q2_CHECK(Tn >= 1, Q2_ESHAPE, "prefill needs at least one token");
  if (!m->page) Q2_TRY(check_batch(m, B, Tn));
  Q2_TRY(check_next(next, B, &ns));
  Rows lg{};
  Q2_TRY(check_logits(m, logits, B, &lg));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m->page)
    Q2_TRY(paged_begin(m, 0, B, Tn, true, 0, s));
  else
    Q2_TRY(sync_len(m, s));
  m->cur_batch = B;
  const int64_t* ip = static_cast<const int64_t*>(ids->data);
  int64_t* np = next ? static_cast<int64_t*>(next->data) : nullptr;
  float* lp = logits ? reinterpret_cast<float*>(lg.data) : nullptr;
  const q2_status st = m->cfg.dtype == Q2_BF16 ? prefill_impl<uint16_t>(m, ip, bs, ts, B, Tn, lp, lg.ld, np, ns, s)
                                               : prefill_impl<float>(m, ip, bs, ts, B, Tn, lp, lg.ld, np, ns, s);
  if (m->page) paged_end(m, 0, B, Tn);
  return st;
}

extern "C" q2_status q2_model_seq_prefill(q2_model* m, int32_t slot, const q2_tensor* ids, const q2_tensor* next,
                                          const q2_tensor* logits, void* stream) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  Q2_CHECK(m->page > 0, Q2_ESTATE, "q2_model_seq_prefill needs a paged KV cache (page_size > 0)");
  Q2_TRY(check_desc(ids, "ids"));
  Q2_CHECK(ids->dtype == Q2_I64, Q2_EDTYPE, "ids must be int64");
  Q2_CHECK(ids->ndim == 1, Q2_ESHAPE, "ids must be [T]");
  const int Tn = static_cast<int>(ids->shape[0]);
  Q2_CHECK(Tn >= 1, Q2_ESHAPE, "prefill needs at least one token");
  int64_t ns = 0;
  Q2_TRY(check_next(next, 1, &ns));
  Rows lg{};
  Q2_TRY(check_logits(m, logits, 1, &lg));
  Q2_CHECK(slot >= 0 && slot < m->cfg.max_batch, Q2_ESHAPE, "slot %d not in [0, %d)", slot, m->cfg.max_batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  Q2_TRY(paged_begin(m, slot, 1, Tn, true, 0, s));
  const int64_t* ip = static_cast<const int64_t*>(ids->data);
  int64_t* np = next ? static_cast<int64_t*>(next->data) : nullptr;
  float* lp = logits ? reinterpret_cast<float*>(lg.data) : nullptr;
  const q2_status st = prefill_impl<uint16_t>(m, ip, 0, ids->stride[0], 1, Tn, lp, lg.ld, np, ns, s);
  paged_end(m, slot, 1, Tn);
  m->cur_batch = std::max(m->cur_batch, static_cast<int>(slot) + 1);
  return st;
}

extern "C" q2_status q2_model_seq_release(q2_model* m, int32_t slot, void* stream) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  Q2_CHECK(m->page > 0, Q2_ESTATE, "q2_model_seq_release needs a paged KV cache (page_size > 0)");
  Q2_CHECK(slot >= 0 && slot < m->cfg.max_batch, Q2_ESHAPE, "slot %d not in [0, %d)", slot, m->cfg.max_batch);
  return paged_release(m, slot, static_cast<hipStream_t>(stream));
}

extern "C" q2_status q2_model_seq_length(const q2_model* m, int32_t slot, int32_t* len) {
  clear_error();
  Q2_CHECK(m && len, Q2_EINVAL, "null argument");
  Q2_CHECK(slot >= 0 && slot < m->cfg.max_batch, Q2_ESHAPE, "slot %d not in [0, %d)", slot, m->cfg.max_batch);
  *len = m->page > 0 ? m->h_lens[slot] : m->len;
  return Q2_OK;
}

extern "C" q2_status q2_model_free_pages(const q2_model* m, int32_t* pages) {
  clear_error();
  Q2_CHECK(m && pages, Q2_EINVAL, "null argument");
  Q2_CHECK(m->page > 0, Q2_ESTATE, "the KV cache is not paged");
  *pages = static_cast<int32_t>(m->free_pages.size());
  return Q2_OK;
}

extern "C" q2_status q2_model_prefill_embeds(q2_model* m, const q2_tensor* embeds, const q2_tensor* next,
                                             const q2_tensor* logits, void* stream) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  Q2_TRY(check_desc(embeds, "embeds"));
  Q2_CHECK(embeds->dtype == m->cfg.dtype, Q2_EDTYPE, "embeds must have the model dtype");
  Q2_CHECK(embeds->ndim == 3 && embeds->shape[2] == m->cfg.hidden, Q2_ESHAPE, "embeds must be [B, T, H]");
  Q2_CHECK(embeds->stride[2] == 1, Q2_ESTRIDE, "embeds rows must be contiguous");
  const int B = static_cast<int>(embeds->shape[0]);
  const int Tn = static_cast<int>(embeds->shape[1]);
  Q2_CHECK(Tn >= 1, Q2_ESHAPE, "prefill needs at least one token");
  Q2_TRY(check_batch(m, B, Tn));
  int64_t ns = 0;
  Q2_TRY(check_next(next, B, &ns));
  Rows lg{};
  Q2_TRY(check_logits(m, logits, B, &lg));
  hipStream_t s = static_cast<hipStream_t>(stream);
  Q2_TRY(sync_len(m, s));
  m->cur_batch = B;
  int64_t* np = next ? static_cast<int64_t*>(next->data) : nullptr;
  float* lp = logits ? reinterpret_cast<float*>(lg.data) : nullptr;
  if (m->cfg.dtype == Q2_BF16)
    return prefill_impl<uint16_t>(m, nullptr, 0, 0, B, Tn, lp, lg.ld, np, ns, s,
                                  static_cast<const uint16_t*>(embeds->data), embeds->stride[0], embeds->stride[1]);
  return prefill_impl<float>(m, nullptr, 0, 0, B, Tn, lp, lg.ld, np, ns, s, static_cast<const float*>(embeds->data),
                             embeds->stride[0], embeds->stride[1]);
}

extern "C" q2_status q2_model_hidden_view(q2_model* m, q2_tensor* x) {
  clear_error();
  Q2_CHECK(m && x, Q2_EINVAL, "null argument");
  memset(x, 0, sizeof *x);
  x->data = m->xcur;
  x->dtype = m->cfg.dtype;
  x->ndim = 2;
  x->shape[0] = m->last_rows;
  x->shape[1] = m->cfg.hidden;
  x->stride[0] = m->cfg.hidden;
  x->stride[1] = 1;
  return Q2_OK;
}

extern "C" q2_status q2_model_decode(q2_model* m, const q2_tensor* ids, const q2_tensor* next,
                                     const q2_tensor* logits, void* stream) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  Q2_TRY(check_desc(ids, "ids"));
  Q2_CHECK(ids->dtype == Q2_I64, Q2_EDTYPE, "ids must be int64");
  Q2_CHECK(ids->ndim == 1 || (ids->ndim == 2 && ids->shape[1] == 1), Q2_ESHAPE, "ids must be [B] or [B, 1]");
  const int B = static_cast<int>(ids->shape[0]);
  if (!m->page) Q2_TRY(check_batch(m, B, 1));
  int64_t ns = 0;
  Q2_TRY(check_next(next, B, &ns));
  Rows lg{};
  Q2_TRY(check_logits(m, logits, B, &lg));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool pers = use_persistent(m, B);
  hipGraphExec_t g = nullptr;
  if (!pers) Q2_TRY(get_graph(m, B, logits != nullptr, &g));
  if (m->page)
    Q2_TRY(paged_begin(m, 0, B, 1, false, 1, s));
  else
    Q2_TRY(sync_len(m, s));
  m->cur_batch = B;
  hipLaunchKernelGGL(copy_ids_kernel, dim3(1), dim3(64), 0, s, m->ids_buf, int64_t(1),
                     static_cast<const int64_t*>(ids->data), ids->stride[0], B);
  Q2_TRY(check_launch("copy_ids"));
  if (pers)
    Q2_TRY(persistent_step(m, B, logits != nullptr, s));
  else
    Q2_HIP(hipGraphLaunch(g, s));
  if (m->page)
    paged_end(m, 0, B, 1);
  else
    m->len += 1;
  m->last_rows = B;
  if (next) {
    hipLaunchKernelGGL(copy_ids_kernel, dim3(1), dim3(64), 0, s, static_cast<int64_t*>(next->data), ns, m->ids_buf,
                       int64_t(1), B);
    Q2_TRY(check_launch("copy_next"));
  }
  if (logits) {
    const int64_t n = int64_t(B) * m->cfg.vocab;
    hipLaunchKernelGGL(copy_logits_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, reinterpret_cast<float*>(lg.data),
                       lg.ld, m->logits_buf, m->cfg.vocab, m->cfg.vocab, B);
    Q2_TRY(check_launch("copy_logits"));
  }
  return Q2_OK;
}

static q2_status run_steps(q2_model* m, int steps, const q2_tensor* out_ids, int first_col, hipStream_t s) {
  const int B = m->cur_batch;
  const bool pers = use_persistent(m, B);
  hipGraphExec_t g = nullptr;
  if (steps > 0 && !pers) Q2_TRY(get_graph(m, B, false, &g));
  if (m->page && steps > 0) Q2_TRY(paged_begin(m, 0, B, steps, false, 1, s));
  const int start = m->len;  // the token produced last sits at position `start`
  for (int i = 0; i < steps; ++i) {
    if (pers)
      Q2_TRY(persistent_step(m, B, false, s));
    else
      Q2_HIP(hipGraphLaunch(g, s));
  }
  if (m->page)
    paged_end(m, 0, B, steps);
  else
    m->len += steps;
  if (steps > 0) m->last_rows = B;
  if (out_ids) {
    const int n = static_cast<int>(out_ids->shape[1]);
    hipLaunchKernelGGL(copy_hist_kernel, dim3(cdiv(int64_t(n) * B, 256)), dim3(256), 0, s,
                       static_cast<int64_t*>(out_ids->data), out_ids->stride[0], m->hist,
                       static_cast<int64_t>(m->cfg.max_seq) + 1, start + 1 - first_col, n, B,
                       m->page > 0 ? m->d_lens : nullptr, steps - 1 + first_col);
    Q2_TRY(check_launch("copy_hist"));
  }
  return Q2_OK;
}

static q2_status check_out_ids(const q2_tensor* out_ids, int B, int cols) {
  Q2_TRY(check_desc(out_ids, "out_ids"));
  Q2_CHECK(out_ids->dtype == Q2_I64, Q2_EDTYPE, "out_ids must be int64");
  Q2_CHECK(out_ids->ndim == 2 && out_ids->shape[0] == B && out_ids->shape[1] == cols, Q2_ESHAPE,
           "out_ids must be [%d, %d]", B, cols);
  Q2_CHECK(out_ids->stride[1] == 1 || cols <= 1, Q2_ESTRIDE, "out_ids rows must be contiguous");
  return Q2_OK;
}

extern "C" q2_status q2_model_generate(q2_model* m, const q2_tensor* prompt, int32_t steps, const q2_tensor* out_ids,
                                       void* stream) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  Q2_CHECK(steps >= 0, Q2_EINVAL, "steps must be >= 0");
  int B = 0, Tn = 0;
  int64_t bs = 0, ts = 0;
  Q2_TRY(check_ids_2d(prompt, &B, &Tn, &bs, &ts));
  Q2_CHECK(Tn >= 1, Q2_ESHAPE, "prompt needs at least one token");
  if (!m->page) Q2_TRY(check_batch(m, B, Tn + steps));
  Q2_TRY(check_out_ids(out_ids, B, steps + 1));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (steps > 0 && !use_persistent(m, B)) {
    hipGraphExec_t g = nullptr;
    Q2_TRY(get_graph(m, B, false, &g));  // capture before any state changes
  }
  if (m->page) {
    for (int b = 0; b < B; ++b)
      Q2_CHECK(static_cast<int64_t>(m->h_lens[b]) + Tn + steps <= m->cfg.max_seq, Q2_ESTATE,
               "sequence %d: capacity exceeded", b);
    Q2_TRY(paged_begin(m, 0, B, Tn, true, 0, s));
  } else {
    Q2_TRY(sync_len(m, s));
  }
  m->cur_batch = B;
  const int64_t* ip = static_cast<const int64_t*>(prompt->data);
  const q2_status st = m->cfg.dtype == Q2_BF16
                           ? prefill_impl<uint16_t>(m, ip, bs, ts, B, Tn, nullptr, 0, nullptr, 0, s)
                           : prefill_impl<float>(m, ip, bs, ts, B, Tn, nullptr, 0, nullptr, 0, s);
  if (m->page) paged_end(m, 0, B, Tn);
  Q2_TRY(st);
  // out column 0 is the prefill's token (position len), then one per step
  return run_steps(m, steps, out_ids, 1, s);
}

extern "C" q2_status q2_model_continue(q2_model* m, int32_t steps, const q2_tensor* out_ids, void* stream) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  Q2_CHECK(steps >= 0, Q2_EINVAL, "steps must be >= 0");
  Q2_CHECK(m->len >= 1 && m->cur_batch >= 1, Q2_ESTATE, "continue needs a prefill first");
  if (!m->page) Q2_TRY(check_batch(m, m->cur_batch, steps));
  if (out_ids) Q2_TRY(check_out_ids(out_ids, m->cur_batch, steps));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!m->page) Q2_TRY(sync_len(m, s));
  return run_steps(m, steps, out_ids, 0, s);
}

extern "C" q2_status q2_model_kv_view(q2_model* m, int32_t layer, q2_tensor* k, q2_tensor* v) {
  clear_error();
  Q2_CHECK(m && k && v, Q2_EINVAL, "null argument");
  Q2_CHECK(layer >= 0 && layer < m->cfg.nlayer, Q2_EINVAL, "layer out of range");
  Q2_CHECK(m->page == 0, Q2_ESTATE, "a paged KV cache has no per-sequence view");
  for (int i = 0; i < 2; ++i) {
    q2_tensor* t = i ? v : k;
    memset(t, 0, sizeof *t);
    t->data = static_cast<char*>(i ? m->vc : m->kc) + int64_t(layer) * m->kv_lstride * (m->fp8 ? 1 : m->esize);
    t->dtype = m->fp8 ? Q2_U8 : m->cfg.dtype;
    t->ndim = 4;
    t->shape[0] = m->cfg.max_batch;
    t->shape[1] = m->cfg.max_seq;
    t->shape[2] = m->cfg.nkv;
    t->shape[3] = m->cfg.dh;
    t->stride[0] = m->kv_bstride;
    t->stride[1] = m->cfg.dh;
    t->stride[2] = m->kv_hstride;
    t->stride[3] = 1;
  }
  return Q2_OK;
}

extern "C" q2_status q2_model_replay_stage(q2_model* m, int32_t stage, int32_t batch, int32_t tokens, int32_t reps,
                                          void* stream) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  Q2_CHECK(stage >= STAGE_QKV && stage <= STAGE_ATTN_CORE, Q2_EINVAL, "stage %d not in [0, 5]", stage);
  Q2_CHECK(batch >= 1 && batch <= m->cfg.max_batch, Q2_ESHAPE, "batch %d not in [1, %d]", batch, m->cfg.max_batch);
  Q2_CHECK(tokens >= 1 && reps >= 0, Q2_ESHAPE, "tokens must be positive and reps non-negative");
  Q2_CHECK(int64_t(batch) * tokens <= m->max_tok, Q2_ESHAPE, "%d x %d rows exceed the activation arena (%d)", batch,
           tokens, m->max_tok);
  const int len_now = m->page > 0 ? m->h_lens[0] : m->len;
  Q2_CHECK(static_cast<int64_t>(len_now) + tokens <= m->cfg.max_seq, Q2_ESTATE,
           "replay at length %d + %d tokens exceeds the cache (%d)", len_now, tokens, m->cfg.max_seq);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m->page > 0) {
    // the replayed positions len .. len + tokens - 1 of every replayed
    // sequence need their pages (the products write and read them); the
    // lengths themselves do not move
    for (int b = 0; b < batch; ++b)
      Q2_CHECK(m->h_lens[b] == m->h_lens[0], Q2_ESTATE, "replay needs sequences of equal length");
    Q2_TRY(paged_reserve(m, 0, batch, tokens, s));
    m->slot0 = 0;
    m->len = m->h_lens[0];
    m->len_dirty = true;
  }
  Q2_TRY(sync_len(m, s));
  for (int i = 0; i < reps; ++i) {
    const int l = i % m->cfg.nlayer;
    Q2_TRY(m->cfg.dtype == Q2_BF16 ? run_layers<uint16_t>(m, batch, tokens, false, s, stage, l)
                                   : run_layers<float>(m, batch, tokens, false, s, stage, l));
  }
  return Q2_OK;
}

extern "C" q2_status q2_model_kv_scale_view(q2_model* m, int32_t layer, q2_tensor* ks, q2_tensor* vs) {
  clear_error();
  Q2_CHECK(m && ks && vs, Q2_EINVAL, "null argument");
  Q2_CHECK(m->fp8 && m->page == 0, Q2_ESTATE, "the model's KV cache is not a contiguous FP8 cache");
  Q2_CHECK(layer >= 0 && layer < m->cfg.nlayer, Q2_EINVAL, "layer out of range");
  const KvLayout f = cache_layout(m, layer);
  for (int i = 0; i < 2; ++i) {
    q2_tensor* t = i ? vs : ks;
    memset(t, 0, sizeof *t);
    t->data = i ? f.vs : f.ks;
    t->dtype = Q2_F32;
    t->ndim = 3;
    t->shape[0] = m->cfg.max_batch;
    t->shape[1] = m->cfg.max_seq;
    t->shape[2] = m->cfg.nkv;
    t->stride[0] = f.bs;
    t->stride[1] = 1;
    t->stride[2] = f.hs;
  }
  return Q2_OK;
}

extern "C" q2_status q2_model_length(const q2_model* m, int32_t* len) {
  clear_error();
  Q2_CHECK(m && len, Q2_EINVAL, "null argument");
  *len = m->page > 0 ? m->h_lens[0] : m->len;
  return Q2_OK;
}

extern "C" q2_status q2_model_reset(q2_model* m) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  if (m->page > 0)
    for (int b = 0; b < m->cfg.max_batch; ++b) Q2_TRY(paged_release(m, b, nullptr));
  m->len = 0;
  m->cur_batch = 0;
  m->len_dirty = true;
  return Q2_OK;
}

extern "C" q2_status q2_model_set_decode_path(q2_model* m, int32_t persistent) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  Q2_CHECK(persistent == 0 || persistent == 1, Q2_EINVAL, "persistent must be 0 or 1");
  m->mk_on = persistent == 1;
  return Q2_OK;
}

extern "C" q2_status q2_model_decode_path(const q2_model* m, int32_t batch, int32_t* persistent) {
  clear_error();
  Q2_CHECK(m && persistent, Q2_EINVAL, "null argument");
  *persistent = use_persistent(m, batch) ? 1 : 0;
  return Q2_OK;
}

extern "C" q2_status q2_model_check(q2_model* m) {
  clear_error();
  Q2_CHECK(m, Q2_EINVAL, "null model");
  Q2_HIP(hipSetDevice(m->device));
  Q2_HIP(hipDeviceSynchronize());
  if (m->mk_ok) {
    unsigned err = 0;
    Q2_HIP(hipMemcpy(&err, m->mk.err, sizeof err, hipMemcpyDeviceToHost));
    Q2_CHECK(err == 0, Q2_EHIP, "a grid barrier of the persistent decode step timed out");
  }
  if (m->skws) {
    unsigned err = 0;
    Q2_HIP(hipMemcpy(&err, static_cast<char*>(m->skws) + stream_k_err_offset(), sizeof err, hipMemcpyDeviceToHost));
    Q2_CHECK(err == 0, Q2_EHIP, "a stream-K hand-over wait of a prefill product timed out");
  }
  return Q2_OK;
}

extern "C" void q2_model_destroy(q2_model* m) {
  if (!m) return;
  (void)hipSetDevice(m->device);
  (void)hipDeviceSynchronize();
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  if (m->cap) (void)hipStreamDestroy(m->cap);
  if (m->mkmem) (void)hipFree(m->mkmem);
  if (m->wmem) (void)hipFree(m->wmem);
  if (m->kvmem) (void)hipFree(m->kvmem);
  if (m->amem) (void)hipFree(m->amem);
  delete m;
}
