// Causal grouped-query attention kernels (attention.hip).
#pragma once

#include "common.hpp"
#include "kvcache.hpp"

namespace q2 {

// Strides are in elements; the head dimension is contiguous everywhere.
// Sequence b, query t, head h:     q + b*q_bs + t*q_ts + h*q_hs
// Sequence b, key j, kv head g:    k + b*k_bs + j*k_ss + g*k_hs   (same for v)
// Query t sits at absolute position S - T + t and sees keys j <= S - T + t.
// When d_len is set, S = *d_len + T is read on the device (graph replay);
// s_max bounds it and sizes the split-KV grid.
struct AttnArgs {
  const void* q;
  int64_t q_bs, q_ts, q_hs;
  const void* k;
  int64_t k_bs, k_ss, k_hs;
  const void* v;
  int64_t v_bs, v_ss, v_hs;
  void* o;
  int64_t o_bs, o_ts, o_hs;
  int B, T, S, nh, nkv, d;
  float scale;
  const int* d_len;
  int s_max;
  void* scratch;               // split-KV partials
  size_t scratch_bytes;
  bool leave_partials;         // split-KV: skip the merge, the consumer merges the partials
  bool unsplit_if_short;       // run unsplit when the partials exceed scratch_bytes (else fail)
  // decode path only: K / V are rows of the model's cache (bf16 or FP8,
  // contiguous or paged, kvcache.hpp) instead of the strided k / v above
  bool use_cache;
  KvLayout cache;
  // per-sequence cached lengths (S_b = lens[b] + T; sequences of different
  // lengths), or null
  const int* lens;
};

q2_status attention_bf16(const AttnArgs& a, hipStream_t s);
q2_status attention_f32(const AttnArgs& a, hipStream_t s);
// Scratch (bytes) the bf16 split-KV decode path needs for these sizes.
size_t attention_scratch_bytes(int B, int T, int s_max, int nh, int nkv, int d);
// Number of key chunks the bf16 decode kernel splits each (sequence, KV head)
// into for these sizes; 0 when the prefill kernel handles them.  Partials
// live at scratch: float O [B*nkv][nsplit][16][d], then float2 (max, sum)
// [B*nkv][nsplit][16].
int attention_decode_splits(int B, int T, int s_max, int nh, int nkv, int d);

}  // namespace q2
