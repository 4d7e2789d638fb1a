// Persistent decode step (decode_mk.hip): arguments and host entry points.
#pragma once

#include "epilogue.hpp"

namespace q2 {

constexpr int MK_THREADS = 512;   // 8 waves per workgroup, one workgroup per CU
constexpr int MK_MAX_BATCH = 16;
constexpr int MK_ATT_SPLITS = 8;  // key chunks per (sequence, KV head) at most
constexpr int MK_DOWN_SPLITS = 2; // K splits of the down projection at most
constexpr int MK_NORM_CHUNKS = 4; // 16-byte chunks of a row per lane in the norm prologue at most

// Per-layer device pointers (packed weights as the model loader lays them out).
struct MkLayer {
  const uint16_t *w_in, *w_post, *w_qkv, *b_qkv, *w_o, *w_gu, *w_d;
  uint16_t *kc, *vc;  // this layer's K and V cache, [B_max][nkv][S_max][128]
};

struct MkArgs {
  const MkLayer* layers;  // device array [L]
  int L, H, nh, nkv, I, V, B;
  float eps, scale;
  const uint16_t* embed;
  const uint16_t* w_final;
  const uint16_t* lm_head;
  int64_t kv_bstride, kv_hstride;
  const float2* rope;     // [S_max][64] (cos, sin)
  int* d_len;             // cached length = position of the new token; advanced by one
  int64_t* ids_buf;       // [B] input token of the step; overwritten with the output
  int64_t* hist;          // [B][hist_ld] output history (token of position p at p)
  int64_t hist_ld;
  unsigned long long* keys;  // argmax key slots [B][KEY_ROW], zero on entry and on exit
  float* logits;          // optional [B][V]
  // activations, each written once per step before it is read
  uint16_t* xres;         // [L+1][B][H] residual entering each layer (and the final norm)
  uint16_t* xmid;         // [L][B][H] residual after attention
  uint16_t* qbuf;         // [L][B][nh*128] rotated queries
  uint16_t* act;          // [L][B][I] SwiGLU output
  float* att_o;           // [L][B][nkv][att_nsplit_max][16][128] attention partial outputs
  float2* att_ml;         // [L][B][nkv][att_nsplit_max][16] (running max, running sum)
                          // att_nsplit_max = MK_ATT_SPLITS
  float* down_part;       // [L][down_splits][B][H] split-K partials of the down projection
  int att_nsplit_max;
  int down_splits, down_bps;
  // grid barrier
  unsigned* bar_flags;    // [grid]
  unsigned* bar_release;  // [grid][32] (one 128-byte line per workgroup)
  unsigned epoch0;        // barrier epoch before this launch
  unsigned* err;          // set when a barrier wait timed out
  int lds_x_bytes;        // LDS bytes of the staged-X / V^T region
};

// LDS the kernel needs for batch B, hidden H and nh*128 = QD.
size_t mk_lds_bytes(int B, int H, int QD);
size_t mk_lds_x_bytes(int B, int H, int QD);
// Grid barriers one step performs (the host advances epoch0 by this much).
int mk_barriers(int L);
// Cooperative grid size that keeps every workgroup resident (0: not possible).
q2_status mk_max_grid(int B, int H, int QD, int* grid);
q2_status mk_launch(const MkArgs& a, int grid, hipStream_t s);

}  // namespace q2
