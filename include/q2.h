/*
 * q2.h -- C ABI of a Qwen2 decoder forward for AMD Instinct MI355X (gfx950).
 *
 * The library exports one call per operator of the decoder and a model driver
 * that owns the weights, the activation buffers and the KV cache.  The
 * operator set follows "LLAISYS 训练营结项报告" (section 3.2, third layer:
 * add, argmax, embedding, linear, rms_norm, rope, self_attention, swiglu,
 * rearrange) and the model follows its fourth layer (weights, intermediate
 * buffers and KV cache resident on the device, KV cache written with
 * rearrange).  Every operator is a hand-written HIP kernel.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are passed as q2_tensor descriptors: a device pointer, a dtype,
 *    the rank and per-dimension sizes and strides (in elements, not bytes).
 *    The caller owns every tensor.  Operator calls never allocate, free or
 *    synchronise: memory beyond their inputs and outputs (split partial
 *    results) comes from a caller-owned `workspace` argument, so an operator
 *    call can be captured into a HIP graph.  Only q2_model_create and
 *    q2_model_destroy allocate and free (the model's own memory).
 *  - Unless a call says otherwise the last dimension must have stride 1 and
 *    the outer dimensions may have any non-negative strides.
 *  - Arithmetic is float32 whatever the storage type ("low precision storage,
 *    float compute, low precision write-back", section 3.3 item 3 of the same
 *    report).  bf16 results are rounded to nearest, ties to even.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call is
 *    asynchronous on that stream; the caller synchronises.
 *  - Every call returns a q2_status.  Arguments are validated on the host
 *    before anything is launched; a call that fails validation launches
 *    nothing and leaves its outputs untouched.  There is no fallback path:
 *    unsupported shapes, dtypes or strides are errors.  q2_last_error()
 *    returns a message describing the last failure on the calling thread.
 *  - Inputs are assumed finite.  Results for NaN inputs are unspecified.
 */
#ifndef Q2_H
#define Q2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  Q2_OK = 0,
  Q2_EINVAL = -1,  /* null pointer, bad count, bad name */
  Q2_EDTYPE = -2,  /* dtype not supported by the call or mismatched */
  Q2_ESHAPE = -3,  /* sizes inconsistent with each other or with the model */
  Q2_ESTRIDE = -4, /* layout not supported (e.g. last dim not contiguous) */
  Q2_ENOMEM = -5,  /* device allocation failed (model creation only) */
  Q2_EHIP = -6,    /* a HIP runtime call failed; see q2_last_error() */
  Q2_ESTATE = -7   /* model state does not allow the call (capacity, batch) */
} q2_status;

/* Q2_U8: bytes (FP8 KV-cache codes). */
typedef enum { Q2_F32 = 0, Q2_BF16 = 1, Q2_I64 = 2, Q2_U8 = 3 } q2_dtype;

#define Q2_MAX_DIMS 5

typedef struct {
  void* data;                    /* device pointer */
  int32_t dtype;                 /* q2_dtype */
  int32_t ndim;                  /* 1 .. Q2_MAX_DIMS */
  int64_t shape[Q2_MAX_DIMS];
  int64_t stride[Q2_MAX_DIMS];   /* in elements */
} q2_tensor;

/* Message for the last failing call on this thread ("" if none). */
const char* q2_last_error(void);

/* Library version string. */
const char* q2_version(void);

/* ------------------------------------------------------------------------
 * Operators
 * ---------------------------------------------------------------------- */

/* out[n, :] = weight[ids[n], :]  (section 3.2, embedding).
 * ids: [N] int64.  weight: [V, H] f32/bf16.  out: [N, H], same dtype.
 * Bit-exact copy.  Ids outside [0, V) produce a zero row (no fault). */
q2_status q2_embedding(const q2_tensor* out, const q2_tensor* ids, const q2_tensor* weight,
                       void* stream);

/* out = in W^T (+ bias)  (section 3.2, linear; bias optional).
 * in: [M, K] or [B, T, K] (flattened to M rows); weight: [N, K] row-major
 * ([out features, in features]); bias: [N] or NULL; out: [M, N] / [B, T, N].
 * dtype: all f32, or in/weight/bias bf16 with out bf16 or f32.  bf16 path:
 * MFMA with float32 accumulation; K must be a multiple of 8 and rows and
 * pointers 16-byte aligned.  Rows of `in` and `out` may be strided.
 * workspace: NULL or a contiguous, 16-byte aligned tensor of any dtype whose
 * bytes the call may overwrite (it must not overlap the operands).  Products
 * of at most 64 rows split K over workgroups when the workspace holds the
 * float32 partial sums (q2_linear_workspace_bytes); with a smaller or no
 * workspace they run unsplit (slower on small N; the sums are then added in
 * another order, so results can differ by float32 rounding).  Calls that
 * share a workspace must be ordered (same stream). */
q2_status q2_linear(const q2_tensor* out, const q2_tensor* in, const q2_tensor* weight,
                    const q2_tensor* bias, const q2_tensor* workspace, void* stream);

/* Workspace bytes q2_linear needs to run its split plan for M rows, N out
 * features, K in features of dtype Q2_F32 / Q2_BF16 (0: it never splits). */
q2_status q2_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t dtype, size_t* bytes);

/* Bytes of the fixed device scratch of q2_linear_noalloc (per GPU). */
#define Q2_LINEAR_NOALLOC_SCRATCH_BYTES (16u << 20)

/* q2_linear for callers that cannot allocate or pass a workspace (code under
 * HIP graph capture, tight serving loops, harnesses that forbid device
 * allocation): the same operation, operands, layout and plan as q2_linear
 * with a large enough workspace, but the split-K partials live in a fixed
 * Q2_LINEAR_NOALLOC_SCRATCH_BYTES array inside the library, one per GPU,
 * held until the process ends.  Calls no allocating routine.  Products whose
 * partials would exceed that size fail with Q2_ESHAPE (nothing launched).
 * Every call on one GPU shares that GPU's array: calls that can overlap on
 * one GPU (different streams, or different host threads) race and must be
 * ordered by the caller.  The array is looked up on the first call on each
 * GPU. */
q2_status q2_linear_noalloc(const q2_tensor* out, const q2_tensor* in, const q2_tensor* weight,
                            const q2_tensor* bias, void* stream);

/* out = in / sqrt(mean(in^2) + eps) * weight over the last dimension
 * (section 3.2, rms_norm; epsilon inside the root).  in/out: [..., H];
 * weight: [H]; all the same dtype (f32 or bf16).  The output is rounded once. */
q2_status q2_rms_norm(const q2_tensor* out, const q2_tensor* in, const q2_tensor* weight,
                      float eps, void* stream);

/* Rotary position embedding, rotate-half pairing (section 3.2, rope):
 * for j < d/2, a = in[t,h,j], b = in[t,h,j+d/2], angle = pos[t] * theta^(-2j/d),
 * out[t,h,j] = a cos - b sin, out[t,h,j+d/2] = b cos + a sin.
 * in/out: [T, nh, d] (or [B, T, nh, d] with pos [B, T] or [T]); pos int64.
 * cos/sin are evaluated from a float64 angle and rounded to float32.
 * out may alias in. */
q2_status q2_rope(const q2_tensor* out, const q2_tensor* in, const q2_tensor* pos, float theta,
                  void* stream);

/* Causal grouped-query attention (section 3.2, self_attention; the scaled
 * Q K^T -> causal mask -> stable softmax -> times V sequence of
 * "万亿参数大模型在国产加速卡上的Day-0适配教程", step 5).
 * q: [T, nh, d] or [B, T, nh, d]; k, v: [S, nkv, d] or [B, S, nkv, d] with
 * S >= T; out: same shape as q.  Query t (absolute position S - T + t) sees
 * keys j <= S - T + t.  Query head h reads KV head h / (nh / nkv).
 * scores = (q . k) * scale, softmax in float32.  k and v may be strided views
 * (e.g. of a KV cache laid out [B, nkv, S_max, d]); their last dim must be
 * contiguous.  dtype f32 (any d <= 256) or bf16 (d = 128 only).
 * workspace: NULL or a caller-owned tensor as for q2_linear.  The bf16 path
 * splits long key ranges over workgroups (decode) and the longest query
 * blocks in two (prefill) when the workspace holds their partial results
 * (q2_self_attention_workspace_bytes); otherwise it runs unsplit. */
q2_status q2_self_attention(const q2_tensor* out, const q2_tensor* q, const q2_tensor* k,
                            const q2_tensor* v, float scale, const q2_tensor* workspace, void* stream);

/* Workspace bytes q2_self_attention needs to run its split plan for B
 * sequences of T queries over S keys, nh query / nkv KV heads of size d. */
q2_status q2_self_attention_workspace_bytes(int32_t B, int32_t T, int32_t S, int32_t nh, int32_t nkv, int32_t d,
                                            int32_t dtype, size_t* bytes);

/* out = silu(gate) * up, silu(g) = g / (1 + exp(-g))  (section 3.2, swiglu).
 * Same shape [..., I] and dtype for all three. */
q2_status q2_swiglu(const q2_tensor* out, const q2_tensor* gate, const q2_tensor* up,
                    void* stream);

/* c = a + b element-wise (section 3.2, add).  Same shape and dtype. c may alias a or b. */
q2_status q2_add(const q2_tensor* c, const q2_tensor* a, const q2_tensor* b, void* stream);

/* Row-wise maximum and its index, lowest index on ties (section 3.2 argmax;
 * section 4.3 item 4: the best score travels with its token id).
 * vals: [V] or [B, V] f32/bf16; max_idx: [] / [B] int64 (shape [1] accepted for
 * a single row); max_val: same count, f32.  max_idx is used as the reduction
 * accumulator, so it must not alias vals.  Bit-exact. */
q2_status q2_argmax(const q2_tensor* max_idx, const q2_tensor* max_val, const q2_tensor* vals,
                    void* stream);

/* out[...] = in[...] for two tensors of the same shape and dtype with any
 * strides (section 3.2 rearrange: contiguous fast path plus a general
 * stride-aware copy).  Bit-exact.  Any dtype, up to 5 dims, strides >= 0;
 * overlapping in/out is undefined. */
q2_status q2_rearrange(const q2_tensor* out, const q2_tensor* in, void* stream);

/* FP8 KV-cache codec ("新一代大模型Day0推理适配与性能调优教程", step 5: the KV
 * cache quantised to FP8 per token x per head x block of 128 elements, with
 * high-precision accumulation).  One block = one row of 128 values.
 *   amax = max |x_i|; scale = amax / 448 in float32 (0 for an all-zero row);
 *   code_i = E4M3(x_i / scale): OCP FP8 E4M3 (bias 7, no infinities, max 448),
 *   round to nearest even, magnitude saturated at 448, sign of x_i kept
 *   (so -0 codes as 0x80).
 * q2_kv_quantize: x [N, 128] bf16 -> codes [N, 128] u8, scales [N] f32.
 * q2_kv_dequantize: x_i = bf16(value(code_i) * scale) (float32 product, then
 * round to nearest even).  Rows 16-byte aligned; scales contiguous.  Codes
 * and dequantised values are bit-exact functions of their inputs. */
q2_status q2_kv_quantize(const q2_tensor* codes, const q2_tensor* scales, const q2_tensor* x, void* stream);
q2_status q2_kv_dequantize(const q2_tensor* x, const q2_tensor* codes, const q2_tensor* scales, void* stream);

/* ------------------------------------------------------------------------
 * Model driver (section 3.2, fourth layer; section 3.3 item 4: per-device
 * handles and intermediate buffers are created once and reused).
 * ---------------------------------------------------------------------- */

typedef struct q2_model q2_model;

typedef struct {
  int32_t dtype;        /* Q2_F32 or Q2_BF16 (weights, activations, KV cache) */
  int32_t nlayer;
  int32_t hidden;       /* H */
  int32_t nh;           /* query heads */
  int32_t nkv;          /* key/value heads, divides nh */
  int32_t dh;           /* head dim (bf16: 128; f32: even, <= 256) */
  int32_t inter;        /* SwiGLU intermediate size */
  int32_t vocab;
  int32_t max_seq;      /* KV-cache capacity per sequence */
  int32_t max_batch;    /* sequences per call, at most */
  float eps;            /* RMSNorm epsilon */
  float theta;          /* RoPE base */
  int32_t kv_fp8;       /* 0: KV cache in the model dtype; 1 (bf16 models): FP8
                           E4M3 codes with one float32 scale per token, KV head
                           and 128-element block ("新一代大模型Day0推理适配与性能调优
                           教程", step 5), see q2_kv_quantize */
  int32_t page_size;    /* 0: each sequence owns a contiguous [max_seq] cache
                           region; > 0 (bf16 models, a multiple of 64): the
                           cache is a pool of pages of page_size positions,
                           taken as sequences grow and given back when they
                           are released ("万亿参数大模型在国产加速卡上的Day-0适配
                           教程", step 8: paged KV cache, continuous batching);
                           sequences may then have different lengths */
  int32_t kv_pages;     /* paged: pages in the pool (0: max_batch * ceil(max_seq
                           / page_size), room for every sequence at max_seq) */
} q2_config;

/* Create a model on `device`: allocates the packed weights, the KV cache
 * (K and V each [nlayer][max_batch][nkv][max_seq][dh]), the RoPE cos/sin
 * table and the activation arena, sized for max_batch x max_seq.  Weights
 * start zeroed.  Returns Q2_ENOMEM if the device cannot hold it. */
q2_status q2_model_create(const q2_config* cfg, int32_t device, q2_model** out);

/* Bytes of device memory the model holds. */
q2_status q2_model_device_bytes(const q2_model* m, size_t* bytes);

/* Copy one weight tensor (device memory, the model's dtype, contiguous) into
 * the model's packed layout.  Names and shapes (Hugging Face Qwen2 naming,
 * layer = -1 for the global tensors):
 *   embed_tokens [V,H], lm_head [V,H], norm [H]                  (layer -1)
 *   input_layernorm [H], post_attention_layernorm [H],
 *   q_proj.weight [nh*d,H], q_proj.bias [nh*d], k_proj.weight [nkv*d,H],
 *   k_proj.bias [nkv*d], v_proj.weight [nkv*d,H], v_proj.bias [nkv*d],
 *   o_proj.weight [H,nh*d], gate_proj.weight [I,H], up_proj.weight [I,H],
 *   down_proj.weight [H,I]                                      (layer 0..L-1)
 * The source may be freed once the stream has passed this call. */
q2_status q2_model_load_weight(q2_model* m, const char* name, int32_t layer, const q2_tensor* src,
                               void* stream);

/* Run ids [B, T] (int64) at positions len .. len+T-1 of every sequence, where
 * len is the current cached length (0 after create/reset), then len += T.
 * next: [B] int64 greedy tokens of the last position.  logits: NULL or
 * [B, V] f32 (last position).  B must not exceed max_batch and must equal
 * the batch of earlier calls since the last reset; len + T must not exceed
 * max_seq (else Q2_ESTATE and nothing changes).  Ids are not range-checked
 * on the host (they are device data): an id outside [0, vocab) embeds as a
 * zero row, as in q2_embedding. */
q2_status q2_model_prefill(q2_model* m, const q2_tensor* ids, const q2_tensor* next,
                           const q2_tensor* logits, void* stream);

/* Same as q2_model_prefill, but the first layer reads the hidden states
 * `embeds` [B, T, H] (model dtype, rows contiguous) instead of looking token
 * ids up in embed_tokens.  Used to check the layer stack on given inputs
 * (layer-by-layer comparison) and for callers that bring their own embeddings. */
q2_status q2_model_prefill_embeds(q2_model* m, const q2_tensor* embeds, const q2_tensor* next,
                                  const q2_tensor* logits, void* stream);

/* Describe the residual stream (the hidden states after the last layer, before
 * the final norm) of the last prefill chunk or decode step: [rows, H] in the
 * model dtype, row b * T + t for sequence b and token t of that chunk.  Valid
 * until the next call on the model. */
q2_status q2_model_hidden_view(q2_model* m, q2_tensor* x);

/* Paged cache only (page_size > 0): sequences of different lengths
 * ("万亿参数大模型在国产加速卡上的Day-0适配教程", step 8: paged KV cache and
 * continuous batching, new requests joining a running batch).
 * q2_model_seq_prefill: run ids [T] int64 for sequence `slot` at its
 * positions len_slot .. len_slot + T - 1 (len_slot = 0 for a new or released
 * slot), taking pages as needed; next: [1] or NULL, logits: [1, V] f32 or
 * NULL.  Q2_ESTATE (nothing changed) if the pool has too few free pages or
 * max_seq would be exceeded.
 * q2_model_decode / q2_model_continue then step slots 0 .. B - 1 together,
 * each at its own length (every one of them must hold at least one
 * position).  q2_model_prefill still takes B sequences of equal length.
 * q2_model_seq_release: the slot's pages return to the pool and its length
 * to 0 (asynchronous on `stream`; no step using the slot may still be
 * pending).  q2_model_seq_length: positions cached for `slot`.
 * q2_model_free_pages: pages left in the pool. */
q2_status q2_model_seq_prefill(q2_model* m, int32_t slot, const q2_tensor* ids, const q2_tensor* next,
                               const q2_tensor* logits, void* stream);
q2_status q2_model_seq_release(q2_model* m, int32_t slot, void* stream);
q2_status q2_model_seq_length(const q2_model* m, int32_t slot, int32_t* len);
q2_status q2_model_free_pages(const q2_model* m, int32_t* pages);

/* One decode step: ids [B] int64 at position len; same outputs as prefill.
 * Replays a HIP graph captured once per batch size. */
q2_status q2_model_decode(q2_model* m, const q2_tensor* ids, const q2_tensor* next,
                          const q2_tensor* logits, void* stream);

/* Greedy generation: prefill prompt [B, T], then `steps` decode steps fed
 * on the device with the previous step's argmax.  out_ids: [B, steps + 1]
 * int64; column 0 is the prefill's token, column s the token of decode step s.
 * Needs len + T + steps <= max_seq. */
q2_status q2_model_generate(q2_model* m, const q2_tensor* prompt, int32_t steps,
                            const q2_tensor* out_ids, void* stream);

/* Continue greedy generation from the current state: `steps` decode steps,
 * each fed on the device with the previous step's token (the token the last
 * prefill, decode or continue call produced).  out_ids: NULL or [B, steps]
 * int64, column s - 1 holding the token of step s.  Needs len >= 1 and
 * len + steps <= max_seq. */
q2_status q2_model_continue(q2_model* m, int32_t steps, const q2_tensor* out_ids, void* stream);

/* Describe layer `layer`'s cache as tensors k, v of shape
 * [max_batch, max_seq, nkv, dh] (strided views of the [B][nkv][S][d] layout;
 * Q2_U8 codes for an FP8 cache). */
q2_status q2_model_kv_view(q2_model* m, int32_t layer, q2_tensor* k, q2_tensor* v);

/* FP8 cache only: layer `layer`'s scales as f32 tensors [max_batch, max_seq,
 * nkv] (Q2_ESTATE for a cache in the model dtype). */
q2_status q2_model_kv_scale_view(q2_model* m, int32_t layer, q2_tensor* k_scale, q2_tensor* v_scale);

/* Measurement hook: launch, `reps` times on `stream`, the kernels of one
 * product of a forward of `batch` sequences x `tokens` new tokens at the
 * current cached length, for layers 0, 1, ..., nlayer - 1, 0, ... in turn:
 * stage 0 QKV (with its fused norm and cache write), 1 attention, 2 o_proj,
 * 3 gate/up, 4 down, 5 the decode attention kernel alone (its split-KV
 * partials left unmerged, where stage 1 also launches the merge when the
 * forward does; for more than one token, as stage 1).
 * The kernels and arguments are those the forward (or
 * the captured decode step) launches, reading the model's own weights and
 * buffers.  The activations, the residual stream and the cache rows at the
 * replayed positions are left undefined: reset before the next forward.
 * Needs batch * tokens within the activation arena and len + tokens <=
 * max_seq. */
q2_status q2_model_replay_stage(q2_model* m, int32_t stage, int32_t batch, int32_t tokens, int32_t reps,
                                void* stream);

/* Cached length (positions per sequence). */
q2_status q2_model_length(const q2_model* m, int32_t* len);

/* Forget the cached sequences (len = 0).  Does not touch device memory. */
q2_status q2_model_reset(q2_model* m);

/* Decode path for steps of up to 16 sequences of a bf16 model: 1 runs each
 * step as one persistent cooperative kernel (one workgroup per CU, grid
 * barriers between the fused stages); 0 (default) replays the graph of
 * per-operator kernels.  Both compute the same operator chain with the same
 * rounding points; summation order inside the products differs.  Larger
 * batches and the float32 model always use the per-operator path.
 * Q2_EINVAL for other values. */
q2_status q2_model_set_decode_path(q2_model* m, int32_t persistent);

/* Which path a decode step of `batch` sequences would take now (1 =
 * persistent kernel). */
q2_status q2_model_decode_path(const q2_model* m, int32_t batch, int32_t* persistent);

/* Synchronises the device and reports failures recorded on it by earlier
 * asynchronous calls: Q2_EHIP if a grid barrier of the persistent decode
 * kernel timed out, or if a prefill product whose tiles are shared between
 * two workgroups (stream-K: long-K products with fewer tiles than CUs)
 * waited past its bound for the other workgroup's partial tile -- which
 * happens only if the device could not hold all of that launch's
 * workgroups at once.  The affected results are then invalid. */
q2_status q2_model_check(q2_model* m);


/* Free everything the model holds.  Synchronises the device first. */
void q2_model_destroy(q2_model* m);

#ifdef __cplusplus
}
#endif
#endif /* Q2_H */
