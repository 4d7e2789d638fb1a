"""Oracle Qwen2 decoder: prefill and single-token greedy decode with a KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer sequence is the standard Qwen2 decoder, which the LLAISYS report
runs and matches against Hugging Face token for token ("LLAISYS 训练营结项报告",
sections 3.2 fourth layer and 3.5):

  x = E[ids]
  per layer:  h = rmsnorm(x, w_in)
              q, k, v = h Wq^T + bq, h Wk^T + bk, h Wv^T + bv
              q, k = rope(q, pos), rope(k, pos);  append k, v to the cache
              o = causal GQA attention(q, K_cache, V_cache)
              x = x + o Wo^T
              h2 = rmsnorm(x, w_post)
              x = x + (silu(h2 Wg^T) * (h2 Wu^T)) Wd^T
  logits = rmsnorm(x_last, w_f) W_lm^T   (float32, last position of each sequence)
  next = argmax(logits)

Storage model ("bf16" mode): every operator output is rounded to bf16 before
the next operator reads it, following section 3.3 item 3 of the report (low
precision storage, float compute, low precision write-back).  Every rounding
goes through ``_st`` with the name of its storage point: the embedding row
("embed"), each RMSNorm output ("attn_norm", "mlp_norm", "final_norm"), q/k/v
after the bias add ("q", "k", "v") and q/k again after RoPE ("q_rope",
"k_rope"), the attention output ("attn"), the o_proj and down outputs
("o_proj", "down"), each residual sum ("resid_attn", "resid_mlp"), gate and
up ("gate", "up") and the SwiGLU output ("swiglu").  The logits stay float32
and argmax runs on them.  "fp32" mode performs no rounding (the tiny fp32
model).

Pinned by: the operator pins, an fp64 brute-force forward on tiny shapes (fp32
mode), a loop-written bf16 forward that rounds at the same named points with
float64 sums (bf16 mode: identical stored values, logits to float32 rounding;
each storage point dropped in turn, or a rounding added inside RMSNorm or
SwiGLU, fails it), the KV-cache decode equalling a full recompute of the
prefix, batch independence, and the closed form when every o_proj and down
weight is zero.
"""
from __future__ import annotations

import numpy as np

from . import ops

F32 = np.float32


class OracleModel:
    """Holds float32 copies of the weights and a float32 KV cache.

    ``weights`` maps (name, layer) -> array as produced by ``synth.make_weights``
    (uint16 bf16 bit patterns or float32).  ``storage`` is "bf16" or "fp32".
    ``accum`` selects the accumulation precision of the linear layers: "f32"
    (the pages' float compute) or "f64" (the same products summed in float64,
    then rounded to float32).  Both are correct readings of the forward; the
    distance between them measures how far two exact implementations that
    differ only in summation rounding drift apart after bf16 storage rounding.
    """

    # float64 copies of the matrices are kept (rather than widened at every
    # product) while they take at most this many bytes
    F64_CACHE_BYTES = 16 << 30

    def __init__(self, shape, weights, storage: str, batch: int, max_seq: int, accum: str = "f32",
                 share_from: "OracleModel | None" = None, cache_f64: bool | None = None, kv: str = "model"):
        """``share_from``: another oracle of the same shape whose float32
        weight copies this one reuses (read-only) instead of widening its own.
        ``cache_f64`` (accum "f64"): keep float64 copies of the matrices
        instead of widening them at every product; None keeps them while they
        take at most F64_CACHE_BYTES.
        ``kv``: "model" keeps the KV cache in the storage type; "fp8" stores
        every new k / v row as FP8 E4M3 blocks of 128 with a float32 scale
        (ops.kv_quantize) and attention reads them back dequantised to bf16
        ("新一代大模型Day0推理适配与性能调优教程", step 5)."""
        if storage not in ("bf16", "fp32") or accum not in ("f32", "f64") or kv not in ("model", "fp8"):
            raise ValueError((storage, accum, kv))
        if kv == "fp8" and (storage != "bf16" or shape.dh != 128):
            raise ValueError("the FP8 KV cache needs bf16 storage and head_dim 128")
        self.kv = kv
        self.shape = shape
        self.storage = storage
        self.accum = accum
        self.batch = batch
        self.max_seq = max_seq
        if share_from is not None:
            if share_from.shape != shape:
                raise ValueError("share_from has another shape")
            self.w = share_from.w
        else:
            self.w = {}
            for key, arr in weights.items():
                self.w[key] = ops.widen_bf16(arr) if arr.dtype == np.uint16 else np.asarray(arr, F32)
        self.w64 = {}
        if cache_f64 is None:
            cache_f64 = sum(a.size for a in self.w.values()) * 8 <= self.F64_CACHE_BYTES
        if accum == "f64" and cache_f64:
            self.w64 = {id(a): a.astype(np.float64) for a in self.w.values() if a.ndim == 2}
        self.on_layer = None        # optional callback(layer) after each layer (progress reports)
        L, nkv, d = shape.nlayer, shape.nkv, shape.dh
        self.k_cache = [np.zeros((batch, nkv, max_seq, d), F32) for _ in range(L)]
        self.v_cache = [np.zeros((batch, nkv, max_seq, d), F32) for _ in range(L)]
        self.length = 0
        self.record = None

    def reset(self):
        self.length = 0

    def _st(self, x, point=None):
        """The write-back of one operator output (``point`` names it).

        bf16 storage rounds to bf16 here and nowhere else; fp32 storage keeps
        the float32 value.  When ``self.record`` is a dict, the stored value
        is appended under its point name (for the tests that check where the
        forward rounds)."""
        y = ops.bf16_round(x) if self.storage == "bf16" else np.asarray(x, F32)
        if self.record is not None and point is not None:
            self.record.setdefault(point, []).append(y.copy())
        return y

    def _weight(self, name, layer=-1):
        return self.w[(name, layer)]

    def _linear(self, x, w, b=None):
        if self.accum == "f32":
            return ops.linear(x, w, b)
        w64 = self.w64.get(id(w))
        y = np.matmul(np.asarray(x, np.float64), (w64 if w64 is not None else np.asarray(w, np.float64)).T)
        if b is not None:
            y = y + np.asarray(b, np.float64)
        return y.astype(F32)

    def forward(self, ids: np.ndarray, all_logits: bool = False, embeds: np.ndarray | None = None,
                layers: range | None = None, hidden: list | None = None):
        """Process ids [B, T] at positions length .. length+T-1.

        Returns (logits, next): logits [B, V] float32 of the last position (or
        [B, T, V] when ``all_logits``), next [B] int64 greedy tokens.
        ``embeds`` [B, T, H] replaces the embedding lookup (ids then only give
        the shape); ``layers`` restricts the layer stack (default: all);
        ``hidden``, if a list, receives the residual stream after each layer.
        """
        if embeds is not None:
            embeds = np.asarray(embeds, F32)
            ids = np.zeros(embeds.shape[:2], np.int64)
        ids = np.asarray(ids, np.int64)
        if ids.ndim == 1:
            ids = ids[:, None]
        B, T = ids.shape
        sh = self.shape
        if B != self.batch:
            raise ValueError("batch mismatch")
        P = self.length
        if P + T > self.max_seq:
            raise ValueError("KV cache capacity exceeded")
        H, nh, nkv, d = sh.hidden, sh.nh, sh.nkv, sh.dh
        st = self._st
        pos = np.arange(P, P + T)
        scale = 1.0 / np.sqrt(d)

        if embeds is not None:
            x = st(embeds, "embed")
        else:
            x = st(ops.embedding(ids.reshape(-1), self._weight("embed_tokens")), "embed").reshape(B, T, H)
        lin = self._linear
        for l in (layers if layers is not None else range(sh.nlayer)):
            W = lambda n: self._weight(n, l)          # noqa: E731
            h = st(ops.rms_norm(x, W("input_layernorm"), sh.eps), "attn_norm")
            q = st(lin(h, W("q_proj.weight"), W("q_proj.bias")), "q").reshape(B, T, nh, d)
            k = st(lin(h, W("k_proj.weight"), W("k_proj.bias")), "k").reshape(B, T, nkv, d)
            v = st(lin(h, W("v_proj.weight"), W("v_proj.bias")), "v").reshape(B, T, nkv, d)
            o = np.empty((B, T, nh, d), F32)
            for b in range(B):
                qb = st(ops.rope(q[b], pos, sh.theta), "q_rope")
                kb = st(ops.rope(k[b], pos, sh.theta), "k_rope")
                vb = v[b]
                if self.kv == "fp8":
                    kb = ops.kv_dequantize(*ops.kv_quantize(kb))
                    vb = ops.kv_dequantize(*ops.kv_quantize(vb))
                self.k_cache[l][b, :, P:P + T, :] = kb.transpose(1, 0, 2)
                self.v_cache[l][b, :, P:P + T, :] = vb.transpose(1, 0, 2)
                kc = self.k_cache[l][b, :, :P + T, :].transpose(1, 0, 2)
                vc = self.v_cache[l][b, :, :P + T, :].transpose(1, 0, 2)
                o[b] = st(ops.attention(qb, kc, vc, scale), "attn")
            a = st(lin(o.reshape(B, T, nh * d), W("o_proj.weight")), "o_proj")
            x = st(ops.add(x, a), "resid_attn")
            h2 = st(ops.rms_norm(x, W("post_attention_layernorm"), sh.eps), "mlp_norm")
            g = st(lin(h2, W("gate_proj.weight")), "gate")
            u = st(lin(h2, W("up_proj.weight")), "up")
            m = st(ops.swiglu(g, u), "swiglu")
            dn = st(lin(m, W("down_proj.weight")), "down")
            x = st(ops.add(x, dn), "resid_mlp")
            if hidden is not None:
                hidden.append(x.copy())
            if self.on_layer is not None:
                self.on_layer(l)
        self.length = P + T
        xs = x if all_logits else x[:, -1, :]
        hf = st(ops.rms_norm(xs, self._weight("norm"), sh.eps), "final_norm")
        logits = lin(hf, self._weight("lm_head"))
        nxt, _ = ops.argmax(logits if not all_logits else logits[:, -1, :])
        return logits, nxt

    def generate(self, prompt: np.ndarray, steps: int, teacher=None):
        """Prefill ``prompt``, then run ``steps`` single-token decode passes.

        The prefill yields token 0; decode pass s (1-based) feeds token s-1 and
        yields token s, so ``steps`` passes give steps + 1 tokens and the context
        grows to prompt + steps.  With ``teacher`` [B, steps + 1] the decode
        inputs come from it (teacher forcing) instead of the model's own argmax.
        Returns (tokens [B, steps + 1], list of steps + 1 logits arrays [B, V]).
        """
        logits, nxt = self.forward(prompt)
        toks = [nxt]
        all_logits = [logits]
        for s in range(1, steps + 1):
            feed = teacher[:, s - 1] if teacher is not None else toks[-1]
            logits, nxt = self.forward(np.asarray(feed)[:, None])
            toks.append(nxt)
            all_logits.append(logits)
        return np.stack(toks, axis=1), all_logits
