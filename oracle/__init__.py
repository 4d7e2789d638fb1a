"""Oracle for the Qwen2 decoder forward -- TEST INFRASTRUCTURE ONLY.

A plain, slow, CPU-only NumPy implementation of what the GPU library computes.
It exists to check the HIP path, never to stand in for it: only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it.  It shares no code with the HIP library (no kernels, headers, helpers or
tables); the only thing both sides read is the seeded input generator in
``synth``.

Sources of the method (page titles as printed on the pages):

* "LLAISYS 训练营结项报告" (PR #49 of InfiniTensor/llaisys), section 3.2
  (third and fourth layers: the operator set add, argmax, embedding, linear,
  rms_norm, rope, self_attention, swiglu, rearrange, and a Qwen2 model that
  keeps weights, buffers and a KV cache on the device), section 3.3 (low
  precision storage, float compute, low precision write-back), section 4.3
  item 4 (argmax returns the best score together with its token id).
* "新一代大模型Day0推理适配与性能调优教程", step 5 (layered quantisation: the KV
  cache stored as FP8 per token x per head x 128-element block, accumulation
  kept in high precision) and its verification section (top-K overlap before
  and after quantisation).
* "万亿参数大模型在国产加速卡上的Day-0适配教程" (Baidu cloud article), step 5 (attention: scaled
  Q K^T, causal mask, numerically stable softmax, times V; mask, scale and the
  position of the norm epsilon are the error-prone spots), step 6 (fp32
  device-independent reference, max-abs-error / cosine comparison, tolerance
  that must not grow with depth), step 7 (KV-cache size formula).

Where the pages leave a step open the standard Qwen2 definition is taken
(rotate-half RoPE, epsilon inside the square root, SiLU on the gate
projection, bias only on q/k/v, untied LM head, first index on argmax ties);
every such reading is listed with the module that implements it.

Modules:
  ops     -- one function per operator, fp32 compute (optional bf16 storage),
             and the FP8 E4M3 KV-cache codec
  model   -- the whole decoder: prefill and single-token decode with a KV cache
             (in the storage type or FP8)
  parity  -- the teacher-forced comparison of another forward's logits with
             the oracle's

Parity status of each function is stated in its docstring ("pinned by ...").
"""
from .ops import (bf16_round, widen_bf16, embedding, rms_norm, rope_cos_sin, rope, linear,
                  attention, silu, swiglu, add, argmax, rearrange, e4m3_values, e4m3_encode, e4m3_decode,
                  kv_quantize, kv_dequantize)
from .model import OracleModel

__all__ = ["bf16_round", "widen_bf16", "embedding", "rms_norm", "rope_cos_sin", "rope", "linear",
           "attention", "silu", "swiglu", "add", "argmax", "rearrange", "e4m3_values", "e4m3_encode",
           "e4m3_decode", "kv_quantize", "kv_dequantize", "OracleModel"]
