"""Seeded synthetic inputs for the Qwen2 decoder forward: shapes, weights, prompts.

This module is shared by the oracle, the tests and the benchmark, and by
nothing else.  It holds no arithmetic of the forward pass itself: it only
describes the five workloads and draws their random weights and token ids.

Workloads (named after the model shapes the LLAISYS report runs, "LLAISYS
训练营结项报告", section 3 / 4: DeepSeek-R1-Distill-Qwen-1.5B, a Qwen2 model):

  A  tiny fp32 decoder: 2 layers, hidden 128, 4 Q / 2 KV heads, head_dim 32,
     intermediate 384, vocab 1024; batch 1, prompt 16, 16 greedy steps.
  B  Qwen2-1.5B shape, bf16: batch 1, prompt 64, 128 greedy steps.
  C  Qwen2-1.5B shape, bf16: batch 1, prefill of 4096 tokens only.
  D  Qwen2-1.5B shape, bf16: 64 sequences x 4096-token prefilled KV cache,
     32 decode steps.
  E  Qwen2-7B shape, bf16: batch 8, prompt 1024, 256 greedy steps.

Weight recipe (every tensor independently seeded, so generation is parallel
and the values do not depend on the thread count):

  * matrices and embeddings: N(0, 0.02)
  * RMSNorm weights: 1 + N(0, 0.02) (so the weight multiply is exercised and
    activations keep unit scale)
  * QKV biases: N(0, 0.02)

For bf16 workloads the normal draw is made in float32 and the bf16 value is the
upper half of its bit pattern (truncation).  The weights are therefore exact
bf16 numbers that both sides read bit-for-bit; how they were drawn is not part
of the method.  Prompt ids are uniform in [0, vocab).
"""
from __future__ import annotations

import dataclasses
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "ModelShape", "Workload", "WORKLOADS", "SHAPES", "weight_names",
    "make_weights", "make_prompt", "tensor_shape",
]


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    dtype: str          # "f32" or "bf16" (storage type of weights and activations)
    nlayer: int
    hidden: int
    nh: int
    nkv: int
    dh: int
    inter: int
    vocab: int
    theta: float
    eps: float = 1e-6

    @property
    def qkv_out(self) -> int:
        return (self.nh + 2 * self.nkv) * self.dh

    def n_params(self) -> int:
        per_layer = (self.qkv_out * self.hidden + self.qkv_out          # qkv + bias
                     + self.hidden * self.nh * self.dh                  # o_proj
                     + 3 * self.inter * self.hidden                     # gate, up, down
                     + 2 * self.hidden)                                 # two norms
        return (self.nlayer * per_layer + 2 * self.vocab * self.hidden + self.hidden)


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    shape: ModelShape
    batch: int
    prompt: int
    steps: int          # greedy decode steps after the prompt
    weight_seed: int = 1234
    prompt_seed: int = 5678
    description: str = ""

    @property
    def max_seq(self) -> int:
        return self.prompt + self.steps


TINY = ModelShape("tiny-qwen2-fp32", "f32", 2, 128, 4, 2, 32, 384, 1024, 10000.0)
Q15B = ModelShape("qwen2-1.5b", "bf16", 28, 1536, 12, 2, 128, 8960, 151936, 10000.0)
Q7B = ModelShape("qwen2-7b", "bf16", 28, 3584, 28, 4, 128, 18944, 152064, 1_000_000.0)
SHAPES = {"tiny": TINY, "1.5b": Q15B, "7b": Q7B}

WORKLOADS = {
    "A": Workload("A", TINY, 1, 16, 16, description="tiny fp32, prompt 16 + 16 greedy steps"),
    "B": Workload("B", Q15B, 1, 64, 128, description="1.5B bf16, batch 1, prompt 64 + 128 greedy steps"),
    "C": Workload("C", Q15B, 1, 4096, 0, description="1.5B bf16, prefill 4096 tokens"),
    "D": Workload("D", Q15B, 64, 4096, 32, description="1.5B bf16, 64 x 4096 KV cache, 32 decode steps"),
    "E": Workload("E", Q7B, 8, 1024, 256, description="7B bf16, batch 8, prompt 1024 + 256 greedy steps"),
}

# Per-layer tensor names (Hugging Face Qwen2 naming) and global tensors.
LAYER_TENSORS = ("input_layernorm", "q_proj.weight", "q_proj.bias", "k_proj.weight", "k_proj.bias",
                 "v_proj.weight", "v_proj.bias", "o_proj.weight", "post_attention_layernorm",
                 "gate_proj.weight", "up_proj.weight", "down_proj.weight")
GLOBAL_TENSORS = ("embed_tokens", "norm", "lm_head")


def weight_names(shape: ModelShape):
    """(name, layer) pairs of every tensor; layer is -1 for global tensors."""
    out = [(n, -1) for n in GLOBAL_TENSORS]
    for l in range(shape.nlayer):
        out += [(n, l) for n in LAYER_TENSORS]
    return out


def tensor_shape(shape: ModelShape, name: str) -> tuple:
    H, d = shape.hidden, shape.dh
    table = {
        "embed_tokens": (shape.vocab, H), "lm_head": (shape.vocab, H), "norm": (H,),
        "input_layernorm": (H,), "post_attention_layernorm": (H,),
        "q_proj.weight": (shape.nh * d, H), "q_proj.bias": (shape.nh * d,),
        "k_proj.weight": (shape.nkv * d, H), "k_proj.bias": (shape.nkv * d,),
        "v_proj.weight": (shape.nkv * d, H), "v_proj.bias": (shape.nkv * d,),
        "o_proj.weight": (H, shape.nh * d),
        "gate_proj.weight": (shape.inter, H), "up_proj.weight": (shape.inter, H),
        "down_proj.weight": (H, shape.inter),
    }
    return table[name]


def _tensor_id(name: str, layer: int) -> int:
    return zlib.crc32(f"{layer}:{name}".encode())


_BLOCK = 1 << 23   # elements per independently seeded block


def _fill_block(args):
    out, seed, tid, blk, offset, scale = args
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, blk])))
    g.standard_normal(out=out, dtype=np.float32)
    out *= np.float32(scale)
    if offset:
        out += np.float32(offset)


def _draw(seed: int, name: str, layer: int, n: int, scale: float, offset: float, pool) -> np.ndarray:
    buf = np.empty(n, np.float32)
    tid = _tensor_id(name, layer)
    jobs = [(buf[b * _BLOCK:(b + 1) * _BLOCK], seed, tid, b, offset, scale)
            for b in range((n + _BLOCK - 1) // _BLOCK)]
    list(pool.map(_fill_block, jobs))
    return buf


def _to_storage(buf: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return buf
    # bf16 bit pattern = upper 16 bits of the float32 draw (truncation)
    return (buf.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def make_weights(wl_or_shape, seed: int | None = None, threads: int | None = None,
                 names=None, norm_offset: float = 1.0):
    """Return {(name, layer): ndarray} for every tensor of the model.

    bf16 tensors are returned as uint16 bit patterns, fp32 tensors as float32.
    ``names`` restricts generation to a subset of (name, layer) pairs.
    """
    if isinstance(wl_or_shape, Workload):
        shape = wl_or_shape.shape
        seed = wl_or_shape.weight_seed if seed is None else seed
    else:
        shape = wl_or_shape
        seed = 1234 if seed is None else seed
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    wanted = names if names is not None else weight_names(shape)
    out = {}
    with ThreadPoolExecutor(threads) as pool:
        for name, layer in wanted:
            shp = tensor_shape(shape, name)
            n = int(np.prod(shp))
            is_norm = name in ("norm", "input_layernorm", "post_attention_layernorm")
            buf = _draw(seed, name, layer, n, 0.02, norm_offset if is_norm else 0.0, pool)
            out[(name, layer)] = _to_storage(buf, shape.dtype).reshape(shp)
    return out


def make_prompt(wl: Workload, seed: int | None = None, batch: int | None = None,
                length: int | None = None) -> np.ndarray:
    """Uniform int64 token ids in [0, vocab), shape [batch, length]."""
    seed = wl.prompt_seed if seed is None else seed
    batch = wl.batch if batch is None else batch
    length = wl.prompt if length is None else length
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x70])))
    return g.integers(0, wl.shape.vocab, size=(batch, length), dtype=np.int64)

