"""Python handle around the q2 model driver (argument marshalling only)."""
from __future__ import annotations

import numpy as np
import torch

from . import _lib
from ._lib import Q2Config, Q2_BF16, Q2_F32


def make_config(shape, max_seq: int, max_batch: int, kv_fp8: bool = False, page_size: int = 0,
                kv_pages: int = 0) -> Q2Config:
    """q2_config from any object with the Qwen2 shape attributes
    (dtype "f32"/"bf16", nlayer, hidden, nh, nkv, dh, inter, vocab, eps, theta);
    ``kv_fp8`` selects the FP8 KV cache, ``page_size`` > 0 the paged cache
    (``kv_pages`` pages, 0 = room for every sequence at max_seq)."""
    c = Q2Config()
    c.kv_fp8 = 1 if kv_fp8 else 0
    c.page_size, c.kv_pages = page_size, kv_pages
    c.dtype = Q2_BF16 if shape.dtype == "bf16" else Q2_F32
    c.nlayer, c.hidden, c.nh, c.nkv = shape.nlayer, shape.hidden, shape.nh, shape.nkv
    c.dh, c.inter, c.vocab = shape.dh, shape.inter, shape.vocab
    c.max_seq, c.max_batch = max_seq, max_batch
    c.eps, c.theta = shape.eps, shape.theta
    return c


class Model:
    """Owns one q2_model.  Weights are loaded from device tensors with
    `load_weight(name, layer, tensor)`; all calls run on the current stream."""

    def __init__(self, shape, max_seq: int, max_batch: int, device: int = 0, kv_fp8: bool = False,
                 page_size: int = 0, kv_pages: int = 0):
        self.shape = shape
        self.max_seq = max_seq
        self.max_batch = max_batch
        self.device = device
        self.kv_fp8 = kv_fp8
        self.page_size = page_size
        self.torch_dtype = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
        self.handle = _lib.q2_model_create(make_config(shape, max_seq, max_batch, kv_fp8, page_size, kv_pages), device)

    def close(self):
        if self.handle:
            _lib.q2_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def device_bytes(self) -> int:
        return _lib.q2_model_device_bytes(self.handle)

    def load_weight(self, name: str, layer: int, tensor):
        _lib.q2_model_load_weight(self.handle, name, layer, tensor)

    def prefill(self, ids, logits: bool = False):
        B = ids.shape[0] if ids.dim() == 2 else 1
        nxt = torch.empty(B, dtype=torch.int64, device=ids.device)
        lg = torch.empty(B, self.shape.vocab, dtype=torch.float32, device=ids.device) if logits else None
        _lib.q2_model_prefill(self.handle, ids, nxt, lg)
        return (nxt, lg) if logits else nxt

    def prefill_embeds(self, embeds, logits: bool = False):
        B = embeds.shape[0]
        nxt = torch.empty(B, dtype=torch.int64, device=embeds.device)
        lg = torch.empty(B, self.shape.vocab, dtype=torch.float32, device=embeds.device) if logits else None
        _lib.q2_model_prefill_embeds(self.handle, embeds, nxt, lg)
        return (nxt, lg) if logits else nxt

    def hidden(self):
        """Copy of the residual stream rows of the last chunk, [rows, H]."""
        view = _lib.q2_model_hidden_view(self.handle)
        out = torch.empty(view.shape[0], view.shape[1], dtype=self.torch_dtype, device=f"cuda:{self.device}")
        _lib.q2_rearrange(out, view)
        return out

    def decode(self, ids, logits: bool = False):
        B = ids.shape[0]
        nxt = torch.empty(B, dtype=torch.int64, device=ids.device)
        lg = torch.empty(B, self.shape.vocab, dtype=torch.float32, device=ids.device) if logits else None
        _lib.q2_model_decode(self.handle, ids, nxt, lg)
        return (nxt, lg) if logits else nxt

    def generate(self, prompt, steps: int, out=None):
        B = prompt.shape[0]
        if out is None:
            out = torch.empty(B, steps + 1, dtype=torch.int64, device=prompt.device)
        _lib.q2_model_generate(self.handle, prompt, steps, out)
        return out

    def continue_(self, steps: int, out=None):
        """Greedy decode `steps` more tokens from the device-resident state."""
        _lib.q2_model_continue(self.handle, steps, out)
        return out

    def seq_prefill(self, slot: int, ids, logits: bool = False):
        """Prefill the token ids [T] of sequence `slot` (paged cache), after
        whatever that slot already holds; returns its next token (and logits)."""
        nxt = torch.empty(1, dtype=torch.int64, device=ids.device)
        lg = torch.empty(1, self.shape.vocab, dtype=torch.float32, device=ids.device) if logits else None
        _lib.q2_model_seq_prefill(self.handle, slot, ids, nxt, lg)
        return (nxt, lg) if logits else nxt

    def seq_release(self, slot: int):
        _lib.q2_model_seq_release(self.handle, slot)

    def seq_length(self, slot: int) -> int:
        return _lib.q2_model_seq_length(self.handle, slot)

    def free_pages(self) -> int:
        return _lib.q2_model_free_pages(self.handle)

    def kv_view(self, layer: int):
        """q2_tensor descriptors (k, v) of layer `layer`'s cache, [max_batch, max_seq, nkv, dh]."""
        return _lib.q2_model_kv_view(self.handle, layer)

    def kv_scale_view(self, layer: int):
        """q2_tensor descriptors (k, v) of layer `layer`'s FP8 scales, [max_batch, max_seq, nkv]."""
        return _lib.q2_model_kv_scale_view(self.handle, layer)

    def length(self) -> int:
        return _lib.q2_model_length(self.handle)

    def reset(self):
        _lib.q2_model_reset(self.handle)

    def set_decode_path(self, persistent: bool):
        _lib.q2_model_set_decode_path(self.handle, 1 if persistent else 0)

    def decode_path(self, batch: int) -> bool:
        return bool(_lib.q2_model_decode_path(self.handle, batch))

    def check(self):
        _lib.q2_model_check(self.handle)


def weight_tensor(arr, device: int = 0) -> torch.Tensor:
    """A host weight as a device tensor, bit for bit: uint16 arrays hold bf16
    bit patterns, float32 arrays float32 values."""
    dev = f"cuda:{device}"
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)


def load_model(shape, weights, max_seq: int, max_batch: int, device: int = 0, kv_fp8: bool = False,
               page_size: int = 0, kv_pages: int = 0) -> Model:
    """Create a model and copy every weight of ``weights`` ({(name, layer):
    host array}, Hugging Face Qwen2 names, layer -1 for the global tensors)
    into it, one tensor at a time (each upload is freed once the library has
    packed it)."""
    m = Model(shape, max_seq, max_batch, device, kv_fp8, page_size, kv_pages)
    for (name, layer), arr in weights.items():
        t = weight_tensor(arr, device)
        m.load_weight(name, layer, t)
        torch.cuda.synchronize(device)
        del t
    return m
