"""ctypes binding of libq2.so: argument marshalling only.

Every function here has the name of the C entry point it calls (include/q2.h)
and does nothing but turn torch tensors into q2_tensor descriptors, pick the
current HIP stream and raise on a non-zero status.  All computation happens in
the library's HIP kernels; there is no fallback of any kind.  Importing this
module fails with an ImportError when libq2.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq2.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "q2.h")

Q2_F32, Q2_BF16, Q2_I64, Q2_U8 = 0, 1, 2, 3
_DTYPES = {torch.float32: Q2_F32, torch.bfloat16: Q2_BF16, torch.int64: Q2_I64, torch.uint8: Q2_U8}
STATUS = {0: "Q2_OK", -1: "Q2_EINVAL", -2: "Q2_EDTYPE", -3: "Q2_ESHAPE", -4: "Q2_ESTRIDE",
          -5: "Q2_ENOMEM", -6: "Q2_EHIP", -7: "Q2_ESTATE"}
MAX_DIMS = 5


class Q2Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_DIMS), ("stride", ctypes.c_int64 * MAX_DIMS)]


class Q2Config(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("nlayer", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("nh", ctypes.c_int32), ("nkv", ctypes.c_int32), ("dh", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("vocab", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("eps", ctypes.c_float), ("theta", ctypes.c_float),
                ("kv_fp8", ctypes.c_int32), ("page_size", ctypes.c_int32), ("kv_pages", ctypes.c_int32)]


class Q2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python qwen2_decoder_forward_amd/build.py` "
                      "(the HIP library is required, there is no fallback)")
lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.POINTER(Q2Tensor)
_S = ctypes.c_void_p
_SIGS = {
    "q2_last_error": ([], ctypes.c_char_p),
    "q2_version": ([], ctypes.c_char_p),
    "q2_embedding": ([_P, _P, _P, _S], ctypes.c_int),
    "q2_linear": ([_P, _P, _P, _P, _P, _S], ctypes.c_int),
    "q2_linear_noalloc": ([_P, _P, _P, _P, _S], ctypes.c_int),
    "q2_linear_workspace_bytes": ([ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "q2_rms_norm": ([_P, _P, _P, ctypes.c_float, _S], ctypes.c_int),
    "q2_rope": ([_P, _P, _P, ctypes.c_float, _S], ctypes.c_int),
    "q2_self_attention": ([_P, _P, _P, _P, ctypes.c_float, _P, _S], ctypes.c_int),
    "q2_self_attention_workspace_bytes": ([ctypes.c_int32] * 7 + [ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "q2_swiglu": ([_P, _P, _P, _S], ctypes.c_int),
    "q2_add": ([_P, _P, _P, _S], ctypes.c_int),
    "q2_argmax": ([_P, _P, _P, _S], ctypes.c_int),
    "q2_rearrange": ([_P, _P, _S], ctypes.c_int),
    "q2_model_create": ([ctypes.POINTER(Q2Config), ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)], ctypes.c_int),
    "q2_model_device_bytes": ([ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "q2_model_load_weight": ([ctypes.c_void_p, ctypes.c_char_p, ctypes.c_int32, _P, _S], ctypes.c_int),
    "q2_model_prefill": ([ctypes.c_void_p, _P, _P, _P, _S], ctypes.c_int),
    "q2_model_prefill_embeds": ([ctypes.c_void_p, _P, _P, _P, _S], ctypes.c_int),
    "q2_model_hidden_view": ([ctypes.c_void_p, _P], ctypes.c_int),
    "q2_model_decode": ([ctypes.c_void_p, _P, _P, _P, _S], ctypes.c_int),
    "q2_model_generate": ([ctypes.c_void_p, _P, ctypes.c_int32, _P, _S], ctypes.c_int),
    "q2_model_continue": ([ctypes.c_void_p, ctypes.c_int32, _P, _S], ctypes.c_int),
    "q2_model_kv_view": ([ctypes.c_void_p, ctypes.c_int32, _P, _P], ctypes.c_int),
    "q2_model_kv_scale_view": ([ctypes.c_void_p, ctypes.c_int32, _P, _P], ctypes.c_int),
    "q2_model_seq_prefill": ([ctypes.c_void_p, ctypes.c_int32, _P, _P, _P, _S], ctypes.c_int),
    "q2_model_seq_release": ([ctypes.c_void_p, ctypes.c_int32, _S], ctypes.c_int),
    "q2_model_seq_length": ([ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    "q2_model_free_pages": ([ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    "q2_model_replay_stage": ([ctypes.c_void_p] + [ctypes.c_int32] * 4 + [_S], ctypes.c_int),
    "q2_kv_quantize": ([_P, _P, _P, _S], ctypes.c_int),
    "q2_kv_dequantize": ([_P, _P, _P, _S], ctypes.c_int),
    "q2_model_length": ([ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    "q2_model_reset": ([ctypes.c_void_p], ctypes.c_int),
    "q2_model_set_decode_path": ([ctypes.c_void_p, ctypes.c_int32], ctypes.c_int),
    "q2_model_decode_path": ([ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    "q2_model_check": ([ctypes.c_void_p], ctypes.c_int),
    "q2_model_destroy": ([ctypes.c_void_p], None),
}
for _name, (_args, _ret) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret


def header_functions(path: str = HEADER_PATH):
    """Names of the functions include/q2.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q2_[a-z0-9_]+)\s*\(", text)))


def version() -> str:
    return lib.q2_version().decode()


def _check(status: int):
    if status != 0:
        raise Q2Error(status, lib.q2_last_error().decode())


def desc(t) -> Q2Tensor | None:
    """q2_tensor descriptor of a torch tensor (None passes through as NULL)."""
    if t is None or isinstance(t, Q2Tensor):
        return t
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > MAX_DIMS:
        raise ValueError("too many dimensions")
    d = Q2Tensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _DTYPES[t.dtype]
    if t.dim() == 0:
        d.ndim = 1
        d.shape[0], d.stride[0] = 1, 1
    else:
        d.ndim = t.dim()
        for i, (n, s) in enumerate(zip(t.shape, t.stride())):
            d.shape[i], d.stride[i] = n, s
    return d


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    if not torch.cuda.is_available():
        return ctypes.c_void_p(None)   # null stream; host-side validation still runs
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ------------------------------------------------------------------ operators

def q2_embedding(out, ids, weight, stream=None):
    _check(lib.q2_embedding(_ref(desc(out)), _ref(desc(ids)), _ref(desc(weight)), _stream(stream)))
    return out


def q2_linear(out, inp, weight, bias=None, workspace=None, stream=None):
    _check(lib.q2_linear(_ref(desc(out)), _ref(desc(inp)), _ref(desc(weight)), _ref(desc(bias)),
                         _ref(desc(workspace)), _stream(stream)))
    return out


def q2_linear_noalloc(out, inp, weight, bias=None, stream=None):
    _check(lib.q2_linear_noalloc(_ref(desc(out)), _ref(desc(inp)), _ref(desc(weight)), _ref(desc(bias)),
                                 _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def q2_linear_workspace_bytes(M, N, K, dtype=Q2_BF16) -> int:
    n = ctypes.c_size_t()
    _check(lib.q2_linear_workspace_bytes(int(M), int(N), int(K), int(dtype), ctypes.byref(n)))
    return n.value


def q2_rms_norm(out, inp, weight, eps, stream=None):
    _check(lib.q2_rms_norm(_ref(desc(out)), _ref(desc(inp)), _ref(desc(weight)), float(eps), _stream(stream)))
    return out


def q2_rope(out, inp, pos, theta, stream=None):
    _check(lib.q2_rope(_ref(desc(out)), _ref(desc(inp)), _ref(desc(pos)), float(theta), _stream(stream)))
    return out


def q2_self_attention(out, q, k, v, scale, workspace=None, stream=None):
    _check(lib.q2_self_attention(_ref(desc(out)), _ref(desc(q)), _ref(desc(k)), _ref(desc(v)), float(scale),
                                 _ref(desc(workspace)), _stream(stream)))
    return out


def q2_self_attention_workspace_bytes(B, T, S, nh, nkv, d, dtype=Q2_BF16) -> int:
    n = ctypes.c_size_t()
    _check(lib.q2_self_attention_workspace_bytes(int(B), int(T), int(S), int(nh), int(nkv), int(d), int(dtype),
                                                 ctypes.byref(n)))
    return n.value


def workspace(nbytes: int, device=None) -> torch.Tensor:
    """A device tensor of at least ``nbytes`` bytes to pass as an operator's
    workspace (float32 elements; 16-byte aligned like every torch allocation)."""
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    return torch.empty(max(4, -(-int(nbytes) // 16) * 4), dtype=torch.float32, device=dev)


def q2_swiglu(out, gate, up, stream=None):
    _check(lib.q2_swiglu(_ref(desc(out)), _ref(desc(gate)), _ref(desc(up)), _stream(stream)))
    return out


def q2_add(c, a, b, stream=None):
    _check(lib.q2_add(_ref(desc(c)), _ref(desc(a)), _ref(desc(b)), _stream(stream)))
    return c


def q2_argmax(max_idx, max_val, vals, stream=None):
    _check(lib.q2_argmax(_ref(desc(max_idx)), _ref(desc(max_val)), _ref(desc(vals)), _stream(stream)))
    return max_idx, max_val


def q2_rearrange(out, inp, stream=None):
    _check(lib.q2_rearrange(_ref(desc(out)), _ref(desc(inp)), _stream(stream)))
    return out


def q2_kv_quantize(codes, scales, x, stream=None):
    _check(lib.q2_kv_quantize(_ref(desc(codes)), _ref(desc(scales)), _ref(desc(x)), _stream(stream)))
    return codes, scales


def q2_kv_dequantize(x, codes, scales, stream=None):
    _check(lib.q2_kv_dequantize(_ref(desc(x)), _ref(desc(codes)), _ref(desc(scales)), _stream(stream)))
    return x


# ------------------------------------------------------------------ model driver

def q2_model_create(cfg: Q2Config, device: int = 0) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(lib.q2_model_create(ctypes.byref(cfg), int(device), ctypes.byref(h)))
    return h


def q2_model_device_bytes(h) -> int:
    n = ctypes.c_size_t()
    _check(lib.q2_model_device_bytes(h, ctypes.byref(n)))
    return n.value


def q2_model_load_weight(h, name: str, layer: int, src, stream=None):
    _check(lib.q2_model_load_weight(h, name.encode(), int(layer), _ref(desc(src)), _stream(stream)))


def q2_model_prefill(h, ids, next_ids, logits=None, stream=None):
    _check(lib.q2_model_prefill(h, _ref(desc(ids)), _ref(desc(next_ids)), _ref(desc(logits)), _stream(stream)))


def q2_model_prefill_embeds(h, embeds, next_ids, logits=None, stream=None):
    _check(lib.q2_model_prefill_embeds(h, _ref(desc(embeds)), _ref(desc(next_ids)), _ref(desc(logits)),
                                       _stream(stream)))


def q2_model_hidden_view(h) -> Q2Tensor:
    x = Q2Tensor()
    _check(lib.q2_model_hidden_view(h, ctypes.byref(x)))
    return x


def q2_model_decode(h, ids, next_ids, logits=None, stream=None):
    _check(lib.q2_model_decode(h, _ref(desc(ids)), _ref(desc(next_ids)), _ref(desc(logits)), _stream(stream)))


def q2_model_generate(h, prompt, steps: int, out_ids, stream=None):
    _check(lib.q2_model_generate(h, _ref(desc(prompt)), int(steps), _ref(desc(out_ids)), _stream(stream)))


def q2_model_continue(h, steps: int, out_ids=None, stream=None):
    _check(lib.q2_model_continue(h, int(steps), _ref(desc(out_ids)), _stream(stream)))


def q2_model_kv_view(h, layer: int):
    k, v = Q2Tensor(), Q2Tensor()
    _check(lib.q2_model_kv_view(h, int(layer), ctypes.byref(k), ctypes.byref(v)))
    return k, v


def q2_model_kv_scale_view(h, layer: int):
    k, v = Q2Tensor(), Q2Tensor()
    _check(lib.q2_model_kv_scale_view(h, int(layer), ctypes.byref(k), ctypes.byref(v)))
    return k, v


def q2_model_seq_prefill(h, slot: int, ids, next_ids=None, logits=None, stream=None):
    _check(lib.q2_model_seq_prefill(h, int(slot), _ref(desc(ids)), _ref(desc(next_ids)), _ref(desc(logits)),
                                    _stream(stream)))


def q2_model_seq_release(h, slot: int, stream=None):
    _check(lib.q2_model_seq_release(h, int(slot), _stream(stream)))


def q2_model_seq_length(h, slot: int) -> int:
    n = ctypes.c_int32()
    _check(lib.q2_model_seq_length(h, int(slot), ctypes.byref(n)))
    return n.value


def q2_model_free_pages(h) -> int:
    n = ctypes.c_int32()
    _check(lib.q2_model_free_pages(h, ctypes.byref(n)))
    return n.value


STAGE_QKV, STAGE_ATTN, STAGE_O, STAGE_GATE_UP, STAGE_DOWN, STAGE_ATTN_CORE = 0, 1, 2, 3, 4, 5


def q2_model_replay_stage(h, stage: int, batch: int, tokens: int, reps: int, stream=None):
    _check(lib.q2_model_replay_stage(h, int(stage), int(batch), int(tokens), int(reps), _stream(stream)))


def q2_model_length(h) -> int:
    n = ctypes.c_int32()
    _check(lib.q2_model_length(h, ctypes.byref(n)))
    return n.value


def q2_model_reset(h):
    _check(lib.q2_model_reset(h))


def q2_model_set_decode_path(h, persistent: int):
    _check(lib.q2_model_set_decode_path(h, int(persistent)))


def q2_model_decode_path(h, batch: int) -> int:
    n = ctypes.c_int32()
    _check(lib.q2_model_decode_path(h, int(batch), ctypes.byref(n)))
    return n.value


def q2_model_check(h):
    _check(lib.q2_model_check(h))


def q2_model_destroy(h):
    lib.q2_model_destroy(h)
