"""Planted mistakes in the oracle must be caught by the pins.

Each case builds a plausible wrong variant of one oracle operator (a dropped
term, a wrong sign or index, a transposed operand, the other RoPE pairing, the
epsilon outside the root, ...) and checks that the corresponding pin check
rejects it.  Model-level mutations are planted by patching ``oracle.ops`` on
the CPU, so the whole-model pins see them.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import ops
from tests import pins

F32 = np.float32


def _fails(fn, *args):
    try:
        fn(*args)
    except Exception:      # AssertionError or a shape error from the wrong variant
        return True
    return False


def rope_interleaved(x, pos, theta):
    x = np.asarray(x, F32)
    d = x.shape[-1]
    c, s = ops.rope_cos_sin(pos, d, theta)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c[:, None] - b * s[:, None]
    out[..., 1::2] = b * c[:, None] + a * s[:, None]
    return out


def rope_wrong_sign(x, pos, theta):
    x = np.asarray(x, F32)
    d = x.shape[-1]
    c, s = ops.rope_cos_sin(pos, d, theta)
    a, b = x[..., :d // 2], x[..., d // 2:]
    return np.concatenate([a * c[:, None] + b * s[:, None], b * c[:, None] - a * s[:, None]], -1)


def rope_wrong_freq(x, pos, theta):
    return ops.rope(x, pos, theta * 10)


def rms_eps_outside(x, w, eps):
    x = np.asarray(x, F32)
    return x / (np.sqrt(np.mean(x * x, -1, keepdims=True)) + F32(eps)) * w


def rms_no_mean(x, w, eps):
    x = np.asarray(x, F32)
    return x / np.sqrt(np.sum(x * x, -1, keepdims=True) + F32(eps)) * w


def attention_no_scale(q, k, v, scale):
    return ops.attention(q, k, v, 1.0)


def attention_mask_off_by_one(q, k, v, scale):
    # sees one key too few (strictly earlier keys plus itself excluded)
    T = q.shape[0]
    out = ops.attention(q, k, v, scale)
    if T > 1:
        out[1:] = ops.attention(q[1:], k[:-1], v[:-1], scale)
    return out


def attention_wrong_group(q, k, v, scale):
    nh, nkv = q.shape[1], k.shape[1]
    kk = k[:, [h % nkv for h in range(nh)]]
    vv = v[:, [h % nkv for h in range(nh)]]
    return ops.attention(q, kk, vv, scale)


def attention_no_max_shift_with_bias(q, k, v, scale):
    # adds a constant to the probabilities (unnormalised softmax)
    return ops.attention(q, k, v, scale) * F32(1.01)


def linear_transposed(x, w, b=None):
    y = np.matmul(np.asarray(x, F32), np.asarray(w, F32))
    return y + b if b is not None else y


def linear_drop_bias(x, w, b=None):
    return ops.linear(x, w)


def silu_is_sigmoid(g):
    g = np.asarray(g, F32)
    return F32(1) / (F32(1) + np.exp(-g))


def swiglu_swapped(g, u):
    return ops.silu(u) * np.asarray(g, F32)


def argmax_last_on_ties(x):
    x = np.asarray(x)
    rev = x[..., ::-1]
    idx = x.shape[-1] - 1 - np.argmax(rev, axis=-1)
    return idx.astype(np.int64), np.take_along_axis(x, idx[..., None], -1)[..., 0]


def bf16_truncate(x):
    return (np.asarray(x, F32).view(np.uint32) & np.uint32(0xFFFF0000)).view(F32)


def bf16_round_half_up(x):
    u = np.asarray(x, F32).view(np.uint32).astype(np.uint64)
    return (((u + 0x8000) >> 16) << 16).astype(np.uint32).view(F32)


def embedding_off_by_one(ids, table):
    return table[np.clip(np.asarray(ids) + 1, 0, table.shape[0] - 1)]


OP_CASES = [
    ("rope interleaved pairing", lambda: pins.check_rope(rope_interleaved, ops.rope_cos_sin)),
    ("rope wrong sign", lambda: pins.check_rope(rope_wrong_sign, ops.rope_cos_sin)),
    ("rope wrong frequency", lambda: pins.check_rope(rope_wrong_freq, ops.rope_cos_sin)),
    ("rmsnorm eps outside root", lambda: pins.check_rms_norm(rms_eps_outside)),
    ("rmsnorm sum instead of mean", lambda: pins.check_rms_norm(rms_no_mean)),
    ("attention without scale", lambda: pins.check_attention(attention_no_scale)),
    ("attention causal off by one", lambda: pins.check_attention(attention_mask_off_by_one)),
    ("attention wrong GQA map", lambda: pins.check_attention(attention_wrong_group)),
    ("attention unnormalised", lambda: pins.check_attention(attention_no_max_shift_with_bias)),
    ("linear transposed weight", lambda: pins.check_linear(linear_transposed)),
    ("linear dropped bias", lambda: pins.check_linear(linear_drop_bias)),
    ("silu is sigmoid", lambda: pins.check_silu_swiglu(silu_is_sigmoid, lambda g, u: silu_is_sigmoid(g) * u)),
    ("swiglu operands swapped", lambda: pins.check_silu_swiglu(ops.silu, swiglu_swapped)),
    ("argmax last index on ties", lambda: pins.check_argmax(argmax_last_on_ties)),
    ("bf16 truncation", lambda: pins.check_bf16_round(bf16_truncate)),
    ("bf16 round half up", lambda: pins.check_bf16_round(bf16_round_half_up)),
    ("embedding off by one", lambda: pins.check_embedding(embedding_off_by_one)),
]


@pytest.mark.parametrize("name,case", OP_CASES, ids=[c[0] for c in OP_CASES])
def test_op_mutation_is_caught(name, case):
    assert _fails(case), f"planted mistake not caught: {name}"


MODEL_PATCHES = [
    ("swiglu operands swapped", "swiglu", swiglu_swapped),
    ("rope interleaved", "rope", rope_interleaved),
    ("rope wrong frequency", "rope", rope_wrong_freq),
    ("rmsnorm eps outside", "rms_norm", rms_eps_outside),
    ("linear dropped bias", "linear", linear_drop_bias),
    ("attention wrong GQA map", "attention", attention_wrong_group),
    ("attention causal off by one", "attention", attention_mask_off_by_one),
    ("attention without scale", "attention", attention_no_scale),
]


@pytest.mark.parametrize("name,attr,bad", MODEL_PATCHES, ids=[c[0] for c in MODEL_PATCHES])
def test_model_mutation_is_caught(monkeypatch, name, attr, bad):
    monkeypatch.setattr(ops, attr, bad)
    assert _fails(pins.check_model_vs_brute, oracle.OracleModel), f"planted mistake not caught: {name}"


def test_model_mutation_residual_dropped(monkeypatch):
    monkeypatch.setattr(ops, "add", lambda a, b: np.asarray(b, F32))
    assert _fails(pins.check_model_vs_brute, oracle.OracleModel)


def test_model_mutation_cache_not_used(monkeypatch):
    """A decode step that forgets the cached keys must break decode == recompute."""
    real = ops.attention

    def only_new(q, k, v, scale):
        T = q.shape[0]
        return real(q, k[-T:], v[-T:], scale)

    monkeypatch.setattr(ops, "attention", only_new)
    assert _fails(pins.check_decode_equals_recompute, oracle.OracleModel, "fp32")


# ----------------------------------------------------------------------------- bf16 write-back points

def _skip_rounding_at(point):
    """An oracle that forgets the bf16 write-back at one storage point (the
    value is kept in float32 there)."""
    real = oracle.OracleModel._st

    def st(self, x, p=None):
        if p == point:
            y = np.asarray(x, F32)
            if self.record is not None:
                self.record.setdefault(p, []).append(y.copy())
            return y
        return real(self, x, p)
    return st


def _skip_rounding_unrecorded(point):
    """As above, but the point still records a rounded copy, so only the
    downstream values can reveal the mistake."""
    real = oracle.OracleModel._st

    def st(self, x, p=None):
        if p == point:
            if self.record is not None:
                self.record.setdefault(p, []).append(oracle.bf16_round(x))
            return np.asarray(x, F32)
        return real(self, x, p)
    return st


# Storage points whose rounding changes later values (the embedding row and
# the value projection are bf16 numbers already: weights are bf16 and v is
# stored as it leaves the bias add).
DROPPABLE = [p for p in pins.BF16_POINTS if p not in ("embed",)]


@pytest.mark.parametrize("point", DROPPABLE)
def test_bf16_dropped_rounding_fails_representability(monkeypatch, point):
    monkeypatch.setattr(oracle.OracleModel, "_st", _skip_rounding_at(point))
    assert _fails(pins.check_bf16_writeback_points, oracle.OracleModel), point


@pytest.mark.parametrize("point", DROPPABLE)
def test_bf16_dropped_rounding_fails_brute(monkeypatch, point):
    """A dropped write-back caught by the loop-written bf16 forward alone,
    through the values stored after it (the final norm: through the logits)."""
    monkeypatch.setattr(oracle.OracleModel, "_st", _skip_rounding_unrecorded(point))
    assert _fails(pins.check_bf16_writeback_vs_brute, oracle.OracleModel), point


def test_bf16_extra_rounding_inside_rmsnorm_fails_brute(monkeypatch):
    """Rounding x / rms to bf16 before the weight multiply (two roundings
    where the rule has one)."""
    def rms_two_roundings(x, w, eps):
        x = np.asarray(x, F32)
        ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
        y = oracle.bf16_round(x * (F32(1.0) / np.sqrt(ms + F32(eps))))
        return y * np.asarray(w, F32)
    monkeypatch.setattr(ops, "rms_norm", rms_two_roundings)
    assert _fails(pins.check_bf16_writeback_vs_brute, oracle.OracleModel)


def test_bf16_extra_rounding_inside_swiglu_fails_brute(monkeypatch):
    """Rounding silu(g) before the multiply by u."""
    monkeypatch.setattr(ops, "swiglu", lambda g, u: oracle.bf16_round(ops.silu(g)) * np.asarray(u, F32))
    assert _fails(pins.check_bf16_writeback_vs_brute, oracle.OracleModel)


def test_bf16_residual_rounded_once_fails_brute(monkeypatch):
    """x + round(o_proj) rounded once, written as round(x + o_proj): the
    product is not rounded before the add."""
    monkeypatch.setattr(oracle.OracleModel, "_st", _skip_rounding_unrecorded("o_proj"))
    assert _fails(pins.check_bf16_writeback_vs_brute, oracle.OracleModel)


# ----------------------------------------------------------------------------- FP8 KV cache

def e4m3_truncating(y):
    """Rounds toward zero instead of to nearest."""
    y = np.asarray(y, F32)
    vals = ops.e4m3_values()
    a = np.minimum(np.abs(y).astype(np.float64), 448.0)
    code = np.searchsorted(vals, a, side="right") - 1
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def e4m3_ties_away(y):
    """Ties away from zero instead of to even."""
    y = np.asarray(y, F32)
    vals = ops.e4m3_values()
    a = np.abs(y).astype(np.float64)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    code = np.where(vals[hi] - a <= a - vals[lo], hi, lo)
    code = np.where(a >= 448, 0x7E, code)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def e4m3_values_fnuz():
    """The bias-8 variant's magnitudes (half of E4M3FN's)."""
    return ops.e4m3_values() / 2


def kv_quantize_wrong_scale(x):
    x = np.asarray(x, F32)
    amax = np.max(np.abs(x), axis=-1, keepdims=True)
    scale = np.where(amax == 0, F32(1), amax / F32(240.0)).astype(F32)
    return ops.e4m3_encode(x / scale), np.where(amax == 0, F32(0), scale)[..., 0].astype(F32)


def kv_quantize_per_tensor(x):
    x = np.asarray(x, F32)
    amax = np.max(np.abs(x))
    scale = F32(amax / F32(448.0))
    return ops.e4m3_encode(x / scale), np.full(x.shape[:-1], scale, F32)


FP8_CASES = [
    ("e4m3 truncation", lambda: pins.check_e4m3(ops.e4m3_values, e4m3_truncating, ops.e4m3_decode)),
    ("e4m3 ties away from zero", lambda: pins.check_e4m3(ops.e4m3_values, e4m3_ties_away, ops.e4m3_decode)),
    ("e4m3 bias-8 table", lambda: pins.check_e4m3(e4m3_values_fnuz, ops.e4m3_encode, ops.e4m3_decode)),
    ("kv scale max/240", lambda: pins.check_kv_quant(kv_quantize_wrong_scale, ops.kv_dequantize)),
    ("kv scale per tensor", lambda: pins.check_kv_quant(kv_quantize_per_tensor, ops.kv_dequantize)),
]


@pytest.mark.parametrize("name,case", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_fp8_mutation_is_caught(name, case):
    assert _fails(case), f"planted mistake not caught: {name}"


def test_fp8_model_mutation_v_not_quantised(monkeypatch):
    """An FP8 cache that quantises k but stores v unquantised."""
    real = ops.kv_dequantize
    calls = [0]

    def only_k(codes, scales):
        calls[0] += 1
        return real(codes, scales)

    def quant_k_only(x):
        calls[0] += 1
        if calls[0] % 2 == 0:      # every second call is the v row
            x = np.asarray(x, F32)
            return ops.e4m3_encode(x), np.ones(x.shape[:-1], F32)
        return ops.kv_quantize(x)
    monkeypatch.setattr(ops, "kv_quantize", quant_k_only)
    assert _fails(pins.check_fp8_cache_values, oracle.OracleModel)
