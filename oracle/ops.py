"""Oracle operators: one plain NumPy function per operator of the decoder.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Compute is float32, as
the LLAISYS report prescribes ("LLAISYS 训练营结项报告", section 3.3 item 3:
low-precision storage, float compute, low-precision write-back); reductions
use NumPy's float32 routines.  ``bf16_round`` emulates the low-precision
write-back: every operator output is rounded to bf16 by the caller when the
model stores bf16.

Each function states what pins it (the checks in tests/test_oracle_*.py that
do not re-derive the function from itself).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the float32 numbers they encode (exact).

    Pinned by: known encodings (0x3F80 = 1.0, 0xC000 = -2.0, 0x7F80 = inf).
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("widen_bf16 expects uint16 bit patterns")
    return (bits.astype(np.uint32) << np.uint32(16)).view(F32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value, ties to even.

    Returns float32 arrays whose low 16 mantissa bits are zero.  Infinities are
    kept; NaN inputs stay NaN (with a quiet payload).  This is the write-back
    step of the "low precision storage, float compute" policy.

    Pinned by: exact ties 1 + 2^-8 -> 1 and 1 + 3*2^-8 -> 1 + 2^-6 (ties to
    even), values already representable are unchanged, the rounding error is
    at most half a bf16 ulp on a random sample (compared in float64).
    """
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32)
    # r = u + 0x7FFF + (bit 16 of u), then clear the low 16 bits.  For every
    # non-NaN pattern the sum stays below 2^32 (the largest, -inf or -max,
    # is 0xFF80xxxx), so uint32 arithmetic is exact; NaNs are replaced below.
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r &= np.uint32(0xFFFF0000)
    out = r.view(F32)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def embedding(ids: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Row gather: out[n, :] = table[ids[n], :] ("LLAISYS 训练营结项报告" 3.2, embedding).

    Pinned by: a table whose rows encode their own index is decoded back to
    the ids; out-of-range ids raise.
    """
    ids = np.asarray(ids)
    if ids.size and (ids.min() < 0 or ids.max() >= table.shape[0]):
        raise IndexError("token id out of range")
    return table[ids]


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * w over the last axis, in float32.

    Reading: the epsilon sits inside the square root, added to the mean square
    ("万亿参数大模型在国产加速卡上的Day-0适配教程", step 5, names the epsilon
    position as an error-prone spot; this is the Qwen2 convention).  The output is rounded once by the
    caller (no intermediate rounding of x / rms before the weight multiply).

    Pinned by: closed form on a constant vector, output RMS = sqrt(ms/(ms+eps))
    for w = 1, scale invariance, fp64 brute force.
    """
    x = np.asarray(x, F32)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    inv = F32(1.0) / np.sqrt(ms + F32(eps))
    return (x * inv) * np.asarray(w, F32)


def rope_cos_sin(pos: np.ndarray, d: int, theta: float):
    """cos/sin tables [T, d/2] for positions ``pos``.

    Frequencies inv_freq_j = theta^(-2j/d), j in [0, d/2); the angle
    pos * inv_freq_j and its cosine and sine are evaluated in float64 and then
    rounded to float32 (reading: the pages do not fix the precision of the
    angle; float64 keeps the table exact to float32 at every position).

    Pinned by: position 0 gives cos = 1, sin = 0; values against math.cos /
    math.sin at hand-picked positions.
    """
    j = np.arange(d // 2, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * j / d)
    ang = np.asarray(pos, np.float64).reshape(-1, 1) * inv_freq.reshape(1, -1)
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding of x [T, h, d] at positions pos [T] (rotate-half pairing).

    Element j is paired with j + d/2 (j < d/2): a' = a cos - b sin,
    b' = b cos + a sin, float32 arithmetic.  Reading: rotate-half, the Qwen2 /
    Hugging Face convention that the LLAISYS report matches token for token
    (section 3.5); the interleaved (2j, 2j+1) pairing is not used.

    Pinned by: identity at position 0, pair norms preserved, R(m) R(n) = R(m+n),
    <R(m) q, R(n) k> depends on m - n only, unit vector e_0 lands on
    (cos, ..., sin at index d/2), fp64 brute force.
    """
    x = np.asarray(x, F32)
    T, h, d = x.shape
    cos, sin = rope_cos_sin(pos, d, theta)
    cos = cos[:, None, :]
    sin = sin[:, None, :]
    a = x[..., : d // 2]
    b = x[..., d // 2:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray | None = None) -> np.ndarray:
    """y = x W^T (+ b); W is [out, in] row-major ("LLAISYS 训练营结项报告" 3.2 linear,
    bias optional).  Float32 BLAS matmul, float32 bias add.

    Pinned by: fp64 brute-force loops on small shapes, W = 0 gives the bias,
    one-hot inputs select weight columns.
    """
    y = np.matmul(np.asarray(x, F32), np.asarray(w, F32).T)
    if b is not None:
        y = y + np.asarray(b, F32)
    return y


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Causal grouped-query attention for one sequence.

    q [T, nh, d]; k, v [S, nkv, d] with S >= T (the first S - T keys are the
    cached past).  Query t sits at absolute position S - T + t and sees keys
    j <= S - T + t.  Query head h reads KV head h // (nh / nkv) (contiguous
    groups).  Per "万亿参数大模型在国产加速卡上的Day-0适配教程", step 5: scores = q k^T * scale, causal
    mask, max-subtracted softmax in float32, probabilities times v.  Masked
    keys get probability exactly 0.

    Pinned by: rows of the probability matrix sum to 1, query 0 of a fresh
    sequence returns v_0 exactly, future keys do not change earlier outputs,
    GQA equals MHA with repeated KV heads, fp64 brute force.
    """
    q = np.asarray(q, F32)
    k = np.asarray(k, F32)
    v = np.asarray(v, F32)
    T, nh, d = q.shape
    S, nkv, _ = k.shape
    if S < T or nh % nkv:
        raise ValueError("bad attention shapes")
    group = nh // nkv
    past = S - T
    allowed = np.arange(S)[None, :] <= (past + np.arange(T))[:, None]   # [T, S]
    out = np.empty((T, nh, d), F32)
    for h in range(nh):
        g = h // group
        s = np.matmul(q[:, h, :], k[:, g, :].T) * F32(scale)
        s = np.where(allowed, s, F32(-np.inf))
        m = np.max(s, axis=1, keepdims=True)
        e = np.where(allowed, np.exp(s - m), F32(0.0)).astype(F32)
        p = e / np.sum(e, axis=1, keepdims=True, dtype=F32)
        out[:, h, :] = np.matmul(p, v[:, g, :])
    return out


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)), float32.

    Pinned by: silu(0) = 0, silu(g) -> g for large g, -> 0 for very negative g,
    closed-form values at +-1 and 2.
    """
    g = np.asarray(g, F32)
    with np.errstate(over="ignore"):
        return g / (F32(1.0) + np.exp(-g))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """out = silu(gate) * up ("LLAISYS 训练营结项报告" 3.2 swiglu).  Reading: SiLU is
    applied to the gate projection, the up projection multiplies it, no bias.

    Pinned by: the silu pins and up = 1 returning silu(gate).
    """
    return silu(gate) * np.asarray(up, F32)


def add(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Element-wise residual add in float32.  Pinned by: integer-valued sums are exact."""
    return np.asarray(a, F32) + np.asarray(b, F32)


def argmax(x: np.ndarray):
    """(index, value) of the maximum along the last axis, lowest index on ties.

    The report's distributed argmax returns the best score with its token id
    ("LLAISYS 训练营结项报告", section 4.3 item 4); the single-device op does the
    same.  Inputs are finite by construction.

    Pinned by: brute-force Python loop on random rows, planted ties.
    """
    x = np.asarray(x)
    idx = np.argmax(x, axis=-1)
    val = np.take_along_axis(x, idx[..., None], axis=-1)[..., 0]
    return idx.astype(np.int64), val.astype(F32)


def rearrange(x: np.ndarray) -> np.ndarray:
    """Copy of x into a fresh contiguous array (same shape and values).

    The operator exists to make strided views contiguous and to write the KV
    cache ("LLAISYS 训练营结项报告" 3.2: contiguous fast path plus a general
    stride-aware copy).  Pinned by: element-wise equality with the source.
    """
    return np.array(x, copy=True, order="C")


# ----------------------------------------------------------------------------- FP8 KV cache

def e4m3_values() -> np.ndarray:
    """Magnitudes of the FP8 E4M3 codes 0x00 .. 0x7E (float64, increasing).

    OCP FP8 E4M3 ("FN", no infinities): 4 exponent bits with bias 7, 3
    mantissa bits; exponent field 0 holds the subnormals m * 2^-9, fields
    1..15 hold (1 + m/8) * 2^(e-7); 0x7F is NaN, so 0x7E = 448 is the largest
    finite value.  The KV-cache quantisation of "新一代大模型Day0推理适配与性能调优教程"
    (step 5) stores FP8 codes; the pages do not name the FP8 variant, and E4M3
    (more mantissa, range 448) is the one used for stored tensors.

    Pinned by: 1.0 = 0x38, 448 = 0x7E, the smallest subnormal 2^-9 = 0x01,
    the values strictly increase, and a loop-written enumeration of the bit
    fields in tests/_brute.py gives the same table.
    """
    codes = np.arange(0x7F)
    e = codes >> 3
    m = (codes & 7).astype(np.float64)
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.power(2.0, e - 7))


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """FP8 E4M3 codes (uint8) of the float32 values y: round to the nearest
    code, ties to the even code (mantissa LSB 0), magnitudes above 448
    saturated to 448, sign bit = sign bit of y (so -0 -> 0x80).

    Pinned by: every table value round-trips, brute-force nearest search on a
    loop-written table, closed-form ties, saturation, signed zero.
    """
    y = np.asarray(y, F32)
    vals = e4m3_values()
    a = np.abs(y).astype(np.float64)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)   # vals[hi] >= a (or top)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(a >= vals[-1], len(vals) - 1, code)
    code = np.where(a == 0, 0, code)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float32 values of FP8 E4M3 codes (0x7F / 0xFF, NaN, are never written)."""
    codes = np.asarray(codes, np.uint8)
    mag = e4m3_values()[np.minimum(codes & 0x7F, 0x7E)]
    return np.where(codes & 0x80, -mag, mag).astype(F32)


def kv_quantize(x: np.ndarray):
    """Blocks of 128 values (last axis) -> (codes uint8, scales float32).

    "新一代大模型Day0推理适配与性能调优教程", step 5: the KV cache is stored in FP8
    with one scale per token x head x 128-element block, so a block's error
    stays inside the block.  Reading (the pages do not give the scale rule):
    absmax scaling in float32, scale = max|x| / 448, code = E4M3(x / scale);
    an all-zero block has scale 0 and zero codes.

    Pinned by: the largest element of a block codes to +-448, the round trip
    error is within half an E4M3 step of each value (plus the bf16 write-back),
    zero blocks, and the brute-force encode pins.
    """
    x = np.asarray(x, F32)
    amax = np.max(np.abs(x), axis=-1, keepdims=True)
    zero = amax == 0
    scale = np.where(zero, F32(1), amax / F32(448.0)).astype(F32)
    y = np.where(zero, x, x / scale).astype(F32)
    return e4m3_encode(y), np.where(zero, F32(0), scale)[..., 0].astype(F32)


def kv_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """bf16 values (as float32) of quantised blocks: round(value(code) * scale)
    with a float32 product, rounded to bf16 (the storage type the attention
    reads).  Pinned by: the kv_quantize pins (round trip)."""
    v = e4m3_decode(codes) * np.asarray(scales, F32)[..., None]
    return bf16_round(v.astype(F32))
