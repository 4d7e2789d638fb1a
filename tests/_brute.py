"""Brute-force float64 Qwen2 forward for tiny shapes (pure Python loops).

An independent second reading of the same definition, written element by
element with explicit indices so that a transposed operand, a wrong head
mapping or a dropped term in the NumPy oracle shows up as a mismatch.

With ``bf16_storage=True`` it also applies the low-precision write-back of
"LLAISYS 训练营结项报告" section 3.3 item 3 (store bf16, compute float, write
back bf16) at the storage points the forward takes: the embedding row, each
RMSNorm output, q/k/v after the bias, q and k again after RoPE, the attention
output, the o_proj and down products, each residual sum, gate and up, the
SwiGLU output.  Logits stay unrounded.  The rounding is a pure-Python
round-to-nearest-even of the float64 value to 8 significant bits
(``bf16``), written from the format's definition, not from the oracle's
bit-pattern routine.  This pins where the oracle's bf16 mode rounds.
"""
import math
import struct


def bf16_bits_to_float(b):
    """The number a bf16 bit pattern encodes: the upper half of a float32."""
    return struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]


def bf16(x):
    """Round a Python float to the nearest bfloat16 value (8 significant
    bits, exponent range of float32), ties to even."""
    if x == 0.0 or math.isinf(x) or math.isnan(x):
        return x
    m, e = math.frexp(x)            # x = m * 2**e, 0.5 <= |m| < 1
    e = max(e, -125)                # below 2**-126 the format is subnormal: fixed step 2**-133
    step = math.ldexp(1.0, e - 8)
    return round(x / step) * step   # round() on a float ties to even


def _num(v, bits):
    return bf16_bits_to_float(v) if bits else float(v)


def _vec(a):
    bits = str(a.dtype) == "uint16"
    return [_num(v, bits) for v in a]


def _mat(a):
    bits = str(a.dtype) == "uint16"
    return [[_num(v, bits) for v in row] for row in a]


def rmsnorm(x, w, eps):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[i] * r * w[i] for i in range(len(x))]


def matvec(W, x, b=None):
    # W[out][in], y[o] = sum_i W[o][i] x[i] (+ b[o])
    out = []
    for o in range(len(W)):
        s = 0.0
        row = W[o]
        for i in range(len(x)):
            s += row[i] * x[i]
        out.append(s + (b[o] if b is not None else 0.0))
    return out


def rope_head(vec, pos, theta):
    d = len(vec)
    half = d // 2
    out = list(vec)
    for j in range(half):
        ang = pos * theta ** (-2.0 * j / d)
        c, s = math.cos(ang), math.sin(ang)
        a, b = vec[j], vec[j + half]
        out[j] = a * c - b * s
        out[j + half] = b * c + a * s
    return out


def silu(g):
    return g / (1.0 + math.exp(-g)) if g > -700 else 0.0


class BruteModel:
    def __init__(self, shape, weights, bf16_storage=False):
        self.sh = shape
        self.bf16 = bf16_storage
        self.record = {}            # storage point -> list of stored vectors, in order
        self.W = {}
        for key, arr in weights.items():
            self.W[key] = _mat(arr) if arr.ndim == 2 else _vec(arr)
        self.K = [[[] for _ in range(shape.nkv)] for _ in range(shape.nlayer)]
        self.V = [[[] for _ in range(shape.nkv)] for _ in range(shape.nlayer)]
        self.pos = 0

    def _store(self, point, vec):
        out = [bf16(v) for v in vec] if self.bf16 else vec
        self.record.setdefault(point, []).append(out)
        return out

    def step(self, token):
        """Process one token of a single sequence; returns its logits (list)."""
        sh = self.sh
        d, nh, nkv = sh.dh, sh.nh, sh.nkv
        grp = nh // nkv
        st = self._store
        x = st("embed", list(self.W[("embed_tokens", -1)][token]))
        for l in range(sh.nlayer):
            W = lambda n: self.W[(n, l)]  # noqa: E731
            h = st("attn_norm", rmsnorm(x, W("input_layernorm"), sh.eps))
            q = st("q", matvec(W("q_proj.weight"), h, W("q_proj.bias")))
            k = st("k", matvec(W("k_proj.weight"), h, W("k_proj.bias")))
            v = st("v", matvec(W("v_proj.weight"), h, W("v_proj.bias")))
            krot = []
            for g in range(nkv):
                krot += rope_head(k[g * d:(g + 1) * d], self.pos, sh.theta)
            krot = st("k_rope", krot)
            for g in range(nkv):
                self.K[l][g].append(krot[g * d:(g + 1) * d])
                self.V[l][g].append(v[g * d:(g + 1) * d])
            qrot = []
            for hh in range(nh):
                qrot += rope_head(q[hh * d:(hh + 1) * d], self.pos, sh.theta)
            qrot = st("q_rope", qrot)
            att = []
            for hh in range(nh):
                g = hh // grp
                qh = qrot[hh * d:(hh + 1) * d]
                keys = self.K[l][g]
                scores = [sum(qh[i] * kk[i] for i in range(d)) / math.sqrt(d) for kk in keys]
                m = max(scores)
                e = [math.exp(s - m) for s in scores]
                z = sum(e)
                o = [0.0] * d
                for j, vv in enumerate(self.V[l][g]):
                    for i in range(d):
                        o[i] += e[j] / z * vv[i]
                att += o
            att = st("attn", att)
            a = st("o_proj", matvec(W("o_proj.weight"), att))
            x = st("resid_attn", [x[i] + a[i] for i in range(len(x))])
            h2 = st("mlp_norm", rmsnorm(x, W("post_attention_layernorm"), sh.eps))
            gt = st("gate", matvec(W("gate_proj.weight"), h2))
            up = st("up", matvec(W("up_proj.weight"), h2))
            mm = st("swiglu", [silu(gt[i]) * up[i] for i in range(len(gt))])
            dn = st("down", matvec(W("down_proj.weight"), mm))
            x = st("resid_mlp", [x[i] + dn[i] for i in range(len(x))])
        self.pos += 1
        hf = st("final_norm", rmsnorm(x, self.W[("norm", -1)], sh.eps))
        return matvec(self.W[("lm_head", -1)], hf)


def e4m3_table():
    """(value, code) of every finite non-negative E4M3 code, from the bit
    fields: code = e << 3 | m; e = 0: m * 2^-9; else (8 + m) * 2^(e - 10);
    e = 15, m = 7 is NaN."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            v = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
            out.append((v, (e << 3) | m))
    return out


def e4m3_nearest(y, table):
    """Code of the table value nearest to |y| (ties: even code), saturating,
    with the sign bit of y."""
    a = abs(y)
    best = None
    for v, c in table:
        d = abs(a - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    code = best[1]
    if a >= 448.0:
        code = 0x7E
    return code | (0x80 if math.copysign(1.0, y) < 0 else 0)
