"""Brute-force float64 Qwen2 forward for tiny shapes (pure Python loops).

An independent second reading of the same definition, written element by
element with explicit indices so that a transposed operand, a wrong head
mapping or a dropped term in the NumPy oracle shows up as a mismatch.  It
performs no bf16 rounding: it pins the oracle's "fp32" mode.
"""
import math


def _vec(a):
    return [float(v) for v in a]


def _mat(a):
    return [[float(v) for v in row] for row in a]


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
    def __init__(self, shape, weights):
        self.sh = shape
        self.W = {}
        for key, arr in weights.items():
            self.W[key] = _mat(arr) if arr.ndim == 2 else _vec(arr)
        self.K = [[[] for _ in range(shape.nkv)] for _ in range(shape.nlayer)]
        self.V = [[[] for _ in range(shape.nkv)] for _ in range(shape.nlayer)]
        self.pos = 0

    def step(self, token):
        """Process one token of a single sequence; returns its logits (list)."""
        sh = self.sh
        d, nh, nkv = sh.dh, sh.nh, sh.nkv
        grp = nh // nkv
        x = list(self.W[("embed_tokens", -1)][token])
        for l in range(sh.nlayer):
            W = lambda n: self.W[(n, l)]  # noqa: E731
            h = rmsnorm(x, W("input_layernorm"), sh.eps)
            q = matvec(W("q_proj.weight"), h, W("q_proj.bias"))
            k = matvec(W("k_proj.weight"), h, W("k_proj.bias"))
            v = matvec(W("v_proj.weight"), h, W("v_proj.bias"))
            for g in range(nkv):
                self.K[l][g].append(rope_head(k[g * d:(g + 1) * d], self.pos, sh.theta))
                self.V[l][g].append(v[g * d:(g + 1) * d])
            att = []
            for hh in range(nh):
                g = hh // grp
                qh = rope_head(q[hh * d:(hh + 1) * d], self.pos, sh.theta)
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
            a = matvec(W("o_proj.weight"), att)
            x = [x[i] + a[i] for i in range(len(x))]
            h2 = rmsnorm(x, W("post_attention_layernorm"), sh.eps)
            gt = matvec(W("gate_proj.weight"), h2)
            up = matvec(W("up_proj.weight"), h2)
            mm = [silu(gt[i]) * up[i] for i in range(len(gt))]
            dn = matvec(W("down_proj.weight"), mm)
            x = [x[i] + dn[i] for i in range(len(x))]
        self.pos += 1
        hf = rmsnorm(x, self.W[("norm", -1)], sh.eps)
        return matvec(self.W[("lm_head", -1)], hf)
