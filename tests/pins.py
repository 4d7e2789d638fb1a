"""Pin checks for the oracle operators, written against closed forms,
invariants and brute force rather than against the oracle itself.

Each ``check_*`` takes the implementation under test as an argument, so the
same check pins the real oracle (tests/test_oracle_ops.py) and is shown to
reject planted mistakes (tests/test_oracle_mutations.py).  Each raises
AssertionError on failure.
"""
import math

import numpy as np

from tests import _brute


def check_bf16_round(bf16_round):
    one = np.float32(1.0)
    # exact ties go to the even neighbour
    assert bf16_round(np.array([1 + 2.0 ** -8], np.float32))[0] == one
    assert bf16_round(np.array([1 + 3 * 2.0 ** -8], np.float32))[0] == np.float32(1 + 2.0 ** -6)
    # just above a tie rounds up, just below rounds down
    assert bf16_round(np.array([1 + 2.0 ** -8 + 2.0 ** -20], np.float32))[0] == np.float32(1 + 2.0 ** -7)
    assert bf16_round(np.array([1 + 2.0 ** -8 - 2.0 ** -20], np.float32))[0] == one
    # negative values round symmetrically
    assert bf16_round(np.array([-(1 + 3 * 2.0 ** -8)], np.float32))[0] == np.float32(-(1 + 2.0 ** -6))
    # representable values are fixed points, infinities are kept
    rep = np.array([0.0, -0.0, 1.0, -2.0, 0.5, 3.0, 2.0 ** -100, np.inf, -np.inf], np.float32)
    assert np.array_equal(bf16_round(rep), rep)
    # random sample: low 16 bits cleared, result is the nearer of the two bf16 neighbours
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    r = bf16_round(x)
    assert np.all(r.view(np.uint32) & 0xFFFF == 0)
    x64 = x.astype(np.float64)
    lo = (x.view(np.uint32) & 0xFFFF0000).view(np.float32).astype(np.float64)   # toward zero
    ulp = 2.0 ** (np.floor(np.log2(np.abs(lo))) - 7)
    hi = lo + np.sign(lo) * ulp                                                # away from zero
    r64 = r.astype(np.float64)
    assert np.all((r64 == lo) | (r64 == hi))
    other = np.where(r64 == lo, hi, lo)
    assert np.all(np.abs(r64 - x64) <= np.abs(other - x64))


def check_widen(widen):
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0000, 0x3F00], np.uint16)
    assert widen(bits).tolist() == [1.0, -2.0, math.inf, 0.0, 0.5]


def check_embedding(embedding):
    V, H = 50, 12
    table = np.zeros((V, H), np.float32)
    table[:, 0] = np.arange(V)                     # each row encodes its own index
    table[:, 1:] = (np.arange(V)[:, None] * 1000 + np.arange(1, H)[None, :])
    ids = np.array([0, 49, 7, 7, 3, 49, 0], np.int64)
    out = embedding(ids, table)
    assert out.shape == (len(ids), H)
    assert out[:, 0].astype(np.int64).tolist() == ids.tolist()
    assert np.all(out[:, 1:] == ids[:, None] * 1000 + np.arange(1, H)[None, :])
    for bad in ([-1], [V]):
        try:
            embedding(np.array(bad), table)
        except IndexError:
            pass
        else:
            raise AssertionError("out-of-range id accepted")


def check_rms_norm(rms_norm):
    eps = 1e-6
    # closed form on a constant vector: y = c / sqrt(c^2 + eps) * w
    H = 64
    w = np.linspace(0.5, 1.5, H).astype(np.float32)
    for c in (3.0, -0.25, 1e-4):
        y = rms_norm(np.full((1, H), c, np.float32), w, eps)
        ref = c / math.sqrt(c * c + eps) * w.astype(np.float64)
        assert np.allclose(y[0], ref, rtol=2e-6, atol=0)
    # output RMS with w = 1 is sqrt(ms / (ms + eps)) (epsilon inside the root)
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((8, H)) * 1e-3).astype(np.float32)
    y = rms_norm(x, np.ones(H, np.float32), eps)
    ms = np.mean(x.astype(np.float64) ** 2, axis=-1)
    assert np.allclose(np.sqrt(np.mean(y.astype(np.float64) ** 2, axis=-1)), np.sqrt(ms / (ms + eps)), rtol=1e-5)
    # scale invariance away from eps
    x = rng.standard_normal((4, H)).astype(np.float32)
    assert np.allclose(rms_norm(x * 8, w, eps), rms_norm(x, w, eps), rtol=1e-5, atol=1e-6)
    # brute force
    for r in range(4):
        ref = _brute.rmsnorm(x[r].tolist(), w.tolist(), eps)
        assert np.allclose(rms_norm(x[r:r + 1], w, eps)[0], ref, rtol=1e-5, atol=1e-6)


def check_rope(rope, rope_cos_sin):
    theta = 10000.0
    rng = np.random.default_rng(2)
    T, h, d = 6, 3, 16
    x = rng.standard_normal((T, h, d)).astype(np.float32)
    # position 0 is the identity
    assert np.array_equal(rope(x[:1], np.array([0]), theta), x[:1])
    # unit vector e_0 at position p lands on cos at index 0 and sin at index d/2 (rotate-half)
    e0 = np.zeros((1, 1, d), np.float32)
    e0[0, 0, 0] = 1
    for p in (1, 5, 1000):
        y = rope(e0, np.array([p]), theta)[0, 0]
        ref = np.zeros(d)
        ref[0], ref[d // 2] = math.cos(p), math.sin(p)
        assert np.allclose(y, ref, atol=1e-6), (p, y)
    # second frequency: e_1 rotates by p * theta^(-2/d) into index 1 + d/2
    e1 = np.zeros((1, 1, d), np.float32)
    e1[0, 0, 1] = 1
    y = rope(e1, np.array([7]), theta)[0, 0]
    ang = 7 * theta ** (-2.0 / d)
    assert abs(y[1] - math.cos(ang)) < 1e-6 and abs(y[1 + d // 2] - math.sin(ang)) < 1e-6
    assert abs(np.sum(np.abs(y)) - abs(math.cos(ang)) - abs(math.sin(ang))) < 1e-6
    # pair norms preserved
    pos = np.array([3, 17, 100, 4095, 0, 9])
    y = rope(x, pos, theta)
    n_in = x[..., :d // 2] ** 2 + x[..., d // 2:] ** 2
    n_out = y[..., :d // 2] ** 2 + y[..., d // 2:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-5, atol=1e-6)
    # R(m) R(n) = R(m + n)
    one = rope(rope(x[:1], np.array([13]), theta), np.array([29]), theta)
    assert np.allclose(one, rope(x[:1], np.array([42]), theta), atol=2e-5)
    # <R(m) q, R(n) k> depends on m - n only
    q, k = x[0:1, 0:1], x[1:2, 0:1]
    dots = [float(np.sum(rope(q, np.array([m]), theta) * rope(k, np.array([m - 5]), theta)))
            for m in (5, 50, 700)]
    assert max(dots) - min(dots) < 1e-4
    # brute force (fp64 angles)
    for t in range(T):
        for hh in range(h):
            ref = _brute.rope_head(x[t, hh].tolist(), int(pos[t]), theta)
            assert np.allclose(y[t, hh], ref, atol=1e-5)
    # table at position 0 and a hand value
    c, s = rope_cos_sin(np.array([0, 2]), 4, 10000.0)
    assert np.all(c[0] == 1) and np.all(s[0] == 0)
    assert abs(c[1, 1] - math.cos(2 * 0.01)) < 1e-7 and abs(s[1, 1] - math.sin(0.02)) < 1e-7


def check_linear(linear):
    rng = np.random.default_rng(3)
    M, K, N = 5, 7, 6
    x = rng.standard_normal((M, K)).astype(np.float32)
    W = rng.standard_normal((N, K)).astype(np.float32)       # [out, in]
    b = rng.standard_normal(N).astype(np.float32)
    y = linear(x, W, b)
    assert y.shape == (M, N)
    for m in range(M):
        assert np.allclose(y[m], _brute.matvec(W.tolist(), x[m].tolist(), b.tolist()), rtol=1e-5, atol=1e-5)
    assert np.allclose(linear(x, W), y - b, atol=1e-5)
    assert np.array_equal(linear(x, np.zeros_like(W), b), np.broadcast_to(b, (M, N)))
    eye = np.eye(K, dtype=np.float32)
    assert np.array_equal(linear(eye, W), W.T)                # one-hot input selects column k of W


def check_attention(attention):
    rng = np.random.default_rng(4)
    # probabilities: V = identity over keys returns the probability rows
    T, S, d = 5, 9, 16
    q = rng.standard_normal((T, 2, d)).astype(np.float32)
    k = rng.standard_normal((S, 1, d)).astype(np.float32)
    v = np.zeros((S, 1, d), np.float32)
    v[np.arange(S), 0, np.arange(S)] = 1
    p = attention(q, k, v, 1 / math.sqrt(d))
    past = S - T
    for t in range(T):
        for h in range(2):
            row = p[t, h, :S]
            assert abs(row.sum() - 1) < 1e-6
            assert np.all(row[past + t + 1:] == 0)            # masked keys contribute exactly 0
            assert np.all(row[:past + t + 1] > 0)
            # softmax of the visible scores, computed in float64
            sc = k[:past + t + 1, 0].astype(np.float64) @ q[t, h].astype(np.float64) / math.sqrt(d)
            e = np.exp(sc - sc.max())
            assert np.allclose(row[:past + t + 1], e / e.sum(), atol=1e-6)
    # fresh sequence: query 0 returns v_0 exactly
    T = S = 4
    q = rng.standard_normal((T, 4, d)).astype(np.float32)
    k = rng.standard_normal((S, 2, d)).astype(np.float32)
    v = rng.standard_normal((S, 2, d)).astype(np.float32)
    o = attention(q, k, v, 0.25)
    assert np.array_equal(o[0, 0], v[0, 0]) and np.array_equal(o[0, 3], v[0, 1])
    # future keys/values do not change earlier outputs
    k2, v2 = k.copy(), v.copy()
    k2[3] += 5
    v2[3] -= 7
    o2 = attention(q, k2, v2, 0.25)
    assert np.array_equal(o2[:3], o[:3]) and not np.allclose(o2[3], o[3])
    # GQA equals MHA with repeated KV heads (contiguous groups: head h reads h // 2)
    krep = np.repeat(k, 2, axis=1)
    vrep = np.repeat(v, 2, axis=1)
    assert np.allclose(attention(q, krep, vrep, 0.25), o, atol=1e-6)
    # brute force in fp64
    for t in range(T):
        for h in range(4):
            g = h // 2
            sc = [float(q[t, h] @ k[j, g]) * 0.25 for j in range(t + 1)]
            m = max(sc)
            e = [math.exp(s - m) for s in sc]
            ref = sum(e[j] / sum(e) * v[j, g].astype(np.float64) for j in range(t + 1))
            assert np.allclose(o[t, h], ref, atol=1e-5)


def check_silu_swiglu(silu, swiglu):
    assert silu(np.array([0.0], np.float32))[0] == 0
    ref = {1.0: 1 / (1 + math.exp(-1)), -1.0: -1 / (1 + math.exp(1)), 2.0: 2 / (1 + math.exp(-2))}
    for g, r in ref.items():
        assert abs(silu(np.array([g], np.float32))[0] - r) < 1e-6
    big = silu(np.array([30.0, -30.0, -200.0], np.float32))
    assert abs(big[0] - 30) < 1e-5 and abs(big[1]) < 1e-10 and big[2] == 0
    g = np.linspace(-6, 6, 25).astype(np.float32)
    assert np.array_equal(swiglu(g, np.ones_like(g)), silu(g))
    u = np.linspace(2, -3, 25).astype(np.float32)
    assert np.allclose(swiglu(g, u), [_brute.silu(float(a)) * float(b) for a, b in zip(g, u)], atol=1e-6)


def check_argmax(argmax):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 300)).astype(np.float32)
    x[1, [10, 200]] = 9.0               # planted tie: lowest index wins
    x[2, :] = 0.0                       # all equal: index 0
    x[3, 299] = 50.0                    # maximum at the last index
    idx, val = argmax(x)
    for r in range(x.shape[0]):
        best = 0
        for j in range(1, x.shape[1]):
            if x[r, j] > x[r, best]:
                best = j
        assert idx[r] == best and val[r] == x[r, best]
    assert idx[1] == 10 and idx[2] == 0 and idx[3] == 299


# ----------------------------------------------------------------------------- model

def tiny_shape(nlayer=2, eps=1e-2):
    """A small Qwen2-like shape.  The large epsilon makes its position visible
    at model level (with 1e-6 it only shows at the operator level)."""
    from synth import ModelShape
    return ModelShape("pin-tiny", "f32", nlayer, 16, 4, 2, 4, 24, 40, 10000.0, eps)


def check_model_vs_brute(model_cls, ops_module=None):
    """fp32-mode oracle against the fp64 loop forward: prompt of 5, then 3 decode steps."""
    import synth
    sh = tiny_shape()
    w = synth.make_weights(sh, seed=11)
    # larger weights than N(0, 0.02) so that every term matters at fp32 tolerance
    w = {k: (v * 20 if k[0] not in ("norm", "input_layernorm", "post_attention_layernorm") else v)
         for k, v in w.items()}
    prompt = np.array([[3, 17, 39, 0, 22]], np.int64)
    m = model_cls(sh, w, "fp32", 1, 16)
    logits, nxt = m.forward(prompt, all_logits=True)
    brute = _brute.BruteModel(sh, w)
    for t in range(prompt.shape[1]):
        ref = brute.step(int(prompt[0, t]))
        assert np.allclose(logits[0, t], ref, rtol=1e-4, atol=1e-4), t
    assert nxt[0] == int(np.argmax(ref))
    tok = int(nxt[0])
    for _ in range(3):
        lg, nx = m.forward(np.array([[tok]]))
        ref = brute.step(tok)
        assert np.allclose(lg[0], ref, rtol=1e-4, atol=1e-4)
        tok = int(nx[0])


def check_decode_equals_recompute(model_cls, storage):
    import synth
    sh = tiny_shape(3)
    w = synth.make_weights(sh, seed=12)
    if storage == "fp32":
        w = {k: v for k, v in w.items()}
    prompt = np.array([[5, 6, 7, 8, 9, 10]], np.int64)
    m = model_cls(sh, w, storage, 1, 32)
    toks, logits = m.generate(prompt, 6)
    for s in range(1, 7):
        full = np.concatenate([prompt, toks[:, :s]], axis=1)
        r = model_cls(sh, w, storage, 1, 32)
        lg, nx = r.forward(full)
        tol = 1e-5 if storage == "fp32" else 2e-2
        assert np.allclose(lg, logits[s], atol=tol, rtol=0), (s, np.abs(lg - logits[s]).max())


def check_batch_independence(model_cls, storage):
    import synth
    sh = tiny_shape()
    w = synth.make_weights(sh, seed=13)
    a = np.array([[1, 2, 3, 4]], np.int64)
    b = np.array([[30, 20, 10, 0]], np.int64)
    mb = model_cls(sh, w, storage, 2, 16)
    tb, lb = mb.generate(np.concatenate([a, b]), 3)
    for i, p in enumerate((a, b)):
        ms = model_cls(sh, w, storage, 1, 16)
        ts, ls = ms.generate(p, 3)
        assert np.array_equal(ts[0], tb[i])
        for s in range(4):
            assert np.allclose(ls[s][0], lb[s][i], atol=1e-5)


def check_zero_mixers_closed_form(model_cls):
    """With every o_proj and down weight zero the residual stream stays E[id],
    so the logits reduce to rmsnorm(E[id], w_f) W_lm^T at every position."""
    import synth
    sh = tiny_shape()
    w = synth.make_weights(sh, seed=14)
    for l in range(sh.nlayer):
        w[("o_proj.weight", l)] = np.zeros_like(w[("o_proj.weight", l)])
        w[("down_proj.weight", l)] = np.zeros_like(w[("down_proj.weight", l)])
    ids = np.array([[7, 0, 39, 12]], np.int64)
    m = model_cls(sh, w, "fp32", 1, 8)
    logits, _ = m.forward(ids, all_logits=True)
    E = w[("embed_tokens", -1)].astype(np.float64)
    wf = w[("norm", -1)].astype(np.float64)
    Wl = w[("lm_head", -1)].astype(np.float64)
    for t in range(ids.shape[1]):
        e = E[ids[0, t]]
        hf = e / np.sqrt(np.mean(e * e) + sh.eps) * wf
        assert np.allclose(logits[0, t], Wl @ hf, rtol=1e-5, atol=1e-6)


# ----------------------------------------------------------------------------- bf16 write-back points

# The storage points of the bf16 forward, in the order one layer stores them
# (plus the embedding row before the layers and the final norm after them).
BF16_POINTS = ("embed", "attn_norm", "q", "k", "v", "k_rope", "q_rope", "attn", "o_proj", "resid_attn",
               "mlp_norm", "gate", "up", "swiglu", "down", "resid_mlp", "final_norm")
LAYER_POINTS = BF16_POINTS[1:-1]


def tiny_bf16_shape(nlayer=2):
    from synth import ModelShape
    return ModelShape("pin-tiny-bf16", "bf16", nlayer, 32, 4, 2, 8, 48, 64, 10000.0, 1e-6)


def _oracle_points(rec, shape, calls):
    """Oracle record -> {point: float64 array [tokens, layers, n]} (one sequence)."""
    L = shape.nlayer
    out = {}
    for p, entries in rec.items():
        if p in ("embed", "final_norm"):
            rows = [np.asarray(e, np.float64).reshape(-1, np.asarray(e).shape[-1]) for e in entries]
            out[p] = np.concatenate(rows)[:, None, :]
            continue
        per_call = []
        i = 0
        for T in calls:
            layers = []
            for _ in range(L):
                layers.append(np.asarray(entries[i], np.float64).reshape(T, -1))
                i += 1
            per_call.append(np.stack(layers, axis=1))
        out[p] = np.concatenate(per_call)
    return out


def _brute_points(rec, shape):
    L = shape.nlayer
    out = {}
    for p, entries in rec.items():
        a = np.asarray(entries, np.float64)
        out[p] = a[:, None, :] if p in ("embed", "final_norm") else a.reshape(-1, L, a.shape[-1])
    return out


def run_bf16_writeback(model_cls):
    """Run the bf16-storage model and the loop-written bf16 forward on the
    same tiny input (a 5-token prefill, then 3 decode steps); return both
    point records and both logit sequences."""
    import synth
    sh = tiny_bf16_shape()
    w = synth.make_weights(sh, seed=31)
    # q and k weights and biases scaled by 16 (exact on bf16 bit patterns: the
    # exponent field grows by 4) so that the scores spread over several units
    # and the softmax is sensitive to the rounding of q and k
    for l in range(sh.nlayer):
        for n in ("q_proj.weight", "q_proj.bias", "k_proj.weight", "k_proj.bias"):
            b = w[(n, l)]
            nz = (b & np.uint16(0x7FFF)) != 0
            w[(n, l)] = np.where(nz, b + np.uint16(4 << 7), b).astype(np.uint16)
    prompt = np.array([[3, 17, 39, 0, 22]], np.int64)
    m = model_cls(sh, w, "bf16", 1, 16)
    m.record = {}
    logits, nxt = m.forward(prompt, all_logits=True)
    got_logits = [logits[0, t] for t in range(prompt.shape[1])]
    brute = _brute.BruteModel(sh, w, bf16_storage=True)
    ref_logits = [brute.step(int(t)) for t in prompt[0]]
    calls = [prompt.shape[1]]
    tok = int(nxt[0])
    for _ in range(3):
        lg, nx = m.forward(np.array([[tok]]))
        got_logits.append(lg[0])
        ref_logits.append(brute.step(tok))
        calls.append(1)
        tok = int(nx[0])
    return (_oracle_points(m.record, sh, calls), _brute_points(brute.record, sh),
            np.array(got_logits, np.float64), np.array(ref_logits, np.float64))


def check_bf16_writeback_points(model_cls):
    """Every stored intermediate of the bf16 forward is a bf16 number, at
    exactly the storage points of the low-precision write-back rule."""
    got, _, logits, _ = run_bf16_writeback(model_cls)
    assert set(got) == set(BF16_POINTS), sorted(set(got) ^ set(BF16_POINTS))
    for p, a in got.items():
        a32 = a.astype(np.float32)
        assert np.array_equal(a32.astype(np.float64), a), p
        assert not (a32.view(np.uint32) & np.uint32(0xFFFF)).any(), f"{p}: not a bf16 value"
    # the logits are float32 results, not bf16
    assert (logits.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF)).any()


def check_bf16_writeback_vs_brute(model_cls, min_equal=0.99, logit_rel=1e-5):
    """The bf16-storage model against the loop-written bf16 forward: the two
    round at the same points, so they store the same bf16 numbers except
    where a float32 and a float64 sum straddle a rounding boundary (none do
    at this size and seed; ``min_equal`` leaves room for one), and their
    logits then differ only by float32 summation rounding.  A rounding point
    dropped or added anywhere flips a large share of the later stored values
    and moves the logits by about a bf16 step (~1e-3 relative)."""
    got, ref, lg, lr = run_bf16_writeback(model_cls)
    assert set(got) == set(ref), sorted(set(got) ^ set(ref))
    for p in BF16_POINTS:
        assert got[p].shape == ref[p].shape, (p, got[p].shape, ref[p].shape)
        eq = float(np.mean(got[p] == ref[p]))
        # a flip is one bf16 step of that value
        rel = np.abs(got[p] - ref[p]) / np.maximum(np.abs(ref[p]), 1e-30)
        assert eq >= min_equal, f"{p}: only {eq:.4f} of stored values equal"
        assert float(rel.max()) <= 2 ** -7 + 1e-12, f"{p}: differs by {rel.max():.3e} relative"
    assert np.abs(lg - lr).max() <= logit_rel * np.abs(lr).max(), np.abs(lg - lr).max() / np.abs(lr).max()


# ----------------------------------------------------------------------------- FP8 KV cache

def check_e4m3(values, encode, decode):
    """The E4M3 table and codec against the loop-written enumeration, closed
    forms and a brute-force nearest search."""
    table = _brute.e4m3_table()
    v = values()
    assert len(v) == 127 and np.array_equal(v, np.array([t[0] for t in table])), "value table"
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    # every value round-trips, both signs
    codes = np.arange(0x7F, dtype=np.uint8)
    assert np.array_equal(encode(v.astype(np.float32)), codes)
    assert np.array_equal(encode(-v.astype(np.float32))[1:], codes[1:] | 0x80)
    assert np.array_equal(decode(codes).astype(np.float64), v)
    # closed-form ties (to even), saturation, signed zero
    ys = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, 460.0, 1e9, -0.0, 0.0, -2.0 ** -12],
                  np.float32)
    assert encode(ys).tolist() == [0x38, 0x3A, 0x00, 0x02, 0x7E, 0x7E, 0x7E, 0x80, 0x00, 0x80]
    # brute force on random magnitudes spanning the subnormals to saturation
    r = np.random.default_rng(41)
    y = (np.exp(r.uniform(np.log(2.0 ** -12), np.log(500.0), 3000)) * r.choice([-1, 1], 3000)).astype(np.float32)
    # plus exact midpoints between neighbouring codes
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    y = np.concatenate([y, mids[(mids.astype(np.float64) == (v[1:] + v[:-1]) / 2)]])
    got = encode(y)
    want = np.array([_brute.e4m3_nearest(float(t), table) for t in y], np.uint8)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:5]


def check_kv_quant(quantize, dequantize):
    """Block quantisation: the block maximum codes to +-448, the round trip
    is within half an E4M3 step of each value plus the bf16 write-back,
    zero blocks stay zero."""
    r = np.random.default_rng(42)
    x = (r.standard_normal((64, 128)) * np.exp(r.uniform(-6, 3, (64, 1)))).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)      # bf16 values
    x[5] = 0.0
    x[6, :] = -0.0
    x[7, 3] = 1e-3
    codes, scales = quantize(x)
    assert codes.dtype == np.uint8 and codes.shape == (64, 128) and scales.shape == (64,)
    amax = np.abs(x).max(-1)
    nz = amax > 0
    assert np.array_equal(scales[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    assert np.all(scales[~nz] == 0) and np.all(codes[5] == 0) and np.all(codes[6] == 0x80)
    top = np.abs(x).argmax(-1)
    assert np.all((codes[np.arange(64), top][nz] & 0x7F) == 0x7E)
    d = dequantize(codes, scales).astype(np.float64)
    assert np.all(d[~nz] == 0)
    # half a step: 2^-4 relative for normal codes, 2^-10 * scale absolute below 2^-6 * scale
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scales[:, None]) * (1 + 2 ** -7) + np.abs(x) * 2 ** -8
    assert np.all(np.abs(d - x) <= bound)


def check_fp8_cache_values(model_cls):
    """The FP8-cache model's cache holds, for every new k (after RoPE) and v
    row, bf16(value(code) * scale) with scale = max|block| / 448 and the code
    of each element found by brute-force nearest search (tests/_brute.py)."""
    import synth
    sh = synth.ModelShape("pin-fp8", "bf16", 2, 256, 4, 2, 128, 256, 64, 10000.0)
    w = synth.make_weights(sh, seed=33)
    m = model_cls(sh, w, "bf16", 1, 8, kv="fp8")
    m.record = {}
    m.forward(np.array([[1, 5, 9, 2]], np.int64))
    table = _brute.e4m3_table()
    value = {c: v for v, c in table}
    for l in range(sh.nlayer):
        for name, cache in (("k_rope", m.k_cache[l]), ("v", m.v_cache[l])):
            src = np.asarray(m.record[name][l], np.float32).reshape(4, sh.nkv, 128)
            got = cache[0, :, :4, :].transpose(1, 0, 2)
            for t in range(4):
                for h in range(sh.nkv):
                    x = src[t, h]
                    scale = np.float32(np.abs(x).max()) / np.float32(448)
                    y = (x / scale).astype(np.float32)
                    for i in range(0, 128, 7):
                        c = _brute.e4m3_nearest(float(y[i]), table)
                        v = value[c & 0x7F] * (-1 if c & 0x80 else 1)
                        prod = np.float32(np.float32(v) * scale)
                        want = (np.array([prod], np.float32).view(np.uint32) + 0x7FFF +
                                ((np.array([prod], np.float32).view(np.uint32) >> 16) & 1)) >> 16 << 16
                        assert got[t, h, i] == want.astype(np.uint32).view(np.float32)[0], (l, name, t, h, i)
