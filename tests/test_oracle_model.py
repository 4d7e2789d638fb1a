"""The oracle's whole-model forward against brute force and model invariants."""
import numpy as np
import pytest

import oracle
import synth
from tests import pins


def test_model_vs_brute_force():
    pins.check_model_vs_brute(oracle.OracleModel)


@pytest.mark.parametrize("storage", ["fp32", "bf16"])
def test_decode_equals_recompute(storage):
    pins.check_decode_equals_recompute(oracle.OracleModel, storage)


@pytest.mark.parametrize("storage", ["fp32", "bf16"])
def test_batch_independence(storage):
    pins.check_batch_independence(oracle.OracleModel, storage)


def test_zero_mixers_closed_form():
    pins.check_zero_mixers_closed_form(oracle.OracleModel)


def test_bf16_storage_close_to_fp32():
    """bf16 storage changes the logits by roughly the bf16 rounding level only."""
    sh = pins.tiny_shape(4)
    w = synth.make_weights(sh, seed=21)
    ids = np.array([[1, 5, 9, 13, 17, 21]], np.int64)
    a, _ = oracle.OracleModel(sh, w, "fp32", 1, 8).forward(ids)
    b, _ = oracle.OracleModel(sh, w, "bf16", 1, 8).forward(ids)
    rel = np.abs(a - b).max() / np.abs(a).max()
    assert 0 < rel < 3e-2


def test_capacity_exceeded_raises():
    sh = pins.tiny_shape()
    w = synth.make_weights(sh, seed=1)
    m = oracle.OracleModel(sh, w, "fp32", 1, 4)
    m.forward(np.array([[1, 2, 3]]))
    with pytest.raises(ValueError):
        m.forward(np.array([[1, 2]]))


def test_workload_a_runs():
    wl = synth.WORKLOADS["A"]
    w = synth.make_weights(wl)
    m = oracle.OracleModel(wl.shape, w, "fp32", wl.batch, wl.max_seq)
    toks, logits = m.generate(synth.make_prompt(wl), wl.steps)
    assert toks.shape == (1, wl.steps + 1) and len(logits) == wl.steps + 1
    assert m.length == wl.max_seq


def test_embeds_layers_hidden_options_compose():
    """forward(embeds=E[ids]) equals forward(ids); running layers [0, k) then
    [k, L) from the recorded hidden state equals the full stack."""
    sh = pins.tiny_shape(4)
    w = synth.make_weights(sh, seed=22)
    ids = np.array([[3, 9, 27, 1, 0]], np.int64)
    full = oracle.OracleModel(sh, w, "bf16", 1, 8)
    hs = []
    ref, _ = full.forward(ids, hidden=hs)
    assert len(hs) == sh.nlayer
    E = w[("embed_tokens", -1)]
    a, _ = oracle.OracleModel(sh, w, "bf16", 1, 8).forward(None, embeds=E[ids])
    assert np.array_equal(a, ref)
    part = oracle.OracleModel(sh, w, "bf16", 1, 8)
    h1 = []
    part.forward(ids, layers=range(0, 2), hidden=h1)
    rest = oracle.OracleModel(sh, w, "bf16", 1, 8)
    # the second half needs the first half's KV cache only for its own layers
    b, _ = rest.forward(None, embeds=h1[-1], layers=range(2, 4))
    assert np.array_equal(b, ref)


def test_f64_accumulation_is_close_in_fp32_storage():
    """In fp32 storage the two accumulation precisions agree to float32
    rounding level (the gap only opens through bf16 storage rounding)."""
    sh = pins.tiny_shape(3)
    w = synth.make_weights(sh, seed=23)
    ids = np.array([[1, 2, 3, 4]], np.int64)
    a, _ = oracle.OracleModel(sh, w, "fp32", 1, 8, accum="f32").forward(ids)
    b, _ = oracle.OracleModel(sh, w, "fp32", 1, 8, accum="f64").forward(ids)
    assert np.abs(a - b).max() <= 1e-5 * np.abs(a).max()


def test_bf16_writeback_points_are_bf16():
    """Every stored intermediate of the bf16 forward is a bf16 number, at the
    named storage points of the low-precision write-back rule."""
    pins.check_bf16_writeback_points(oracle.OracleModel)


def test_bf16_writeback_matches_loop_forward():
    """The bf16 forward against the loop-written bf16 forward that rounds at
    the same points (float64 sums): same stored values, same logits."""
    pins.check_bf16_writeback_vs_brute(oracle.OracleModel)


def test_fp8_cache_holds_quantised_rows():
    pins.check_fp8_cache_values(oracle.OracleModel)


def test_fp8_cache_decode_equals_recompute_and_batch_independence():
    """With the FP8 cache each row is quantised once, on its own block, so a
    decode step still equals the recompute of its prefix and a batched
    sequence equals the same sequence alone."""
    sh = synth.ModelShape("pin-fp8", "bf16", 2, 256, 4, 2, 128, 256, 64, 10000.0)
    w = synth.make_weights(sh, seed=34)
    prompts = np.array([[3, 1, 4, 1, 5], [9, 2, 6, 5, 3]], np.int64)
    mb = oracle.OracleModel(sh, w, "bf16", 2, 16, kv="fp8")
    toks, logits = mb.generate(prompts, 4)
    for b in range(2):
        ms = oracle.OracleModel(sh, w, "bf16", 1, 16, kv="fp8")
        ts, ls = ms.generate(prompts[b:b + 1], 4)
        assert np.array_equal(ts[0], toks[b])
        # float32 products of a different row count may sum in another order:
        # a bf16 flip moves a logit by a few 1e-3 at most at this size
        assert all(np.abs(a[0] - c[b]).max() <= 2e-2 for a, c in zip(ls, logits))
    full = np.concatenate([prompts[:1], toks[:1, :3]], axis=1)
    r = oracle.OracleModel(sh, w, "bf16", 1, 16, kv="fp8")
    lg, _ = r.forward(full)
    assert np.abs(lg[0] - logits[3][0]).max() <= 2e-2
