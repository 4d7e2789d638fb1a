"""The persistent decode kernel (one cooperative launch per step) against the
per-operator graph path and the oracle.

Both paths compute the same operator chain with the same bf16 rounding
points; only float32 summation order inside the products differs, so their
logits agree to a few bf16 ulps per step and the tokens agree wherever the
top-1 margin is not a near tie.  The oracle comparison applies the same bar as
the other model tests (tests/model_util.teacher_forced).  Every test ends with
q2_model_check, which fails if a grid barrier of the kernel timed out.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.model_util import DEV, build_model, reduced_shape, teacher_forced

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.ModelShape("small-bf16", "bf16", 3, 256, 4, 2, 128, 512, 1000, 10000.0)


def _paths_logits(model, prompt, steps, persistent):
    """Greedy decode on one path: logits [steps, B, V], the token fed at each
    step [steps, B] (the prefill's pick, then the path's own picks) and the
    token picked at each step."""
    model.reset()
    model.set_decode_path(persistent)
    ids = torch.from_numpy(prompt).to(DEV)
    nxt = model.prefill(ids)
    out, fed, toks = [], [], []
    cur = nxt.clone()
    for _ in range(steps):
        fed.append(cur.cpu().numpy())
        nxt, lg = model.decode(cur, logits=True)
        out.append(lg.float().cpu().numpy())
        toks.append(nxt.cpu().numpy())
        cur = nxt.clone()
    model.check()
    return np.stack(out), np.stack(fed), np.stack(toks)


def _forced_logits(model, prompt, forced, persistent):
    """Decode logits when fed the token stream `forced` [steps, B]."""
    model.reset()
    model.set_decode_path(persistent)
    ids = torch.from_numpy(prompt).to(DEV)
    model.prefill(ids)
    out = []
    for s in range(forced.shape[0]):
        _, lg = model.decode(torch.from_numpy(forced[s]).to(DEV), logits=True)
        out.append(lg.float().cpu().numpy())
    model.check()
    return np.stack(out)


@pytest.mark.parametrize("batch", [1, 3, 16])
def test_persistent_matches_graph_path_small(batch):
    wl = synth.Workload("t", SMALL_BF16, batch, 9, 12)
    w = synth.make_weights(wl)
    prompt = synth.make_prompt(wl)
    model = build_model(SMALL_BF16, w, wl.max_seq + 8, batch)
    model.set_decode_path(True)
    assert model.decode_path(batch)
    lg_g, fed_g, tok_g = _paths_logits(model, prompt, wl.steps, False)
    lg_p = _forced_logits(model, prompt, fed_g, True)
    d = np.abs(lg_p - lg_g).max()
    print(f"\n[persistent vs graph, small, B={batch}] max |dlogit| = {d:.3e}", flush=True)
    assert d <= 2e-2
    # same picks wherever the graph path's top-1 margin is not a near tie
    srt = np.sort(lg_g, axis=-1)
    margin = srt[..., -1] - srt[..., -2]
    pick_p = lg_p.argmax(-1)
    decisive = margin > 2 * d + 1e-6
    assert np.array_equal(pick_p[decisive], tok_g[decisive])
    model.close()


def test_persistent_against_oracle_small():
    wl = synth.Workload("t", SMALL_BF16, 2, 11, 14)
    w = synth.make_weights(wl)
    prompt = synth.make_prompt(wl)
    model = build_model(SMALL_BF16, w, wl.max_seq, 2)
    model.set_decode_path(True)
    orc = oracle.OracleModel(SMALL_BF16, w, "bf16", 2, wl.max_seq)
    orc64 = oracle.OracleModel(SMALL_BF16, w, "bf16", 2, wl.max_seq, accum="f64", share_from=orc)
    r = teacher_forced(model, orc, prompt, wl.steps, orc64)
    model.check()
    print(f"\n[persistent small vs oracle] {r.summary()}", flush=True)
    assert r.ok(), r.summary()
    model.close()


def test_persistent_full_width_two_layers():
    """The 1.5B layer shapes (H 1536, I 8960, V 151936) with two layers: the
    persistent path against the oracle, and against the graph path within the
    same derived bound (two correct bf16-storage forwards that differ only in
    summation order differ by up to the oracle's float32/float64 spread)."""
    shape = reduced_shape(synth.SHAPES["1.5b"], nlayer=2)
    wl = synth.Workload("t", shape, 1, 20, 6)
    w = synth.make_weights(wl)
    prompt = synth.make_prompt(wl)
    model = build_model(shape, w, wl.max_seq + 4, 1)
    model.set_decode_path(True)
    assert model.decode_path(1)
    orc = oracle.OracleModel(shape, w, "bf16", 1, wl.max_seq + 4)
    orc64 = oracle.OracleModel(shape, w, "bf16", 1, wl.max_seq + 4, accum="f64", share_from=orc)
    model.set_decode_path(True)
    r = teacher_forced(model, orc, prompt, wl.steps, orc64)
    model.check()
    print(f"\n[persistent 1.5B width vs oracle] {r.summary()}", flush=True)
    assert r.ok(), r.summary()
    lg_g, fed_g, tok_g = _paths_logits(model, prompt, wl.steps, False)
    lg_p = _forced_logits(model, prompt, fed_g, True)
    d = np.abs(lg_p - lg_g).max()
    print(f"[persistent vs graph, 1.5B width, 2 layers] max |dlogit| = {d:.3e} (bound {r.tol:.3e})", flush=True)
    assert d <= r.tol
    model.close()


def test_persistent_generate_continue_history():
    """generate + continue on the persistent path return the same token
    history as the graph path (greedy, small model, batch 2)."""
    wl = synth.Workload("t", SMALL_BF16, 2, 7, 10)
    w = synth.make_weights(wl)
    prompt = torch.from_numpy(synth.make_prompt(wl)).to(DEV)
    model = build_model(SMALL_BF16, w, wl.max_seq + 6, 2)
    outs = []
    for pers in (False, True):
        model.reset()
        model.set_decode_path(pers)
        a = model.generate(prompt, 4)
        b = torch.empty(prompt.shape[0], 6, dtype=torch.int64, device=DEV)
        model.continue_(6, b)
        torch.cuda.synchronize()
        outs.append((a.cpu().numpy(), b.cpu().numpy()))
    model.check()
    print(f"\n[generate/continue] graph {outs[0][1][0][:6]} persistent {outs[1][1][0][:6]}", flush=True)
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])
    model.close()


def test_persistent_workload_b_full_depth_teacher_forced():
    """The 28-layer 1.5B model (prompt 64, 32 decode steps) on the persistent
    path, teacher-forced against the oracle with the same bar as the graph
    path's full-workload test."""
    wl = synth.Workload("b-depth", synth.WORKLOADS["B"].shape, 1, 64, 32)
    w = synth.make_weights(wl)
    prompt = synth.make_prompt(wl)
    model = build_model(wl.shape, w, wl.max_seq, 1)
    model.set_decode_path(True)
    assert model.decode_path(1)
    orc = oracle.OracleModel(wl.shape, w, "bf16", 1, wl.max_seq)
    orc64 = oracle.OracleModel(wl.shape, w, "bf16", 1, wl.max_seq, accum="f64", share_from=orc)
    r = teacher_forced(model, orc, prompt, wl.steps, orc64)
    model.check()
    model.close()
    print(f"\n[persistent, full workload B] {r.summary()}", flush=True)
    assert r.ok(), r.summary()
