"""Paged KV cache with sequences of different lengths ("万亿参数大模型在国产加速卡
上的Day-0适配教程", step 8: a paged KV cache, new requests joining a running
batch), through the C ABI.

Bars:
  * a batch of equal-length sequences gives bit-identical logits with the
    paged and the contiguous cache (the products and the attention
    arithmetic are the same; only where the rows live differs);
  * sequences of different lengths decoded together, and a sequence that
    joins after another is released, each match the oracle run on that
    sequence alone, under teacher forcing, with oracle.parity's bar (a
    sequence's results do not depend on the others in the batch);
  * an exhausted page pool is a state error that changes nothing.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import qwen2_decoder_forward_amd as q2
import synth
from tests.gpu_util import DEV
from tests.model_util import build_model

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.ModelShape("small-bf16", "bf16", 3, 256, 4, 2, 128, 512, 1000, 10000.0)


def _prompt(seed, n, vocab):
    return np.random.default_rng(seed).integers(0, vocab, n).astype(np.int64)


@pytest.mark.parametrize("B", [3, 20])
def test_paged_uniform_batch_equals_contiguous(B):
    """Equal-length sequences: the paged model's logits equal the contiguous
    model's bit for bit.  At 3 sequences the decode products are GEMVs, at 20
    the skinny split-K tiles; either way the QKV reduction writes the new k /
    v rows straight into their pages instead of the contiguous rows."""
    sh = SMALL_BF16
    w = synth.make_weights(sh, seed=41)
    prompts = torch.from_numpy(np.stack([_prompt(i, 70, sh.vocab) for i in range(B)])).to(DEV)
    mc = build_model(sh, w, 96, B)
    mp = q2.load_model(sh, w, 96, B, page_size=64)
    nc, lc = mc.prefill(prompts, logits=True)
    npg, lp = mp.prefill(prompts, logits=True)
    assert torch.equal(lc, lp) and torch.equal(nc, npg)
    feed = nc
    for _ in range(6):
        nc, lc = mc.decode(feed, logits=True)
        npg, lp = mp.decode(feed, logits=True)
        assert torch.equal(lc, lp) and torch.equal(nc, npg)
        feed = nc
    assert mp.seq_length(0) == 76 and mp.seq_length(B - 1) == 76
    mc.close()
    mp.close()


def _oracle_alone(sh, w, prompt, steps, max_seq, kv="model"):
    orc = oracle.OracleModel(sh, w, "bf16", 1, max_seq, kv=kv)
    orc64 = oracle.OracleModel(sh, w, "bf16", 1, max_seq, accum="f64", share_from=orc, kv=kv)
    return parity.reference(orc, prompt[None, :], steps, orc64)


def _ragged(kv_fp8, lens=(5, 70, 130), steps=8):
    sh = SMALL_BF16
    w = synth.make_weights(sh, seed=42)
    lens, max_seq = list(lens), max(lens) + steps + 22
    B = len(lens)
    prompts = [_prompt(10 + i, n, sh.vocab) for i, n in enumerate(lens)]
    refs = [_oracle_alone(sh, w, p, steps, max_seq, "fp8" if kv_fp8 else "model") for p in prompts]
    m = q2.load_model(sh, w, max_seq, B, kv_fp8=kv_fp8, page_size=64)
    got_l = [[] for _ in lens]
    got_t = [[] for _ in lens]
    for b, p in enumerate(prompts):
        nxt, lg = m.seq_prefill(b, torch.from_numpy(p).to(DEV), logits=True)
        got_l[b].append(lg.cpu().numpy())
        got_t[b].append(nxt.cpu().numpy())
    assert [m.seq_length(b) for b in range(B)] == lens
    for s in range(1, steps + 1):
        feed = torch.tensor([int(refs[b][0][0, s - 1]) for b in range(B)], dtype=torch.int64, device=DEV)
        nxt, lg = m.decode(feed, logits=True)
        lg, nxt = lg.cpu().numpy(), nxt.cpu().numpy()
        for b in range(B):
            got_l[b].append(lg[b:b + 1])
            got_t[b].append(nxt[b:b + 1])
    assert [m.seq_length(b) for b in range(B)] == [n + steps for n in lens]
    m.close()
    for b in range(B):
        toks, ref_logits, spread = refs[b]
        r = parity.compare(got_l[b], np.stack(got_t[b], axis=1), ref_logits, toks, spread, True)
        print(f"\n[paged{' fp8' if kv_fp8 else ''} ragged, sequence {b} (prompt {lens[b]})] {r.summary()}", flush=True)
        assert r.ok(), r.summary()


def test_paged_ragged_batch_matches_each_sequence_alone():
    _ragged(False)


def test_paged_fp8_ragged_batch_matches_each_sequence_alone():
    _ragged(True)


# 20 sequences of 3 to 193 cached positions (one to four pages): the decode
# products take the skinny split-K path, whose QKV reduction writes each new
# k / v row into its own sequence's page (and, FP8, quantises it there)
RAGGED_20 = tuple(3 + 10 * i for i in range(20))


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_paged_ragged_batch_20_matches_each_sequence_alone(kv_fp8):
    _ragged(kv_fp8, RAGGED_20, steps=5)


def test_paged_continuous_batching_release_and_join():
    """Three sequences decode together; after 4 steps sequence 1 is released
    and a new one (its own prompt) is prefilled into its slot; the three
    then decode 5 more steps.  Each sequence matches the oracle alone."""
    sh = SMALL_BF16
    w = synth.make_weights(sh, seed=43)
    max_seq = 128
    pa, pb, pc, pd = (_prompt(20 + i, n, sh.vocab) for i, n in enumerate([30, 90, 10, 50]))
    ra = _oracle_alone(sh, w, pa, 9, max_seq)
    rb = _oracle_alone(sh, w, pb, 4, max_seq)
    rc = _oracle_alone(sh, w, pc, 9, max_seq)
    rd = _oracle_alone(sh, w, pd, 5, max_seq)
    m = q2.load_model(sh, w, max_seq, 3, page_size=64)
    free0 = m.free_pages()
    seqs = {0: (pa, ra), 1: (pb, rb), 2: (pc, rc)}
    got = {k: ([], []) for k in "abcd"}
    name = {0: "a", 1: "b", 2: "c"}
    for slot, (p, _) in seqs.items():
        nxt, lg = m.seq_prefill(slot, torch.from_numpy(p).to(DEV), logits=True)
        got[name[slot]][0].append(lg.cpu().numpy())
        got[name[slot]][1].append(nxt.cpu().numpy())
    step_of = {0: 0, 1: 0, 2: 0}
    for phase in range(2):
        for _ in range(4 if phase == 0 else 5):
            feed = []
            for slot in range(3):
                ref = seqs[slot][1]
                feed.append(int(ref[0][0, step_of[slot]]))
            nxt, lg = m.decode(torch.tensor(feed, dtype=torch.int64, device=DEV), logits=True)
            lg, nxt = lg.cpu().numpy(), nxt.cpu().numpy()
            for slot in range(3):
                got[name[slot]][0].append(lg[slot:slot + 1])
                got[name[slot]][1].append(nxt[slot:slot + 1])
                step_of[slot] += 1
        if phase == 0:
            used = m.free_pages()
            m.seq_release(1)
            assert m.free_pages() == used + 2 and m.seq_length(1) == 0     # 94 positions: 2 pages back
            seqs[1] = (pd, rd)
            name[1] = "d"
            step_of[1] = 0
            nxt, lg = m.seq_prefill(1, torch.from_numpy(pd).to(DEV), logits=True)
            got["d"][0].append(lg.cpu().numpy())
            got["d"][1].append(nxt.cpu().numpy())
    assert m.seq_length(0) == 39 and m.seq_length(1) == 55 and m.seq_length(2) == 19
    m.reset()
    assert m.free_pages() == free0
    m.close()
    for key, ref in (("a", ra), ("b", rb), ("c", rc), ("d", rd)):
        toks, ref_logits, spread = ref
        gl, gt = got[key]
        r = parity.compare(gl, np.stack(gt, axis=1), ref_logits[:len(gl)], toks[:, :len(gl)], spread, True)
        print(f"\n[continuous batching, sequence {key}] {r.summary()}", flush=True)
        assert r.ok(), r.summary()


def test_paged_pool_exhaustion_is_state_error_and_changes_nothing():
    sh = SMALL_BF16
    w = synth.make_weights(sh, seed=44)
    m = q2.load_model(sh, w, 256, 2, page_size=64, kv_pages=3)
    m.seq_prefill(0, torch.from_numpy(_prompt(1, 130, sh.vocab)).to(DEV))
    assert m.free_pages() == 0
    with pytest.raises(q2.Q2Error) as e:
        m.seq_prefill(1, torch.from_numpy(_prompt(2, 10, sh.vocab)).to(DEV))
    assert e.value.name == "Q2_ESTATE"
    assert m.free_pages() == 0 and m.seq_length(1) == 0 and m.seq_length(0) == 130
    m.seq_release(0)
    assert m.free_pages() == 3
    m.seq_prefill(1, torch.from_numpy(_prompt(2, 10, sh.vocab)).to(DEV))
    assert m.free_pages() == 2 and m.seq_length(1) == 10
    torch.cuda.synchronize()
    m.close()


def test_paged_replay_stage_reserves_its_positions():
    """The measurement hook on a paged cache takes the pages of the positions
    it replays (it writes and reads them), and a forward after a reset is
    unchanged."""
    sh = SMALL_BF16
    w = synth.make_weights(sh, seed=45)
    m = q2.load_model(sh, w, 160, 2, page_size=64)
    ids = torch.from_numpy(np.stack([_prompt(5, 64, sh.vocab), _prompt(6, 64, sh.vocab)])).to(DEV)
    before = m.prefill(ids, logits=True)[1].cpu().numpy()
    free = m.free_pages()
    for stage in range(5):
        q2.q2_model_replay_stage(m.handle, stage, 2, 1, sh.nlayer)      # position 64: a new page each
    assert m.free_pages() == free - 2
    torch.cuda.synchronize()
    m.reset()
    after = m.prefill(ids, logits=True)[1].cpu().numpy()
    m.close()
    assert np.array_equal(before, after)
