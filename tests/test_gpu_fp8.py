"""The FP8 KV cache ("新一代大模型Day0推理适配与性能调优教程", step 5: KV cache
in FP8 per token x head x 128-element block; verification by top-K overlap
before and after quantisation) on the GPU, through the C ABI.

Bars:
  * the codec (q2_kv_quantize / q2_kv_dequantize): codes, scales and
    dequantised values bit-exact against the oracle (the codes are integer
    decisions taken in float32 on both sides);
  * the model with an FP8 cache against the oracle with the same FP8 cache
    under teacher forcing: the bf16 bar of oracle.parity (the quantisation
    is part of the definition on both sides);
  * the cache contents: the first layer's dequantised rows equal the
    oracle's except where a bf16 flip of k or v upstream changed a block;
  * top-K overlap, the check the page asks for after quantising: the GPU's
    FP8-cache logits against its bf16-cache logits on the same tokens keep a
    top-10 overlap within 0.05 of what the oracle's own FP8 and bf16 caches
    give, and at least 0.8.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import qwen2_decoder_forward_amd as q2
import synth
from tests.gpu_util import DEV, down, up
from tests.model_util import build_model, gpu_teacher_forced, teacher_forced

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.ModelShape("small-bf16", "bf16", 3, 256, 4, 2, 128, 512, 1000, 10000.0)


def _bf16_blocks(seed, n):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((n, 128)) * np.exp(r.uniform(-8, 4, (n, 1)))).astype(np.float32)
    x = oracle.bf16_round(x)
    x[0] = 0.0
    x[1] = -0.0
    x[2, :] = 0.0
    x[2, 7] = 3.0                                          # one non-zero element
    x[3] = oracle.bf16_round(np.linspace(-448, 448, 128).astype(np.float32))
    x[4] = oracle.bf16_round((np.arange(128) - 64).astype(np.float32) * 2.0 ** -12)  # subnormal codes
    return x


def test_kv_quantize_bit_exact():
    x = _bf16_blocks(5, 333)
    codes = torch.empty(333, 128, dtype=torch.uint8, device=DEV)
    scales = torch.empty(333, dtype=torch.float32, device=DEV)
    q2.q2_kv_quantize(codes, scales, up(x, torch.bfloat16))
    rc, rs = oracle.kv_quantize(x)
    assert np.array_equal(down(scales), rs)
    got = codes.cpu().numpy()
    assert np.array_equal(got, rc), np.argwhere(got != rc)[:5]


def test_kv_dequantize_bit_exact_every_code():
    codes = np.concatenate([np.arange(0x7F), np.arange(0x80, 0xFF), np.zeros(2)]).astype(np.uint8).reshape(2, 128)
    codes = np.tile(codes, (3, 1))
    scales = np.array([1.0, 2.0 ** -10, 0.0123, 3.7, 1e-3, 1.0 / 448], np.float32)
    x = torch.empty(6, 128, dtype=torch.bfloat16, device=DEV)
    q2.q2_kv_dequantize(x, torch.from_numpy(codes).to(DEV), up(scales))
    want = oracle.kv_dequantize(codes, scales)
    got = down(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _fp8_run(shape, batch, prompt_len, steps, seed=1234):
    wl = synth.Workload("fp8", shape, batch, prompt_len, steps, seed, 5678)
    w = synth.make_weights(wl)
    prompt = synth.make_prompt(wl)
    orc = oracle.OracleModel(shape, w, "bf16", batch, wl.max_seq, kv="fp8")
    orc64 = oracle.OracleModel(shape, w, "bf16", batch, wl.max_seq, accum="f64", share_from=orc, kv="fp8")
    model = q2.load_model(shape, w, wl.max_seq, batch, kv_fp8=True)
    r = teacher_forced(model, orc, prompt, steps, orc64)
    return r, model, orc, w, prompt


def _check_layer0_cache(model, orc, batch, nkv, tag):
    """The first layer's cache -- GPU codes and scales, dequantised -- against
    the oracle's, over every cached position (prompt rows from the prefill's
    store, the rest from the decode steps' QKV reductions)."""
    k, v = model.kv_view(0)
    ks, vs = model.kv_scale_view(0)
    L0 = orc.length
    for name, cdesc, sdesc, ref in (("k", k, ks, orc.k_cache[0]), ("v", v, vs, orc.v_cache[0])):
        codes = torch.empty(batch, L0, nkv, 128, dtype=torch.uint8, device=DEV)
        c2 = q2.Q2Tensor.from_buffer_copy(cdesc)
        c2.shape[0], c2.shape[1] = batch, L0
        q2.q2_rearrange(codes, c2)
        sc = torch.empty(batch, L0, nkv, dtype=torch.float32, device=DEV)
        s2 = q2.Q2Tensor.from_buffer_copy(sdesc)
        s2.shape[0], s2.shape[1] = batch, L0
        q2.q2_rearrange(sc, s2)
        deq = torch.empty(batch * L0 * nkv, 128, dtype=torch.bfloat16, device=DEV)
        q2.q2_kv_dequantize(deq, codes.view(-1, 128), sc.view(-1))
        got = down(deq).reshape(batch, L0, nkv, 128).transpose(0, 2, 1, 3)
        want = ref[:, :, :L0, :]
        eq = float(np.mean(got == want))
        print(f"  [{tag}] layer-0 {name} cache rows equal to the oracle's: {eq:.4f}", flush=True)
        assert eq >= 0.99


def test_fp8_model_small_teacher_forced():
    r, model, orc, _, _ = _fp8_run(SMALL_BF16, 3, 40, 12)
    print(f"\n[fp8 small] {r.summary()}", flush=True)
    _check_layer0_cache(model, orc, 3, SMALL_BF16.nkv, "fp8 small")
    model.close()
    assert r.ok(), r.summary()


def test_fp8_model_batched_decode_1p5b_width():
    """1.5B layer shapes with 4 layers, 64 sequences, 96-token prompts, 4
    batched decode steps (the 64-sequence decode path with an FP8 cache,
    whose QKV split-K reduction quantises the new k / v rows itself)."""
    sh = dataclasses.replace(synth.SHAPES["1.5b"], nlayer=4)
    r, model, orc, _, _ = _fp8_run(sh, 64, 96, 4)
    print(f"\n[fp8 1.5B width, batch 64] {r.summary()}", flush=True)
    _check_layer0_cache(model, orc, 64, sh.nkv, "fp8 batch 64")
    model.close()
    assert r.ok(), r.summary()


def _topk_overlap(a_list, b_list, k=10):
    ov, agree = [], []
    for a, b in zip(a_list, b_list):
        for r in range(a.shape[0]):
            ia = set(np.argpartition(-a[r], k)[:k])
            ib = set(np.argpartition(-b[r], k)[:k])
            ov.append(len(ia & ib) / k)
            agree.append(int(np.argmax(a[r]) == np.argmax(b[r])))
    return float(np.mean(ov)), float(np.mean(agree))


def test_fp8_topk_overlap_against_bf16_cache():
    sh = dataclasses.replace(synth.SHAPES["1.5b"], nlayer=4)
    wl = synth.Workload("ov", sh, 2, 96, 8, 1234, 5678)
    w = synth.make_weights(wl)
    prompt = synth.make_prompt(wl)
    ob = oracle.OracleModel(sh, w, "bf16", 2, wl.max_seq)
    of = oracle.OracleModel(sh, w, "bf16", 2, wl.max_seq, kv="fp8", share_from=ob)
    toks, lb = ob.generate(prompt, wl.steps)
    _, lf = of.generate(prompt, wl.steps, teacher=toks)
    ref_ov, ref_top1 = _topk_overlap(lb, lf)
    gb = q2.load_model(sh, w, wl.max_seq, 2)
    glb, _ = gpu_teacher_forced(gb, prompt, toks, wl.steps)
    gb.close()
    gf = q2.load_model(sh, w, wl.max_seq, 2, kv_fp8=True)
    glf, _ = gpu_teacher_forced(gf, prompt, toks, wl.steps)
    gf.close()
    ov, top1 = _topk_overlap(glb, glf)
    print(f"\n[fp8 vs bf16 cache] top-10 overlap GPU {ov:.3f} oracle {ref_ov:.3f}; "
          f"top-1 agreement GPU {top1:.3f} oracle {ref_top1:.3f}", flush=True)
    assert ov >= 0.8 and ov >= ref_ov - 0.05
