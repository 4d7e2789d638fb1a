"""Helpers for model-level GPU tests and the benchmark: build a q2 model on
the GPU from the seeded synthetic weights, and compare it with the oracle
under teacher forcing."""
import dataclasses

import numpy as np
import torch

import oracle
import synth
from qwen2_decoder_forward_amd import Model

DEV = "cuda:0"


def to_device(arr: np.ndarray) -> torch.Tensor:
    """Upload a synthetic weight (uint16 bf16 bits or float32) bit-for-bit."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def build_model(shape, weights, max_seq, max_batch) -> Model:
    m = Model(shape, max_seq, max_batch)
    for (name, layer), arr in weights.items():
        t = to_device(arr)
        m.load_weight(name, layer, t)
        torch.cuda.synchronize()
        del t
    return m


def reduced_shape(shape, **kw):
    return dataclasses.replace(shape, **kw)


@dataclasses.dataclass
class TFResult:
    steps: int
    max_abs_err: float          # over all compared logits, after rounding both to bf16 (bf16 models)
    max_rel_err: float          # max |d| / max |ref| per step, worst step
    agreement: float            # fraction of positions whose argmax matches, all sequences
    cosine_min: float
    gpu_tokens: np.ndarray
    ref_tokens: np.ndarray
    spread: float = 0.0         # max |oracle(f32 accum) - oracle(f64 accum)| on the same inputs
    tol: float = 0.0            # the bound applied: max(2e-2, 2 * spread)
    decisive: int = 0           # positions whose oracle top-1 margin exceeds tol
    decisive_agreement: float = 1.0
    valid_picks: float = 1.0    # fraction of GPU picks within tol of the oracle maximum

    def summary(self):
        return (f"steps={self.steps} max_abs_err={self.max_abs_err:.3e} spread={self.spread:.3e} "
                f"tol={self.tol:.3e} agreement={self.agreement:.4f} decisive={self.decisive} "
                f"decisive_agreement={self.decisive_agreement:.4f} valid_picks={self.valid_picks:.4f} "
                f"max_rel_err={self.max_rel_err:.3e} cos_min={self.cosine_min:.6f}")

    def ok(self):
        return (self.max_abs_err <= self.tol and self.decisive_agreement >= 0.99 and self.valid_picks == 1.0)


def teacher_forced(model: Model, orc: oracle.OracleModel, prompt: np.ndarray, steps: int,
                   orc64: oracle.OracleModel | None = None) -> TFResult:
    """Oracle runs greedily; the GPU is fed the oracle's tokens; logits of the
    prefill and of every decode step are compared.

    With ``orc64`` (the same model summing in float64) the bf16 bound is
    derived from the reference itself: two exact implementations that differ
    only in summation rounding drift apart by ``spread`` after bf16 storage
    rounding, so the GPU must stay within max(2e-2, 2 * spread), pick the
    oracle's token wherever the oracle's top-1 margin exceeds that bound, and
    elsewhere pick a token whose oracle logit is within the bound of the max.
    """
    ref_toks, ref_logits = orc.generate(prompt, steps)
    spread = 0.0
    if orc64 is not None:
        _, l64 = orc64.generate(prompt, steps, teacher=ref_toks)
        for a, b in zip(ref_logits, l64):
            spread = max(spread, float(np.abs(oracle.bf16_round(a) - oracle.bf16_round(b)).max()))
    bf = orc.storage == "bf16"
    nxt, lg = model.prefill(torch.from_numpy(prompt).to(DEV), logits=True)
    gpu_logits = [lg.cpu().numpy()]
    gpu_toks = [nxt.cpu().numpy()]
    for s in range(1, steps + 1):
        feed = torch.from_numpy(np.ascontiguousarray(ref_toks[:, s - 1])).to(DEV)
        nxt, lg = model.decode(feed, logits=True)
        gpu_logits.append(lg.cpu().numpy())
        gpu_toks.append(nxt.cpu().numpy())
    max_abs = max_rel = 0.0
    cos_min = 1.0
    for g, r in zip(gpu_logits, ref_logits):
        if bf:
            g, r = oracle.bf16_round(g), oracle.bf16_round(r)
        d = np.abs(g.astype(np.float64) - r)
        max_abs = max(max_abs, float(d.max()))
        max_rel = max(max_rel, float(d.max() / np.abs(r).max()))
        for b in range(g.shape[0]):
            c = float(np.dot(g[b], r[b]) / (np.linalg.norm(g[b]) * np.linalg.norm(r[b])))
            cos_min = min(cos_min, c)
    gt = np.stack(gpu_toks, axis=1)
    agree = float(np.mean(gt == ref_toks))
    tol = max(2e-2, 2 * spread)
    dec = dec_ok = valid = total = 0
    for s_, r in enumerate(ref_logits):
        for b in range(r.shape[0]):
            top2 = np.partition(r[b], -2)[-2:]
            margin = float(top2[1] - top2[0])
            pick = int(gt[b, s_])
            total += 1
            valid += int(r[b, pick] >= r[b].max() - tol)
            if margin > tol:
                dec += 1
                dec_ok += int(pick == int(ref_toks[b, s_]))
    return TFResult(steps, max_abs, max_rel, agree, cos_min, gt, ref_toks, spread, tol, dec,
                    dec_ok / dec if dec else 1.0, valid / total)
