"""Comparison of a forward's logits with the oracle's under teacher forcing.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It takes the other
side's logits and tokens as plain arrays; it never runs or imports the GPU
library.

Method ("万亿参数大模型在国产加速卡上的Day-0适配教程", step 6: fix a
device-independent float32 reference, feed both sides the same inputs,
compare by maximum absolute error and cosine similarity, and require the
error not to grow with depth; "LLAISYS 训练营结项报告", section 3.5: the
generated tokens must match the reference's):

  * the oracle decodes greedily; the other side is fed the oracle's tokens
    (teacher forcing), so every step is compared on the same context;
  * ``spread``: the same oracle summing its products in float64 instead of
    float32, fed the same tokens.  Both are exact readings of the forward;
    under bf16 storage their summation rounding turns into whole-ulp flips
    that compound over the layers, and ``spread`` (max |difference| of the
    bf16-rounded logits) measures how far two correct bf16 forwards drift
    apart on these inputs;
  * bound on the logits: max(2e-2, 1.5 * spread) for bf16 storage (2e-2 is
    the stated bound; 1.5 * spread the floor that any other summation order
    can be held to, the GPU having measured 1.0 - 1.42 x spread);
  * top-1 agreement, raw (all positions) and decisive (positions whose
    oracle top-1 margin exceeds ``spread``: there a correct forward must pick
    the oracle's token).  Decisive agreement must be >= 99 %, at least a
    fifth of the positions must be decisive, and every pick must be a token
    whose oracle logit is within the bound of the oracle maximum.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from .ops import bf16_round


@dataclasses.dataclass
class Parity:
    positions: int
    max_abs_err: float          # over all compared logits (bf16-rounded on both sides for bf16 storage)
    max_rel_err: float          # max |d| / max |ref|, worst position
    top1_raw: float             # fraction of positions whose argmax equals the oracle's
    cosine_min: float
    spread: float               # oracle(f32 sums) vs oracle(f64 sums), same inputs
    tol: float                  # bound applied to max_abs_err
    decisive: int               # positions whose oracle top-1 margin exceeds spread
    top1_decisive: float        # agreement on those
    valid_picks: float          # fraction of picks within tol of the oracle maximum
    min_decisive: int           # decisive positions required
    bf16: bool = True           # storage; float32 models are held to 1e-4 relative and equal tokens

    def summary(self):
        return (f"positions={self.positions} max_abs_err={self.max_abs_err:.3e} spread={self.spread:.3e} "
                f"tol={self.tol:.3e} top1_raw={self.top1_raw:.4f} decisive={self.decisive}/{self.positions} "
                f"top1_decisive={self.top1_decisive:.4f} valid_picks={self.valid_picks:.4f} "
                f"max_rel_err={self.max_rel_err:.3e} cos_min={self.cosine_min:.6f}")

    def ok(self):
        if not self.bf16:
            return self.max_rel_err <= 1e-4 and self.top1_raw == 1.0
        return (self.max_abs_err <= self.tol and self.top1_decisive >= 0.99 and self.valid_picks == 1.0
                and self.decisive >= self.min_decisive)

    def record(self):
        """The figures as a JSON-ready dict."""
        return {k: (round(v, 6) if isinstance(v, float) else v) for k, v in dataclasses.asdict(self).items()}


def reference(orc, prompt, steps, orc64=None):
    """Oracle tokens [B, steps + 1] and logits (list of [B, V]) of a greedy
    run, and the spread against ``orc64`` fed the same tokens (0 without)."""
    toks, logits = orc.generate(prompt, steps)
    spread = 0.0
    if orc64 is not None:
        _, l64 = orc64.generate(prompt, steps, teacher=toks)
        for a, b in zip(logits, l64):
            spread = max(spread, float(np.abs(bf16_round(a) - bf16_round(b)).max()))
    return toks, logits, spread


def compare(got_logits, got_tokens, ref_logits, ref_tokens, spread, bf16: bool, min_decisive_frac=0.2):
    """``got_logits``: list of [B, V] arrays, one per position (prefill, then
    each decode step), the other side fed the oracle's tokens; ``got_tokens``
    [B, positions] its argmax picks."""
    max_abs = max_rel = 0.0
    cos_min = 1.0
    for g, r in zip(got_logits, ref_logits):
        g = np.asarray(g, np.float32)
        r = np.asarray(r, np.float32)
        if bf16:
            g, r = bf16_round(g), bf16_round(r)
        d = np.abs(g.astype(np.float64) - r)
        max_abs = max(max_abs, float(d.max()))
        max_rel = max(max_rel, float(d.max() / np.abs(r).max()))
        for b in range(g.shape[0]):
            c = float(np.dot(g[b].astype(np.float64), r[b]) / (np.linalg.norm(g[b]) * np.linalg.norm(r[b])))
            cos_min = min(cos_min, c)
    gt = np.asarray(got_tokens)
    top1_raw = float(np.mean(gt == ref_tokens))
    tol = max(2e-2, 1.5 * spread) if bf16 else 0.0
    dec = dec_ok = valid = total = 0
    for s, r in enumerate(ref_logits):
        for b in range(r.shape[0]):
            top2 = np.partition(r[b], -2)[-2:]
            margin = float(top2[1] - top2[0])
            pick = int(gt[b, s])
            total += 1
            valid += int(r[b, pick] >= r[b].max() - tol)
            if margin > spread:
                dec += 1
                dec_ok += int(pick == int(ref_tokens[b, s]))
    return Parity(total, max_abs, max_rel, top1_raw, cos_min, spread, tol, dec, dec_ok / dec if dec else 0.0,
                  valid / total, int(math.ceil(min_decisive_frac * total)), bf16)
