"""Helpers for model-level GPU tests: build a q2 model on the GPU from the
seeded synthetic weights, and compare it with the oracle under teacher
forcing (the comparison itself is oracle.parity)."""
import dataclasses

import numpy as np
import torch

import oracle
from oracle import parity
from qwen2_decoder_forward_amd import Model, load_model, weight_tensor

DEV = "cuda:0"


def to_device(arr: np.ndarray) -> torch.Tensor:
    """Upload a synthetic weight (uint16 bf16 bits or float32) bit-for-bit."""
    return weight_tensor(arr)


def build_model(shape, weights, max_seq, max_batch) -> Model:
    return load_model(shape, weights, max_seq, max_batch)


def reduced_shape(shape, **kw):
    return dataclasses.replace(shape, **kw)


def gpu_teacher_forced(model: Model, prompt: np.ndarray, teacher: np.ndarray, steps: int, rows=None):
    """Prefill ``prompt`` on the GPU, then ``steps`` decode steps fed the
    teacher's tokens; logits of every position (rows ``rows`` of the batch
    only, default all) and the GPU's own picks."""
    sel = slice(None) if rows is None else list(rows)
    nxt, lg = model.prefill(torch.from_numpy(prompt).to(DEV), logits=True)
    logits = [lg.cpu().numpy()[sel]]
    toks = [nxt.cpu().numpy()[sel]]
    for s in range(1, steps + 1):
        feed = torch.from_numpy(np.ascontiguousarray(teacher[:, s - 1])).to(DEV)
        nxt, lg = model.decode(feed, logits=True)
        logits.append(lg.cpu().numpy()[sel])
        toks.append(nxt.cpu().numpy()[sel])
    return logits, np.stack(toks, axis=1)


def teacher_forced(model: Model, orc: oracle.OracleModel, prompt: np.ndarray, steps: int,
                   orc64: oracle.OracleModel | None = None) -> parity.Parity:
    """Oracle runs greedily; the GPU is fed the oracle's tokens; logits of the
    prefill and of every decode step are compared (oracle.parity.compare)."""
    ref_toks, ref_logits, spread = parity.reference(orc, prompt, steps, orc64)
    got_logits, got_toks = gpu_teacher_forced(model, prompt, ref_toks, steps)
    return parity.compare(got_logits, got_toks, ref_logits, ref_toks, spread, orc.storage == "bf16")
