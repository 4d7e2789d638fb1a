"""Helpers for the GPU parity tests: seeded inputs, uploads, bf16 comparisons."""
import numpy as np
import torch

import oracle

DEV = "cuda:0"


def bf16_vals(rng, shape, scale=1.0):
    """Random float32 array whose values are exact bf16 numbers."""
    return oracle.bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))


def up(x, dtype=None):
    """Upload a numpy array (float32 -> given torch dtype; int64 stays int64)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def down(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.int64 else t.cpu().numpy()


def bf16_ulps(a, b):
    """Distance in bf16 ulps between arrays of bf16-representable float32 values."""
    def key(x):
        u = (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a) - key(b))


def assert_close(got, ref, atol, rtol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = np.asarray(atol, np.float64) + rtol * np.abs(ref)
    # NaN anywhere in got fails (it compares false against any bound); exact
    # matches, infinities included, pass
    bad = ~((err <= bound) | (got == ref))
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        a = np.broadcast_to(np.asarray(atol, np.float64), err.shape)[i]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} (atol {a}, rtol {rtol})")
