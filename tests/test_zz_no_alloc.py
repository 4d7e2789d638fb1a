"""q2_linear_noalloc (split-K partials in the library's fixed per-GPU scratch,
no allocation) against q2_linear with a caller workspace: the same plan and
kernels, so the outputs are bit-equal; and against the oracle to the linear
operator's bar.  Two calls in a row, the second smaller, then a product
whose partials exceed the scratch (rejected, nothing written)."""
import numpy as np
import pytest
import torch

import oracle
import qwen2_decoder_forward_amd as q2
from tests.gpu_util import DEV, assert_close, bf16_vals, down, up

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _case(r, M, N, K, bias):
    x = bf16_vals(r, (M, K))
    w = bf16_vals(r, (N, K), 0.05)
    b = bf16_vals(r, (N,), 0.1) if bias else None
    return x, w, b


def test_noalloc_linear_matches_workspace_linear():
    r = np.random.default_rng(91)
    # first a split-K skinny product with large partials, then a smaller
    # split GEMV: the second call reuses (and must not read stale) scratch
    for M, N, K, bias in [(48, 1536, 8960, False), (2, 1536, 8960, True)]:
        need = q2.q2_linear_workspace_bytes(M, N, K)
        assert 0 < need <= q2.NOALLOC_SCRATCH_BYTES, (M, N, K, need)
        x, w, b = _case(r, M, N, K, bias)
        X, W, Bt = up(x, BF), up(w, BF), (up(b, BF) if bias else None)
        got = torch.full((M, N), float("nan"), dtype=BF, device=DEV)
        q2.q2_linear_noalloc(got, X, W, Bt)
        ref_ws = torch.empty(M, N, dtype=BF, device=DEV)
        q2.q2_linear(ref_ws, X, W, Bt, q2.workspace(need))
        torch.cuda.synchronize()
        assert torch.equal(got, ref_ws), (M, N, K)
        ref = oracle.bf16_round(oracle.linear(x, w, b))
        assert_close(down(got), ref, 1e-6 * (np.abs(x) @ np.abs(w).T), 2 ** -7, f"noalloc linear {M}x{N}x{K}")


def test_noalloc_linear_rejects_partials_beyond_scratch():
    M, N, K = 64, 65536, 8192
    need = q2.q2_linear_workspace_bytes(M, N, K)
    assert need > q2.NOALLOC_SCRATCH_BYTES, need
    X = torch.zeros(M, K, dtype=BF, device=DEV)
    W = torch.empty(N, K, dtype=BF, device=DEV)
    out = torch.full((M, N), 3.0, dtype=BF, device=DEV)
    with pytest.raises(q2.Q2Error) as e:
        q2.q2_linear_noalloc(out, X, W)
    assert e.value.name == "Q2_ESHAPE" and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
