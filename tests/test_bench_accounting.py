"""The benchmark's algorithmic byte and flop counts (the roofline numerators),
checked against independent derivations: the tensor inventory of the model
(every tensor's shape, as the weight generator draws them), a brute-force
count of the causal (query, key) pairs, and the per-step totals of the
workloads (3.091 GB for the 1.5B batch-1 decode, 1.2177e13 flop for the
4096-token prefill, 10.63 GB for the 64 x 4096 decode, 14.67 GB for the 7B
batch-8 decode); and the command line's refusals.  No GPU."""
import math
import os
import subprocess
import sys

import numpy as np

import bench
import synth


def _tensor_bytes(sh, es=2):
    """Bytes of every tensor of the model, from the generator's inventory."""
    return {(n, l): es * math.prod(synth.tensor_shape(sh, n)) for n, l in synth.weight_names(sh)}


def test_decode_weight_bytes_match_the_tensor_inventory():
    for sh in (synth.Q15B, synth.Q7B):
        tb = _tensor_bytes(sh)
        # every tensor but the embedding, read once per decode step
        total = sum(b for (n, _), b in tb.items() if n != "embed_tokens")
        assert bench.weight_bytes(sh) == total
        # the step adds one embedding row per sequence and the KV rows
        assert bench.decode_step_bytes(sh, 3, 10) == total + 3 * (2 * sh.hidden + 10 * bench.kv_bytes_per_token(sh))


def test_kv_bytes_per_token():
    for sh in (synth.Q15B, synth.Q7B):
        # K and V, every layer, every KV head, head_dim bf16 values
        assert bench.kv_bytes_per_token(sh) == sh.nlayer * 2 * sh.nkv * sh.dh * 2
        # FP8: one byte per value plus a float32 scale per 128-value block
        assert bench.kv_bytes_per_token(sh, kv_fp8=True) == sh.nlayer * 2 * sh.nkv * (sh.dh + 4 * sh.dh // 128)
    assert bench.kv_bytes_per_token(synth.Q15B) == 28672


def test_prefill_flops_brute_force_causal_pairs():
    sh = synth.Q15B
    for T in (1, 7, 128, 300):
        pairs = int(np.tril(np.ones((T, T), np.int64)).sum())        # (query, key) with key <= query
        att = sh.nlayer * sh.nh * pairs * 2 * 2 * sh.dh                 # q.k and p.v, 2 flop per MAC
        tb = _tensor_bytes(sh, es=1)
        macs_per_token = sum(v for (n, _), v in tb.items() if n.endswith(".weight"))
        lin = 2 * T * macs_per_token
        head = 2 * sh.hidden * sh.vocab                                 # the last position's logits only
        assert bench.prefill_flops(sh, 1, T) == lin + att + head


def test_workload_totals():
    wl = synth.WORKLOADS
    B = wl["B"]
    ctx_b = range(B.prompt + 1, B.prompt + B.steps + 1)
    step_b = np.mean([bench.decode_step_bytes(B.shape, 1, c) for c in ctx_b])
    assert abs(step_b / 1e9 - 3.091) < 5e-4
    assert abs(bench.prefill_flops(wl["C"].shape, 1, 4096) / 1e13 - 1.2177) < 5e-4
    D = wl["D"]
    step_d = np.mean([bench.decode_step_bytes(D.shape, D.batch, c) for c in range(D.prompt + 1, D.prompt + D.steps + 1)])
    assert abs(step_d / 1e9 - 10.63) < 0.01
    E = wl["E"]
    step_e = np.mean([bench.decode_step_bytes(E.shape, E.batch, c) for c in range(E.prompt + 1, E.prompt + E.steps + 1)])
    assert abs(step_e / 1e9 - 14.67) < 0.01


def test_prefill_stage_flops_sum_to_the_layer():
    sh = synth.Q15B
    T = 4096
    stages = sum(bench.prefill_stage_flops(sh, T, s) for s in bench.PREFILL_STAGES)
    per_layer = (bench.prefill_flops(sh, 1, T) - 2 * sh.hidden * sh.vocab) // sh.nlayer
    assert stages == per_layer


def _bench(*args):
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    return subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_bench_refuses_more_than_one_gpu():
    """One GPU only: --gpus 2 exits with status 2 and says so, before touching
    any device."""
    r = _bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr, (r.returncode, r.stderr)


def test_bench_stage_only_for_prefill_kernel_runs():
    r = _bench("--stage", "down")
    assert r.returncode != 0 and "--stage applies to --only-kernel runs of workload C" in r.stderr, r.stderr
