#!/usr/bin/env python3
"""Benchmark of the Qwen2 decoder forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload B|C|D|E] [--no-cpu]

Default workload B: Qwen2-1.5B shape, bf16, random-init weights, batch 1,
64-token random prompt, 128 greedy decode steps.  One "step" is one pass of
the whole hot path over one batch: prefill of the prompt, then the decode
steps with the argmax fed back on the device.  `value` is decode tokens/s
(the generated tokens over the decode-loop time, HIP events on the stream
the library launches on); prefill tokens/s is reported beside it.  Weights
and prompts are resident in HBM before the timed region.

Also reported:
  roofline      the dominant kernel of the step, launched through the C ABI at
                its in-step shape and timed with HIP events on the same stream
                (bandwidth-bound kernels cycle through operands several times
                the last-level cache); `traffic` is its HBM bytes per launch
                from profiler counters (profiles/traffic.json) while the
                kernel source is unchanged since they were taken.
  step_roofline algorithmic bytes (or flops) of a whole decode (prefill) step
                against the HBM (MFMA) peak.
  cpu_baseline  the oracle (plain NumPy) timed on this host on a bounded
                sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="B", choices=["B", "C", "D", "E"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--only-kernel", action="store_true",
                    help="time only the dominant kernel (for profiler counter runs) and print its record")
    return ap.parse_args()


# ----------------------------------------------------------------------------- byte / flop accounting

def weight_bytes(sh, es=2):
    """Bytes of every weight a decode step reads (embedding: one row per token)."""
    H, I, V, qkv, qd = sh.hidden, sh.inter, sh.vocab, sh.qkv_out, sh.nh * sh.dh
    per_layer = (qkv * H + qkv + qd * H + 2 * I * H + H * I + 2 * H) * es
    return sh.nlayer * per_layer + V * H * es + H * es


def kv_bytes_per_token(sh, es=2):
    """K and V bytes of one cached position across all layers (Day-0 article, step 7)."""
    return 2 * sh.nlayer * sh.nkv * sh.dh * es


def decode_step_bytes(sh, batch, ctx):
    """Algorithmic HBM bytes of one decode step at context ctx (keys incl. the new one)."""
    return weight_bytes(sh) + batch * (ctx * kv_bytes_per_token(sh) + sh.hidden * 2)


def prefill_flops(sh, batch, T):
    H, I, qkv, qd = sh.hidden, sh.inter, sh.qkv_out, sh.nh * sh.dh
    lin = 2 * batch * T * sh.nlayer * (qkv * H + qd * H + 3 * I * H)
    att = 4 * sh.dh * sh.nh * sh.nlayer * batch * T * (T + 1) // 2
    head = 2 * batch * H * sh.vocab
    return lin + att + head


# ----------------------------------------------------------------------------- timing helpers

def time_launches(fn, reps, stream):
    import torch
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps * 1e-3   # seconds per launch


# Weight buffers the dominant-kernel timing cycles through: together they are
# several times the 256 MB last-level (Infinity) cache, so every launch streams
# its operand from HBM as it does inside a decode step.
CYCLE_BYTES = 1 << 30
CALIB_COPY_BYTES = 512 << 20   # plain device copy, the reference for the HBM byte counters


def dominant_kernel(wl, reps):
    """Time the dominant kernel at its in-step shape through the C ABI."""
    import torch
    import qwen2_decoder_forward_amd as q2
    sh = wl.shape
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    g = torch.Generator(device=dev).manual_seed(0)
    # a copy of known size, so that profiler byte counters can be scaled
    src = torch.empty(CALIB_COPY_BYTES // 4, device=dev, dtype=torch.float32).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if wl.key in ("B", "E"):
        # decode GEMV/skinny GEMM over the packed gate/up weight [2I, H]
        M, N, K = wl.batch, 2 * sh.inter, sh.hidden
        nbuf = max(2, -(-CYCLE_BYTES // (N * K * 2)))
        Ws = [(torch.randn(N, K, device=dev, generator=g) * 0.02).to(torch.bfloat16) for _ in range(nbuf)]
        X = torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16)
        out = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
        it = [0]

        def launch():
            q2.q2_linear(out, X, Ws[it[0] % nbuf])
            it[0] += 1
        dt = time_launches(launch, reps, stream)
        traffic = N * K * 2 + M * K * 2 + M * N * 2
        return {"kernel": "gemv_kernel (q2_linear, bf16, M=%d N=%d K=%d, %d weight buffers cycled)" % (M, N, K, nbuf),
                "bound": "hbm", "achieved": traffic / dt / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "bytes_per_launch": traffic, "avg_launch_us": dt * 1e6}
    if wl.key == "C":
        M, N, K = wl.prompt, 2 * sh.inter, sh.hidden
        W = (torch.randn(N, K, device=dev, generator=g) * 0.02).to(torch.bfloat16)
        X = torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16)
        out = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
        dt = time_launches(lambda: q2.q2_linear(out, X, W), reps, stream)
        flops = 2 * M * N * K
        return {"kernel": "gemm_dtl_mix_kernel (q2_linear, bf16, M=%d N=%d K=%d)" % (M, N, K),
                "bound": "mfma", "achieved": flops / dt / 1e12, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "flops_per_launch": flops, "avg_launch_us": dt * 1e6}
    # D: split-KV decode attention over a 4097-key cache for 64 sequences
    B, S = wl.batch, wl.prompt + 1
    kv_bytes = 2 * B * S * sh.nkv * sh.dh * 2
    nbuf = max(2, -(-CYCLE_BYTES // kv_bytes))
    q = torch.randn(B, 1, sh.nh, sh.dh, device=dev, generator=g).to(torch.bfloat16)
    kvs = [(torch.randn(B, S, sh.nkv, sh.dh, device=dev, generator=g).to(torch.bfloat16),
            torch.randn(B, S, sh.nkv, sh.dh, device=dev, generator=g).to(torch.bfloat16)) for _ in range(nbuf)]
    o = torch.empty_like(q)
    it = [0]

    def launch():
        k, v = kvs[it[0] % nbuf]
        q2.q2_self_attention(o, q, k, v, sh.dh ** -0.5)
        it[0] += 1
    dt = time_launches(launch, reps, stream)
    traffic = kv_bytes + 2 * q.numel() * 2
    return {"kernel": "attn_decode_kernel + attn_combine_kernel (q2_self_attention, B=%d S=%d, %d caches cycled)"
            % (B, S, nbuf), "bound": "hbm", "achieved": traffic / dt / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "bytes_per_launch": traffic, "avg_launch_us": dt * 1e6}


def measured_traffic(wl):
    """HBM bytes per launch of the dominant kernel from the committed profiler
    counter runs, or None when they are absent or the kernel source changed
    since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(wl.key)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["traffic_bytes"]


def cpu_baseline(wl, weights, budget_s):
    """Time the oracle, as it stands, on a bounded sample of the workload."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        cores = len(os.sched_getaffinity(0))
    sh = wl.shape
    if wl.key == "B" or wl.key == "D":
        batch = 1 if wl.key == "B" else 2
        plen = wl.prompt if wl.key == "B" else 512
        prompt = synth.make_prompt(wl, batch=batch, length=plen)
        orc = oracle.OracleModel(sh, weights, "bf16", batch, plen + 256)
        t0 = time.perf_counter()
        _, nxt = orc.forward(prompt)
        t_pre = time.perf_counter() - t0
        n = 0
        t0 = time.perf_counter()
        while n < 256 and (n < 2 or time.perf_counter() - t0 < budget_s):
            _, nxt = orc.forward(nxt[:, None])
            n += 1
        t_dec = time.perf_counter() - t0
        sample = (f"oracle bf16-storage forward, batch {batch}, prefill {plen} tokens then {n} greedy decode "
                  f"steps (decode timed)")
        return {"value": batch * n / t_dec, "unit": "tok/s", "cores": int(cores), "kind": "oracle",
                "sample": sample, "prefill_tok_s": batch * plen / t_pre}
    if wl.key == "C":
        plen = 512
        prompt = synth.make_prompt(wl, length=plen)
        orc = oracle.OracleModel(sh, weights, "bf16", 1, plen)
        t0 = time.perf_counter()
        orc.forward(prompt)
        dt = time.perf_counter() - t0
        return {"value": plen / dt, "unit": "tok/s", "cores": int(cores), "kind": "oracle",
                "sample": f"oracle bf16-storage prefill of the first {plen} prompt tokens (of 4096)"}
    return None


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported by this build "
              "(the forward is single-GPU; see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import qwen2_decoder_forward_amd as q2
    from tests.model_util import build_model

    wl = synth.WORKLOADS[args.workload]
    sh = wl.shape
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.only_kernel:
        dk = dominant_kernel(wl, args.kernel_reps)
        print(json.dumps({"workload": wl.key, "dominant_kernel": dk}), flush=True)
        return
    t0 = time.perf_counter()
    weights = synth.make_weights(wl)
    t_gen = time.perf_counter() - t0
    max_seq = wl.prompt + wl.steps
    t0 = time.perf_counter()
    model = build_model(sh, weights, max_seq, wl.batch)
    torch.cuda.synchronize()
    t_load = time.perf_counter() - t0
    prompt = torch.from_numpy(synth.make_prompt(wl)).to(dev)
    nxt = torch.empty(wl.batch, dtype=torch.int64, device=dev)
    out = torch.empty(wl.batch, max(wl.steps, 1), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    pre_ms, dec_ms, step_ms = [], [], []

    def one_step(record):
        model.reset()
        e0, e1, e2 = ev(), ev(), ev()
        e0.record(stream)
        q2.q2_model_prefill(model.handle, prompt, nxt)
        e1.record(stream)
        if wl.steps:
            q2.q2_model_continue(model.handle, wl.steps, out)
        e2.record(stream)
        if record:
            e2.synchronize()
            pre_ms.append(e0.elapsed_time(e1))
            dec_ms.append(e1.elapsed_time(e2))
            step_ms.append(e0.elapsed_time(e2))

    for _ in range(args.warmup):
        one_step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_s = float(np.mean(pre_ms)) * 1e-3
    dec_s = float(np.mean(dec_ms)) * 1e-3 if wl.steps else 0.0
    prefill_tok_s = wl.batch * wl.prompt / pre_s
    decode_tok_s = wl.batch * wl.steps / dec_s if wl.steps else None

    dk = dominant_kernel(wl, args.kernel_reps)
    roofline = {"bound": dk["bound"], "achieved": round(dk["achieved"], 2), "peak": dk["peak"], "unit": dk["unit"],
                "frac": round(dk["achieved"] / dk["peak"], 4), "traffic": measured_traffic(wl), "kernel": dk["kernel"],
                "avg_launch_us": round(dk["avg_launch_us"], 2)}
    for key in ("bytes_per_launch", "flops_per_launch"):
        if key in dk:
            roofline[key] = dk[key]

    if wl.steps:
        ctxs = range(wl.prompt + 1, wl.prompt + wl.steps + 1)
        step_bytes = float(np.mean([decode_step_bytes(sh, wl.batch, c) for c in ctxs]))
        gbs = step_bytes / (dec_s / wl.steps) / 1e9
        step_roof = {"what": "decode step", "bound": "hbm", "bytes_per_step": step_bytes, "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        fl = prefill_flops(sh, wl.batch, wl.prompt)
        tf = fl / pre_s / 1e12
        step_roof = {"what": "prefill", "bound": "mfma", "flops": fl, "achieved": round(tf, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4)}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, weights, args.cpu_seconds)

    if wl.steps:
        metric, value = "decode tok/s", decode_tok_s
    else:
        metric, value = "prefill tok/s", prefill_tok_s
    rec = {
        "metric": metric + " (Qwen2 decoder forward, 1 GPU) + % HBM/MFMA roofline",
        "value": round(value, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(step_ms)), 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded random-init weights and prompt ids)",
        "config": {"workload": f"{wl.key}: {wl.description}", "shape": sh.name, "batch": wl.batch,
                   "prompt": wl.prompt, "decode_steps": wl.steps, "parallelism": "single GPU"},
        "prefill_tok_s": round(prefill_tok_s, 1),
        "decode_tok_s": round(decode_tok_s, 2) if decode_tok_s else None,
        "prefill_ms": round(pre_s * 1e3, 3), "decode_ms": round(dec_s * 1e3, 3),
        "roofline": roofline, "step_roofline": step_roof, "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3), "weight_gen_s": round(t_gen, 1), "load_s": round(t_load, 2),
        "library": q2.version(),
    }
    model.close()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
