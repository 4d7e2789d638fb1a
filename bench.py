#!/usr/bin/env python3
"""Benchmark of the Qwen2 decoder forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload B|C|D|E] [--no-cpu]
                    [--also C,D] [--kv bf16|fp8] [--paged N]

Default workload B: Qwen2-1.5B shape, bf16, random-init weights, batch 1,
64-token random prompt, 128 greedy decode steps.  One "step" is one pass of
the whole hot path over one batch: prefill of the prompt, then the decode
steps with the argmax fed back on the device.  `value` is decode tokens/s
(the generated tokens over the decode-loop time, HIP events on the stream
the library launches on); prefill tokens/s is reported beside it.  Weights
and prompts are resident in HBM before the timed region.

Also reported:
  roofline      the dominant kernel of the step, relaunched as the step
                launches it (q2_model_replay_stage: the forward's kernels and
                arguments on the model's own weights and buffers, layers
                cycled so that every launch streams from HBM) and timed with
                HIP events on the launch stream: B and E the gate/up GEMV, C
                the prefill gate/up GEMM, D the decode attention kernel;
                `traffic` is its HBM bytes per launch from profiler counters
                (profiles/traffic.json) while the kernel source is unchanged
                since they were taken; `achievable` is what plain library
                code reaches on the box (a device copy for HBM, torch.matmul
                on the prefill gate/up shape for MFMA) and the kernel's
                fraction of it.
  step_roofline algorithmic bytes (or flops) of a whole decode (prefill) step
                against the HBM (MFMA) peak.
  cpu_baseline  the oracle (plain NumPy) timed on this host on a bounded
                sample of the same workload (for B: the whole workload),
                with the BLAS thread count and the CPU model.
  parity        (B) after the timed region: the GPU fed the oracle's greedy
                tokens, its logits against the oracle's at every position
                (raw max abs error, raw and decisive top-1 agreement, the
                oracle's own float32/float64 spread and the derived bound).
  also          (B, unless --also says otherwise) workloads C and D on the
                same weights, after the main one: value, step time,
                dominant-kernel and step rooflines of each, as measured by
                this same run (they do not enter `value`).
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
    ap.add_argument("--stage", default=None, choices=sorted(PREFILL_STAGES),
                    help="with --only-kernel and workload C: the prefill product (or the attention) to replay "
                         "instead of gate/up")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="KV cache: bf16 (the workloads' definition) or FP8 E4M3 blocks with per-block scales")
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads of the same model shape timed after the main one, each "
                         "reported as a compact record under `also` (default: C,D after B; '' for none)")
    ap.add_argument("--also-steps", type=int, default=3, help="timed passes of each --also workload")
    ap.add_argument("--paged", type=int, default=0,
                    help="positions per page of a paged KV cache (0: contiguous per-sequence cache)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- byte / flop accounting

def weight_bytes(sh, es=2):
    """Bytes of every weight a decode step reads (embedding: one row per token)."""
    H, I, V, qkv, qd = sh.hidden, sh.inter, sh.vocab, sh.qkv_out, sh.nh * sh.dh
    per_layer = (qkv * H + qkv + qd * H + 2 * I * H + H * I + 2 * H) * es
    return sh.nlayer * per_layer + V * H * es + H * es


def kv_bytes_per_token(sh, kv_fp8=False):
    """K and V bytes of one cached position across all layers ("万亿参数大模型
    在国产加速卡上的Day-0适配教程", step 7, KV-cache memory estimate); the FP8
    cache stores one byte per element plus a float32 scale per 128-element
    block."""
    if kv_fp8:
        return 2 * sh.nlayer * sh.nkv * (sh.dh + 4 * (sh.dh // 128))
    return 2 * sh.nlayer * sh.nkv * sh.dh * 2


def decode_step_bytes(sh, batch, ctx, kv_fp8=False):
    """Algorithmic HBM bytes of one decode step at context ctx (keys incl. the new one)."""
    return weight_bytes(sh) + batch * (ctx * kv_bytes_per_token(sh, kv_fp8) + sh.hidden * 2)


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


CALIB_COPY_BYTES = 512 << 20   # plain device copy, the reference for the HBM byte counters

STAGE_NAMES = {0: "QKV", 1: "attention", 2: "o_proj", 3: "gate/up", 4: "down",
               5: "attention (split-KV kernel without its merge)"}


PREFILL_STAGES = {"qkv": 0, "attn": 1, "o": 2, "gate_up": 3, "down": 4}


def prefill_stage_flops(sh, T, stage):
    """Algorithmic flops of one prefill product (or causal attention) over T tokens."""
    H, I, qd = sh.hidden, sh.inter, sh.nh * sh.dh
    return {"qkv": 2 * T * H * sh.qkv_out, "o": 2 * T * qd * H, "gate_up": 2 * T * 2 * I * H,
            "down": 2 * T * I * H, "attn": 4 * sh.dh * sh.nh * T * (T + 1) // 2}[stage]


def in_step_kernel(model, wl, prompt, reps, kv_fp8, stage_name=None):
    """Time the dominant kernel of the step as the step launches it: the
    model replays that product (q2_model_replay_stage: the same kernels and
    arguments as the forward, on the model's own weights and buffers) for
    layers 0, 1, ... in turn, `reps` launches between two HIP events on the
    launch stream.  Cycling the 28 layers keeps every launch streaming its
    weights (or KV rows) from HBM, as in the step.  The model is reset
    afterwards."""
    import torch
    import qwen2_decoder_forward_amd as q2
    sh = wl.shape
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    # a copy of known size first, so that profiler byte counters can be scaled
    src = torch.empty(CALIB_COPY_BYTES // 4, device=dev, dtype=torch.float32).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    model.reset()
    B, H, I = wl.batch, sh.hidden, sh.inter
    if wl.key == "C":
        # the prefill product at length 0 (gate/up unless another is asked for)
        stage, tokens = PREFILL_STAGES[stage_name or "gate_up"], wl.prompt
    else:
        nxt = torch.empty(B, dtype=torch.int64, device=dev)
        q2.q2_model_prefill(model.handle, prompt, nxt)        # decode products at length = prompt
        stage = q2.STAGE_ATTN_CORE if wl.key == "D" else q2.STAGE_GATE_UP
        tokens = 1

    def launch(n):
        q2.q2_model_replay_stage(model.handle, stage, B, tokens, n)
    launch(sh.nlayer)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    launch(reps)
    e1.record(stream)
    e1.synchronize()
    dt = e0.elapsed_time(e1) / reps * 1e-3
    model.reset()
    name = f"{STAGE_NAMES[stage]} product of the step (q2_model_replay_stage, {B} x {tokens} rows, layers cycled)"
    if wl.key == "C":
        flops = prefill_stage_flops(sh, wl.prompt, stage_name or "gate_up")
        kern = {"gate_up": "gemm_dtl_mix_kernel", "down": "gemm_dtl_sk_kernel", "attn": "attn_prefill_kernel",
                "qkv": "gemm_dtl_kernel", "o": "gemm_dtl_kernel"}[stage_name or "gate_up"]
        return {"kernel": kern + ", " + name, "bound": "mfma", "achieved": flops / dt / 1e12,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "flops_per_launch": flops, "avg_launch_us": dt * 1e6}
    if wl.key == "D":
        keys = wl.prompt + 1
        per_key = sh.nkv * (sh.dh * (1 if kv_fp8 else 2) + (4 if kv_fp8 else 0))
        traffic = 2 * B * keys * per_key + B * sh.nh * sh.dh * 2
        kern = "attn_decode_kernel<%s>" % ("fp8" if kv_fp8 else "bf16")
        return {"kernel": kern + ", " + name, "bound": "hbm", "achieved": traffic / dt / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "bytes_per_launch": traffic, "avg_launch_us": dt * 1e6}
    # weights, norm weight, residual rows and their sums of squares, SwiGLU output
    traffic = 2 * I * H * 2 + H * 2 + B * H * 2 + B * (H // 16) * 4 + B * I * 2
    return {"kernel": "gemv_kernel (norm prologue, SwiGLU epilogue), " + name, "bound": "hbm",
            "achieved": traffic / dt / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes_per_launch": traffic,
            "avg_launch_us": dt * 1e6}


def achievable(bound, sh, reps=20):
    """What plain library code reaches on this machine, beside the published
    peak: for an HBM-bound kernel a device-to-device copy of 512 MiB (read +
    write bytes over its time); for an MFMA-bound one torch.matmul
    (hipBLASLt) on the prefill gate/up shape [4096, H] x [H, 2 I] in bf16."""
    import torch
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    if bound == "hbm":
        src = torch.empty(CALIB_COPY_BYTES // 4, device=dev, dtype=torch.float32).fill_(1.0)
        dst = torch.empty_like(src)
        dt = time_launches(lambda: dst.copy_(src), reps, stream)
        del src, dst
        return {"what": "device copy of 512 MiB (torch)", "value": round(2 * CALIB_COPY_BYTES / dt / 1e9, 1),
                "unit": "GB/s"}
    g = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn(4096, sh.hidden, device=dev, generator=g).to(torch.bfloat16)
    w = torch.randn(sh.hidden, 2 * sh.inter, device=dev, generator=g).to(torch.bfloat16)
    dt = time_launches(lambda: torch.matmul(x, w), reps, stream)
    del x, w
    return {"what": f"torch.matmul bf16 [4096, {sh.hidden}] x [{sh.hidden}, {2 * sh.inter}]",
            "value": round(2 * 4096 * sh.hidden * 2 * sh.inter / dt / 1e12, 1), "unit": "TFLOP/s"}


def measured_traffic(wl, kv="bf16"):
    """HBM bytes per launch of the dominant kernel from the committed profiler
    counter runs, or None when they are absent or the kernel source changed
    since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(wl.key if kv == "bf16" else f"{wl.key}-{kv}")
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(wl, weights, budget_s, kv="bf16"):
    """Time the oracle, as it stands, on a bounded sample of the workload.
    Returns (record, reference) where reference holds the oracle's greedy
    tokens and logits when the sample is the whole workload (B), for the
    parity check, else None."""
    import oracle
    import synth
    sh = wl.shape
    base = {"unit": "tok/s", "cores": int(blas_threads()), "cpu_model": cpu_model(), "kind": "oracle"}
    if wl.key == "B":
        # the whole workload: prefill of the prompt, then every greedy decode step
        prompt = synth.make_prompt(wl)
        orc = oracle.OracleModel(sh, weights, "bf16", 1, wl.prompt + wl.steps, kv="fp8" if kv == "fp8" else "model")
        t0 = time.perf_counter()
        logits, nxt = orc.forward(prompt)
        t_pre = time.perf_counter() - t0
        toks, all_logits = [nxt], [logits]
        t0 = time.perf_counter()
        for _ in range(wl.steps):
            logits, nxt = orc.forward(nxt[:, None])
            toks.append(nxt)
            all_logits.append(logits)
        t_dec = time.perf_counter() - t0
        sample = (f"the whole workload on the oracle (bf16 storage, float32 sums): batch 1, prefill "
                  f"{wl.prompt} tokens, then {wl.steps} greedy decode steps (decode timed)")
        rec = dict(base, value=wl.steps / t_dec, sample=sample, prefill_tok_s=wl.prompt / t_pre)
        import numpy as np
        return rec, (orc, prompt, np.stack(toks, axis=1), all_logits)
    if wl.key == "D":
        batch, plen, n = 2, 512, 0
        prompt = synth.make_prompt(wl, batch=batch, length=plen)
        orc = oracle.OracleModel(sh, weights, "bf16", batch, plen + 256)
        t0 = time.perf_counter()
        _, nxt = orc.forward(prompt)
        t_pre = time.perf_counter() - t0
        t0 = time.perf_counter()
        while n < 256 and (n < 2 or time.perf_counter() - t0 < budget_s):
            _, nxt = orc.forward(nxt[:, None])
            n += 1
        t_dec = time.perf_counter() - t0
        sample = (f"oracle bf16-storage forward, batch {batch}, prefill {plen} tokens then {n} greedy decode "
                  f"steps (decode timed)")
        return dict(base, value=batch * n / t_dec, sample=sample, prefill_tok_s=batch * plen / t_pre), None
    if wl.key == "C":
        plen = 512
        prompt = synth.make_prompt(wl, length=plen)
        orc = oracle.OracleModel(sh, weights, "bf16", 1, plen)
        t0 = time.perf_counter()
        orc.forward(prompt)
        dt = time.perf_counter() - t0
        return dict(base, value=plen / dt,
                    sample=f"oracle bf16-storage prefill of the first {plen} prompt tokens (of 4096)"), None
    return None, None


def parity_record(model, wl, weights, ref):
    """The GPU fed the oracle's greedy tokens over the whole workload, against
    the oracle's logits (oracle.parity: raw max abs error and top-1 agreement,
    the float32/float64 spread of the oracle itself, and the derived bound)."""
    import numpy as np
    import torch
    import oracle
    from oracle import parity
    orc, prompt, toks, ref_logits = ref
    orc64 = oracle.OracleModel(wl.shape, weights, "bf16", 1, wl.prompt + wl.steps, accum="f64", share_from=orc,
                               kv=orc.kv)
    _, l64 = orc64.generate(prompt, wl.steps, teacher=toks)
    spread = max(float(np.abs(oracle.bf16_round(a) - oracle.bf16_round(b)).max()) for a, b in zip(ref_logits, l64))
    del orc64
    model.reset()
    dev = "cuda:0"
    nxt, lg = model.prefill(torch.from_numpy(prompt).to(dev), logits=True)
    got_logits, got_toks = [lg.cpu().numpy()], [nxt.cpu().numpy()]
    for s in range(1, wl.steps + 1):
        nxt, lg = model.decode(torch.from_numpy(np.ascontiguousarray(toks[:, s - 1])).to(dev), logits=True)
        got_logits.append(lg.cpu().numpy())
        got_toks.append(nxt.cpu().numpy())
    r = parity.compare(got_logits, np.stack(got_toks, axis=1), ref_logits, toks, spread, True)
    rec = r.record()
    rec["ok"] = bool(r.ok())
    rec["what"] = ("teacher-forced logits of the prefill and every decode step against the oracle "
                   "(bf16-rounded on both sides); bound max(2e-2, 1.5 x spread)")
    return rec


# ----------------------------------------------------------------------------- main

def measure(wl, weights, steps, warmup, kv="bf16", paged=0, kernel_reps=50, only_kernel=False, stage=None):
    """Load the model of workload `wl`, run `warmup` untimed and `steps` timed
    passes of the hot path (prefill of the prompt, then the greedy decode
    steps with the argmax fed back on the device), and time the dominant
    kernel in the step.  Returns (record, model); the caller closes the model."""
    import numpy as np
    import torch
    import synth
    import qwen2_decoder_forward_amd as q2

    sh = wl.shape
    dev = "cuda:0"
    kv_fp8 = kv == "fp8"
    max_seq = wl.prompt + wl.steps
    t0 = time.perf_counter()
    model = q2.load_model(sh, weights, max_seq, wl.batch, kv_fp8=kv_fp8, page_size=paged)
    torch.cuda.synchronize()
    t_load = time.perf_counter() - t0
    prompt = torch.from_numpy(synth.make_prompt(wl)).to(dev)
    if only_kernel:
        return {"dominant_kernel": in_step_kernel(model, wl, prompt, kernel_reps, kv_fp8, stage)}, model
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

    for _ in range(warmup):
        one_step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_s = float(np.mean(pre_ms)) * 1e-3
    dec_s = float(np.mean(dec_ms)) * 1e-3 if wl.steps else 0.0
    prefill_tok_s = wl.batch * wl.prompt / pre_s
    decode_tok_s = wl.batch * wl.steps / dec_s if wl.steps else None

    dk = in_step_kernel(model, wl, prompt, kernel_reps, kv_fp8)
    roofline = {"bound": dk["bound"], "achieved": round(dk["achieved"], 2), "peak": dk["peak"], "unit": dk["unit"],
                "frac": round(dk["achieved"] / dk["peak"], 4), "traffic": measured_traffic(wl, kv),
                "kernel": dk["kernel"], "avg_launch_us": round(dk["avg_launch_us"], 2)}
    for key in ("bytes_per_launch", "flops_per_launch"):
        if key in dk:
            roofline[key] = dk[key]
    ach = achievable(dk["bound"], sh)
    ach["frac"] = round(dk["achieved"] / ach["value"], 4)
    roofline["achievable"] = ach

    if wl.steps:
        ctxs = range(wl.prompt + 1, wl.prompt + wl.steps + 1)
        step_bytes = float(np.mean([decode_step_bytes(sh, wl.batch, c, kv_fp8) for c in ctxs]))
        gbs = step_bytes / (dec_s / wl.steps) / 1e9
        step_roof = {"what": "decode step", "bound": "hbm", "bytes_per_step": step_bytes, "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        fl = prefill_flops(sh, wl.batch, wl.prompt)
        tf = fl / pre_s / 1e12
        step_roof = {"what": "prefill", "bound": "mfma", "flops": fl, "achieved": round(tf, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4)}

    if wl.steps:
        metric, value = "decode tok/s", decode_tok_s
    else:
        metric, value = "prefill tok/s", prefill_tok_s
    rec = {
        "metric": metric + " (Qwen2 decoder forward, 1 GPU) + % HBM/MFMA roofline",
        "value": round(value, 2), "unit": "tok/s", "steps": steps, "warmup": warmup,
        "ms_per_step": round(float(np.mean(step_ms)), 3),
        "workload": f"{wl.key}: {wl.description}" + (" (FP8 KV cache)" if kv_fp8 else ""),
        "kv_cache": kv + (f", paged ({paged} positions per page)" if paged else ""),
        "prefill_tok_s": round(prefill_tok_s, 1),
        "decode_tok_s": round(decode_tok_s, 2) if decode_tok_s else None,
        "prefill_ms": round(pre_s * 1e3, 3), "decode_ms": round(dec_s * 1e3, 3),
        "roofline": roofline, "step_roofline": step_roof,
        "wall_s_timed": round(wall, 3), "load_s": round(t_load, 2),
    }
    return rec, model


# workloads timed after B when --also is not given (same 1.5B weights): C
# (4096-token prefill) and D (64 x 4096 batched decode)
ALSO_DEFAULT = "C,D"


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the forward runs on one GPU and exchanges nothing between GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.stage and (not args.only_kernel or args.workload != "C"):
        raise SystemExit("--stage applies to --only-kernel runs of workload C")
    import torch

    import synth
    import qwen2_decoder_forward_amd as q2

    wl = synth.WORKLOADS[args.workload]
    sh = wl.shape
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    weights = synth.make_weights(wl)
    t_gen = time.perf_counter() - t0
    if args.only_kernel:
        r, model = measure(wl, weights, 0, 0, args.kv, args.paged, args.kernel_reps, only_kernel=True,
                           stage=args.stage)
        model.close()
        print(json.dumps({"workload": wl.key, "kv": args.kv, **r}), flush=True)
        return
    r, model = measure(wl, weights, args.steps, args.warmup, args.kv, args.paged, args.kernel_reps)

    cpu = par = None
    if not args.no_cpu:
        cpu, ref = cpu_baseline(wl, weights, args.cpu_seconds, args.kv)
        if ref is not None:
            par = parity_record(model, wl, weights, ref)
    model.close()
    del model
    torch.cuda.empty_cache()

    # the other workloads of the same model shape, each a compact record of
    # its own (not part of `value`)
    also = {}
    keys = (ALSO_DEFAULT if wl.key == "B" else "") if args.also is None else args.also
    for key in [k for k in keys.split(",") if k and k != wl.key]:
        wk = synth.WORKLOADS[key]
        if wk.shape.name != sh.name:
            raise SystemExit(f"--also {key}: workload {key} has another model shape than {wl.key}")
        print(f"[bench] timing workload {key}", file=sys.stderr, flush=True)
        ra, ma = measure(wk, weights, args.also_steps, 1, args.kv, args.paged, args.kernel_reps)
        ma.close()
        del ma
        torch.cuda.empty_cache()
        also[key] = {k: ra[k] for k in ("workload", "metric", "value", "unit", "steps", "warmup", "ms_per_step",
                                        "prefill_tok_s", "decode_tok_s")}
        also[key]["roofline"] = {k: ra["roofline"][k] for k in ("kernel", "bound", "achieved", "peak", "unit",
                                                                 "frac", "avg_launch_us", "achievable")}
        also[key]["step_roofline"] = {k: ra["step_roofline"][k] for k in ("what", "achieved", "unit", "frac")}

    rec = {
        "metric": r["metric"], "value": r["value"], "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded random-init weights and prompt ids)",
        "config": {"workload": r["workload"], "shape": sh.name, "batch": wl.batch, "prompt": wl.prompt,
                   "decode_steps": wl.steps, "kv_cache": r["kv_cache"], "parallelism": "single GPU"},
        "prefill_tok_s": r["prefill_tok_s"], "decode_tok_s": r["decode_tok_s"],
        "prefill_ms": r["prefill_ms"], "decode_ms": r["decode_ms"],
        "roofline": r["roofline"], "step_roofline": r["step_roofline"], "cpu_baseline": cpu, "parity": par,
        "also": also or None,
        "wall_s_timed": r["wall_s_timed"], "weight_gen_s": round(t_gen, 1), "load_s": r["load_s"],
        "library": q2.version(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
