#!/usr/bin/env python3
"""Decode-step benchmark of the MI355X quantized Llama decode library.

One "step" = one greedy batch-1 decode step of the whole model (embedding,
every layer's RMSNorm + QKV + RoPE/KV-append, GQA attention, Wo, RMSNorm +
gate/up + SwiGLU, down, then final norm + LM head + argmax) on synthetic
seeded weights already resident in HBM.  The default workload is the
Llama-3.1-8B-shaped Q8_0 model at KV context 512 (+64 steps), batch 1.

Prints ONE JSON line:
  value           decode tokens/s over the timed steps (whole job; one GPU)
  roofline        the dominant kernel (gate/up dequant-GEMV): algorithmic bytes
                  per launch / average launch time from HIP events on the
                  model's stream, against 8 TB/s
  cpu_baseline    the fp64 oracle on this host's cores, on a bounded sample
Usage: python bench.py [--gpus 1] [--steps 64] [--warmup 2] [--workload llama8b_q8]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
DOMINANT = "gateup"
WORKLOAD_TEXT = {
    "llama8b_q8": "Llama-3.1-8B-shaped synthetic decoder (vocab 128256, hidden 4096, 32 layers, "
                  "32/8 heads, hd 128, ffn 14336), Q8_0 weights resident in HBM, batch 1, "
                  "KV context 512 (+steps), greedy decode",
}


def log(*a):
    print(time.strftime("%H:%M:%S"), *a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("lm_kernels.hip", "lm_internal.h"):
        with open(os.path.join(ROOT, "token_decode_llama_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kind: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            d = json.load(fh)
        if d.get("kernel_source_sha256_16") != kernel_source_digest():
            return None
        return float(d["hbm_bytes_per_launch"])
    except Exception:
        return None


def cpu_baseline(model, cfg, budget_s: float):
    """The oracle as it stands, timed on this host on the same workload."""
    import numpy as np
    import oracle
    import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    om = oracle.OracleModel(model, max_seqs=1, max_ctx=cfg.ctx + 64)
    for l in range(cfg.n_layers):
        om.load_kv(0, l, *synth.make_kv(cfg, 0, l))
    tok = synth.start_tokens(cfg, 1)
    n = 0
    t0 = time.perf_counter()
    while True:
        _, am = om.step(tok)
        tok = am
        n += 1
        if time.perf_counter() - t0 >= budget_s or n >= 64:
            break
    dt = time.perf_counter() - t0
    om.close()
    return {"value": round(n / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} greedy decode steps of the same model from context {cfg.ctx} "
                      f"({dt:.1f} s, fp64, OpenMP over output rows)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama8b_q8")
    ap.add_argument("--timing-steps", type=int, default=8,
                    help="eager steps with per-kernel HIP events for the roofline")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-kernels", action="store_true",
                    help="skip the timed loop: run the per-kernel timing steps only (for profilers)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run two calibration dispatches of known traffic for HBM counters: "
                         "a plain read of 1 GiB (k_read_bw) and a dequant of 64 down-projection rows "
                         "that writes 64*ffn*4 bytes (k_dequant)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the per-GPU throughput is the --gpus 1 figure)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import token_decode_llama_amd as lm

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    base = synth.CONFIGS[args.workload]
    extra = max(args.steps, args.warmup, args.timing_steps, 1)
    cfg = synth.variant(args.workload, steps=extra)
    log(f"generating {args.workload} ({cfg.weight_bytes() / 1e9:.2f} GB of quantized weights)")
    model = synth.make_model(cfg)
    stream = torch.cuda.Stream()          # the model's stream (default priority)
    log("loading into HBM")
    g = lm.open_model(model, lambda s, l: synth.make_kv(cfg, s, l), max_seqs=1, kv_seqs=1,
                      stream=stream.cuda_stream)
    dev = torch.device("cuda:0")
    with torch.cuda.stream(stream):
        tok = torch.from_numpy(synth.start_tokens(cfg, 1)).to(dev)
        d_tok = tok.clone()
    torch.cuda.synchronize()

    # warm-up (also captures the step graph), then rewind to the prefill length
    for _ in range(args.warmup):
        g.step_dev(d_tok, 1, d_tok)
    torch.cuda.synchronize()
    g.set_position(0, cfg.ctx)
    with torch.cuda.stream(stream):
        d_tok.copy_(tok)
    torch.cuda.synchronize()

    ms_per_step = None
    if not args.only_kernels:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            g.step_dev(d_tok, 1, d_tok)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_per_step = e0.elapsed_time(e1) / args.steps
        log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step")

    # per-kernel durations from HIP events on the model's stream (eager steps)
    g.set_position(0, cfg.ctx)
    with torch.cuda.stream(stream):
        d_tok.copy_(tok)
    torch.cuda.synchronize()
    g.kernel_timing(True)
    for _ in range(args.timing_steps):
        g.step_dev(d_tok, 1, d_tok)
    torch.cuda.synchronize()
    kstats = {}
    for k in lm.KERNEL_KINDS:
        n, ms = g.kernel_stats(k)
        kstats[k] = (n, ms)
    g.kernel_timing(False)
    L = cfg.n_layers
    # bytes at the positions the timing steps ran at (their mean position)
    g.set_position(0, cfg.ctx + args.timing_steps // 2)
    kbytes = {k: g.kernel_bytes(k, 1) for k in lm.KERNEL_KINDS}
    g.set_position(0, cfg.ctx + args.steps // 2)
    step_bytes = sum(g.kernel_bytes(k, 1) for k in lm.KERNEL_KINDS)
    g.set_position(0, cfg.ctx)

    n_dom, ms_dom = kstats[DOMINANT]
    per_launch_bytes = kbytes[DOMINANT] / L
    avg_ms = ms_dom / max(n_dom, 1)
    achieved = per_launch_bytes / (avg_ms * 1e-3) / 1e9
    kernels = {k: {"launches": kstats[k][0],
                   "avg_us": round(1e3 * kstats[k][1] / max(kstats[k][0], 1), 3),
                   "algorithmic_GBps": round((kbytes[k] / (L if k not in ("embed", "lmhead") else 1))
                                             / (kstats[k][1] / max(kstats[k][0], 1) * 1e-3) / 1e9, 1)
                   if kstats[k][0] else None}
               for k in lm.KERNEL_KINDS}
    read_ms = g.debug_read_bw(4 << 30, 5)
    read_ceiling = (4 << 30) / (read_ms * 1e-3) / 1e9

    if args.calibrate:
        g.debug_read_bw(1 << 30, 1)
        g.debug_dequant(0, 6, 0, 64, cfg.ffn)
        torch.cuda.synchronize()
        log(f"calibration: read {1 << 30} bytes; dequant wrote {64 * cfg.ffn * 4} bytes")
    traffic = traffic_from_profiles(DOMINANT, args.workload)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "k_gemv<Q8_0, gate/up, SwiGLU epilogue>",
                "bytes_per_launch": int(per_launch_bytes), "avg_launch_us": round(avg_ms * 1e3, 3)}

    out = {"metric": "decode tokens/s + achieved HBM GB/s (% of peak), 8B-shape Q8_0 batch 1"}
    if ms_per_step is not None:
        tps = 1000.0 / ms_per_step
        gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
        out.update({"value": round(tps, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                    "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
                    "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                    "dtype": "f32", "data": "synthetic",
                    "achieved_hbm_GBps": round(gbps, 1),
                    "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
                    "step_bytes": int(step_bytes)})
    out["config"] = {"workload": WORKLOAD_TEXT.get(args.workload, args.workload), "name": args.workload,
                     "batch": 1, "ctx": base.ctx, "qtype": "Q8_0" if cfg.qtype == synth.Q8_0 else "Q4_0",
                     "weights": "random N(0,0.02), quantized, resident in HBM"}
    out["roofline"] = roofline
    out["read_ceiling_GBps"] = round(read_ceiling, 1)
    out["kernels"] = kernels
    if not args.no_cpu_baseline and not args.only_kernels:
        log("oracle baseline")
        out["cpu_baseline"] = cpu_baseline(model, cfg, args.cpu_budget)
    g.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
