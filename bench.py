#!/usr/bin/env python3
"""Decode-step benchmark of the MI355X quantized Llama decode library.

One "step" = one greedy decode step of the whole model (embedding, every
layer's RMSNorm + QKV + RoPE/KV-append, GQA attention, Wo, RMSNorm +
gate/up + SwiGLU, down, then final norm + LM head + argmax) on synthetic
seeded weights.  The default workload (the headline line) is the
Llama-3.1-8B-shaped Q8_0 model at KV context 512 (+64 steps), batch 1, with
every weight resident in HBM.

Other workloads (--workload), each printing one JSON line of its own:
  llama8b_q4   8B shape, Q4_0, four sequences decoded together at KV context
               4096 (+32 steps): the multi-sequence (MFMA) path
  multi        Llama-3.2-1B, Qwen2-0.5B and SmolLM2-360M shapes (Q8_0, KV
               context 2048, 32 steps each) decoded round-robin, each model on
               its own HIP stream; value = aggregate tokens/s
  llama70b_q4  70B shape, Q4_0, KV context 1024, 16 steps: (a) all weights
               resident in HBM, then (b) layer streaming from pinned host
               memory through two HBM layer buffers, (c) the engine page's
               hybrid split, (d) streaming with 20 layers skipped
  llama8b_q4k, llama8b_q5k, llama8b_q6k   8B shape in the GGUF K formats, batch 1, KV
               context 512 (+64 steps), weights resident
  llama70b_q4k, llama70b_q6k  70B shape in the K formats, as llama70b_q4;
               the hybrid split is the page's for that format (Q4_K_M: 36
               of 80 layers in GPU memory, Q6_K: 26)

Every line carries:
  value           decode tokens/s over the timed steps (whole job; one GPU)
  roofline        the dominant kernel: algorithmic bytes per launch / average
                  launch duration from HIP events on the model's stream
  cpu_baseline    the fp64 oracle on this host's cores, on a bounded sample
Side legs (--extras: self-speculative rounds) only add
fields; a failure in one becomes an "error" entry and never drops the line.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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
PAGES_8B_Q8_TOKS = 48.9     # engine page, section 1 table: Llama 3.1 8B Q8_0, all layers in GPU memory
HEADLINE_METRIC = "decode tokens/s + achieved HBM GB/s (% of peak), 8B-shape Q8_0 batch 1"
SHAPE_8B = "vocab 128256, hidden 4096, 32 layers, 32/8 heads, hd 128, ffn 14336"
WORKLOAD_TEXT = {
    "llama8b_q8": f"Llama-3.1-8B-shaped synthetic decoder ({SHAPE_8B}), Q8_0 weights resident "
                  "in HBM, batch 1, KV context 512 (+steps), greedy decode",
    "llama8b_q4": f"Llama-3.1-8B-shaped synthetic decoder ({SHAPE_8B}), Q4_0 weights resident "
                  "in HBM, 4 independent sequences decoded together, KV context 4096 (+steps)",
    "multi": "three concurrently resident Q8_0 models decoded round-robin on three HIP streams: "
             "Llama-3.2-1B shape (hidden 2048, 16 layers, 32/8 heads, hd 64, ffn 8192, vocab 128256), "
             "Qwen2-0.5B shape (hidden 896, 24 layers, 14/2 heads, hd 64, ffn 4864, vocab 151936), "
             "SmolLM2-360M shape (hidden 960, 32 layers, 15/5 heads, hd 64, ffn 2560, vocab 49152); "
             "KV context 2048 (+steps) each, batch 1",
    "llama70b_q4": "Llama-3.1-70B-shaped synthetic decoder (vocab 128256, hidden 8192, 80 layers, "
                   "64/8 heads, hd 128, ffn 28672), Q4_0 weights, batch 1, KV context 1024 (+steps)",
}
for _qt in ("q4k", "q5k", "q6k"):
    _fmt = {"q4k": "Q4_K", "q5k": "Q5_K", "q6k": "Q6_K"}[_qt]
    WORKLOAD_TEXT[f"llama8b_{_qt}"] = (f"Llama-3.1-8B-shaped synthetic decoder ({SHAPE_8B}), {_fmt} weights "
                                       "resident in HBM, batch 1, KV context 512 (+steps), greedy decode")
    WORKLOAD_TEXT[f"llama70b_{_qt}"] = WORKLOAD_TEXT["llama70b_q4"].replace("Q4_0", _fmt)
# layers in GPU memory in the engine page's 70B figures (section 1 table: Q6_K 26 of 80, Q4_K_M 36 of 80)
HYBRID_RESIDENT = {"llama70b_q4": 36, "llama70b_q4k": 36, "llama70b_q6k": 26}
KERNEL_NAMES = {
    "qkv": "k_gemv<QKV, RMSNorm prologue, RoPE + KV-append epilogue>",
    "attn": "k_attn (GQA decode attention on the matrix cores, split over context, in-launch merge)",
    "wo": "k_gemv<Wo, residual epilogue>",
    "gateup": "k_gemv<gate/up, RMSNorm prologue, SwiGLU epilogue>",
    "down": "k_gemv<down, residual epilogue>",
    "lmhead": "k_gemv<LM head, RMSNorm prologue, argmax epilogue>",
}


def log(*a):
    print(time.strftime("%H:%M:%S"), *a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("lm_kernels.hip", "lm_internal.h", "lm_device.h"):
        with open(os.path.join(ROOT, "token_decode_llama_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kind: str, workload: str):
    """HBM bytes (fetched + written) per launch of one operator from the
    committed counter summary of the workload, if it was taken on the current
    kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            d = json.load(fh)
        if d.get("kernel_source_sha256_16") != kernel_source_digest():
            return None
        e = d["per_launch_bytes"][kind]
        return float(e["fetch"] + e["write"])
    except Exception:
        return None


# ---------------------------------------------------------------------------
# rocprofv3 summaries (--summarize): the kernel trace and the two HBM counter
# runs of this script, reduced to the per-operator tables under profiles/
# ---------------------------------------------------------------------------
def kind_of(kernel: str):
    """The step operator a kernel symbol belongs to, from its template
    arguments (the residual GEMVs: Wo takes inputs of up to 8192 columns, the
    down projection wider ones - the 8B and 70B shapes)."""
    import re
    m = re.search(r"k_gemv<(\d+), (\d+), (\d+), (\d+), (\d+), (?:true|false)>", kernel)
    if m:
        epi, xr = int(m.group(3)), int(m.group(4))
        return {0: "qkv", 2: "gateup", 3: "lmhead"}.get(epi, "down" if xr == 8 else "wo")
    m = re.search(r"k_gemv_mb<(\d+), (\d+), (\d+), (true|false), (?:true|false)>", kernel)
    if m:
        epi, xl = int(m.group(2)), m.group(4) == "true"
        return {0: "qkv", 2: "gateup", 3: "lmhead"}.get(epi, "wo" if xl else "down")
    for key, kind in (("k_attn", "attn"), ("k_embed", "embed"), ("k_xdigits", "digits"),
                      ("k_read_bw", "read_bw"), ("k_dequant", "dequant"), ("k_layer_cos", "layer_cos"),
                      ("k_zero", "zero")):
        if key in kernel:
            return kind
    return None


def _counter_rows(d: str):
    import csv
    import glob
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            yield from csv.DictReader(fh)


def summarize(d: str, workload: str, commands: list):
    """Reads <d>/trace (kernel trace + stats), <d>/fetch and <d>/write
    (FETCH_SIZE / WRITE_SIZE runs with --calibrate) and writes
    profiles/kernels_<workload>.md and profiles/pmc_<workload>.json."""
    import csv
    import glob
    import statistics
    stats = glob.glob(os.path.join(d, "trace", "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(d, "trace", "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        raise SystemExit(f"no kernel trace under {d}/trace")
    rows = list(csv.DictReader(open(stats[0])))
    durs = {}
    for r in csv.DictReader(open(trace[0])):
        k = kind_of(r["Kernel_Name"]) or r["Kernel_Name"]
        durs.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    # HBM counters per dispatch, KiB
    per = {}
    for which, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        for r in _counter_rows(os.path.join(d, which)):
            if r["Counter_Name"] != counter:
                continue
            k = kind_of(r["Kernel_Name"]) or r["Kernel_Name"]
            per.setdefault(k, {}).setdefault(which, []).append(float(r["Counter_Value"]) * 1024.0)
    # calibration: a plain read of 1 GiB, a dequant writing 64 down-projection rows of fp32
    import synth
    cfg = synth.CONFIGS[workload]
    read_ref, write_ref = float(1 << 30), float(64 * cfg.ffn * 4)
    # (the read-ceiling probe reads more than 1 GiB: the calibration read is the smallest)
    reads = per.get("read_bw", {}).get("fetch", [])
    writes = per.get("dequant", {}).get("write", [])
    if not reads or not writes:
        raise SystemExit("calibration dispatches missing (run the counter passes with --calibrate)")
    ff = read_ref / min(reads)
    wf = write_ref / statistics.median(writes)
    table = {}
    for k, e in per.items():
        if k in ("read_bw", "dequant"):
            continue
        f = e.get("fetch", [0.0])
        w = e.get("write", [0.0])
        table[k] = {"fetch": int(ff * statistics.mean(f)), "write": int(wf * statistics.mean(w)),
                    "launches": max(len(f), len(w))}
    out = {"kernel_source_sha256_16": kernel_source_digest(), "workload": workload,
           "calibration": {"fetch_factor": round(ff, 5), "fetch_ref": "k_read_bw over 1 GiB",
                           "write_factor": round(wf, 5),
                           "write_ref": f"k_dequant writing 64*{cfg.ffn}*4 bytes"},
           "per_launch_bytes": table, "commands": commands}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"pmc_{workload}.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    lines = [f"# Kernel time and HBM traffic: {workload} ({WORKLOAD_TEXT[workload]})", "",
             "Commands (repository root, MI355X host; one run each):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "rocprofv3 `kernel_stats` of the trace run (warm-up, the timed graph-replayed steps, the "
              "timing steps with HIP events in the step graph, the one-family timing graphs, the "
              "read-ceiling probe):", "",
              "| operator | kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        k = kind_of(r["Name"]) or "-"
        lines.append(f"| {k} | `{r['Name'][:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    lines += ["", "Median dispatch duration per operator (kernel trace):", "",
              "| operator | dispatches | median us |", "|---|---|---|"]
    for k in sorted(durs, key=lambda k: -statistics.median(durs[k])):
        if k in KERNEL_NAMES or k in ("embed", "digits"):
            lines.append(f"| {k} | {len(durs[k])} | {statistics.median(durs[k]):.2f} |")
    lines += ["", f"HBM counters (FETCH_SIZE and WRITE_SIZE runs; KiB per dispatch x calibration: fetch factor "
              f"{ff:.4f} from k_read_bw reading 1 GiB, write factor {wf:.4f} from k_dequant writing "
              f"{int(write_ref)} bytes):", "",
              "| operator | launches | HBM fetch bytes / launch | HBM write bytes / launch |", "|---|---|---|---|"]
    for k in sorted(table, key=lambda k: -table[k]["fetch"]):
        lines.append(f"| {k} | {table[k]['launches']} | {table[k]['fetch']:,} | {table[k]['write']:,} |")
    lines += ["", f"Kernel sources hashed (lm_kernels.hip, lm_internal.h, lm_device.h): "
              f"{kernel_source_digest()}; bench.py reports `roofline.traffic` from this file only while "
              "that hash matches."]
    with open(os.path.join(ROOT, "profiles", f"kernels_{workload}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote profiles/pmc_{workload}.json and profiles/kernels_{workload}.md")


def host_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))


def cpu_baseline(model, cfg, n_seq: int, budget_s: float, max_steps: int = 64):
    """The oracle as it stands, timed on this host on the same workload."""
    import oracle
    import synth
    om = oracle.OracleModel(model, max_seqs=n_seq, max_ctx=cfg.ctx + max_steps)
    for s in range(n_seq):
        for l in range(cfg.n_layers):
            om.load_kv(s, l, *synth.make_kv(cfg, s, l))
    tok = synth.start_tokens(cfg, n_seq)
    n = 0
    t0 = time.perf_counter()
    while True:
        _, am = om.step(tok)
        tok = am
        n += 1
        if time.perf_counter() - t0 >= budget_s or n >= max_steps:
            break
    dt = time.perf_counter() - t0
    om.close()
    what = "sequence" if n_seq == 1 else f"batch of {n_seq} sequences"
    return {"value": round(n * n_seq / dt, 4), "unit": "tokens/s", "cores": host_threads(), "kind": "oracle",
            "sample": f"{n} greedy decode steps ({what}) of the same model from context {cfg.ctx} "
                      f"({dt:.1f} s, fp64, OpenMP over output rows)",
            "_tokens": n * n_seq, "_seconds": dt}


def public(d):
    return {k: v for k, v in d.items() if not k.startswith("_")}


def side_leg(name: str, fn):
    """Runs an optional measurement; an exception becomes {"error": ...}."""
    try:
        return fn()
    except Exception as e:  # noqa: BLE001 - reported in the line, never fatal
        log(f"{name} failed: {type(e).__name__}: {e}")
        return {"error": f"{type(e).__name__}: {e}"}


def input_digests(model, n_seq: int) -> dict:
    """SHA-256 of every input tensor kind: the global tensors one by one, each
    per-layer kind over its layers' bytes concatenated in layer order, and the
    prefilled KV of every (sequence, layer) in order (K then V)."""
    import synth
    cfg = model.cfg
    out = {"tok_embd": hashlib.sha256(model.tok_embd.tobytes()).hexdigest(),
           "out_norm": hashlib.sha256(model.out_norm.tobytes()).hexdigest(),
           "lm_head": hashlib.sha256(model.lm_head.tobytes()).hexdigest()}
    for kind in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
        h = hashlib.sha256()
        for lw in model.layers:
            h.update(memoryview(getattr(lw, kind)).cast("B"))
        out[f"layers.{kind}"] = h.hexdigest()
    h = hashlib.sha256()
    for s in range(n_seq):
        for l in range(cfg.n_layers):
            k, v = synth.make_kv(cfg, s, l)
            h.update(k.tobytes())
            h.update(v.tobytes())
    out["kv_prefill"] = h.hexdigest()
    out["start_tokens"] = [int(t) for t in synth.start_tokens(cfg, n_seq)]
    return out


class Runner:
    """One opened model with its torch stream and device token buffers."""

    def __init__(self, model, n_seq: int, kv_fn=None, loader=None):
        import torch
        import synth
        import token_decode_llama_amd as lm
        self.cfg = cfg = model.cfg
        self.n_seq = n_seq
        self.stream = torch.cuda.Stream()          # the model's stream (default priority)
        kv_fn = kv_fn or (lambda s, l: synth.make_kv(cfg, s, l))
        if loader is None:
            self.g = lm.open_model(model, kv_fn, max_seqs=n_seq, kv_seqs=n_seq,
                                   stream=self.stream.cuda_stream)
        else:
            self.g = loader(self.stream.cuda_stream)
        dev = torch.device("cuda:0")
        with torch.cuda.stream(self.stream):
            self.tok = torch.from_numpy(synth.start_tokens(cfg, n_seq)).to(dev)
            self.d_tok = self.tok.clone()
        torch.cuda.synchronize()

    def rewind(self):
        import torch
        torch.cuda.synchronize()
        for s in range(self.n_seq):
            self.g.set_position(s, self.cfg.ctx)
        with torch.cuda.stream(self.stream):
            self.d_tok.copy_(self.tok)
        torch.cuda.synchronize()

    def step(self):
        self.g.step_dev(self.d_tok, self.n_seq, self.d_tok)

    def warm(self, n: int):
        import torch
        for _ in range(n):
            self.step()
        torch.cuda.synchronize()
        self.rewind()

    def timed(self, n: int) -> float:
        """ms per step over n steps, HIP events on the model's stream."""
        import torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(n):
            self.step()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def step_percentiles(self, n: int) -> dict:
        """Per-step durations (ms) from an event pair around each of n steps on
        the model's stream (a separate pass: the events add their own cost)."""
        import torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        ev[0].record(self.stream)
        for i in range(n):
            self.step()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        d = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))
        pick = lambda q: d[min(n - 1, int(q * (n - 1) + 0.5))]
        return {"p10": round(pick(0.1), 4), "median": round(pick(0.5), 4), "p90": round(pick(0.9), 4),
                "steps": n}

    def kernel_profile(self, timing_steps: int):
        """Per-kind (launches, total ms) over graph-replayed steps with HIP events
        captured around every kernel inside the step graph, and the algorithmic
        bytes of one step at those steps' mean position."""
        import torch
        import token_decode_llama_amd as lm
        self.rewind()
        # events captured into the step graph: the kernels as the replayed step runs them
        self.g.kernel_timing(2)
        for _ in range(timing_steps):
            self.step()
        torch.cuda.synchronize()
        kstats = {k: self.g.kernel_stats(k) for k in lm.KERNEL_KINDS}
        self.g.kernel_timing(0)
        for s in range(self.n_seq):
            self.g.set_position(s, self.cfg.ctx + timing_steps // 2)
        kbytes = {k: self.g.kernel_bytes(k, self.n_seq) for k in lm.KERNEL_KINDS}
        self.rewind()
        return kstats, kbytes

    def step_bytes(self, at_step: int) -> float:
        import token_decode_llama_amd as lm
        for s in range(self.n_seq):
            self.g.set_position(s, self.cfg.ctx + at_step)
        b = sum(self.g.kernel_bytes(k, self.n_seq) for k in lm.KERNEL_KINDS if k != "copy")
        self.rewind()
        return b

    def close(self):
        self.g.close()


def per_launch(kind: str, n_layers: int) -> int:
    return 1 if kind in ("embed", "lmhead") else n_layers


def graph_times(r, kstats, n_seq: int) -> dict:
    """µs per launch of every kernel family, its launches of one step replayed
    alone as a HIP graph (lm_time_kind) - without the cost of event nodes."""
    out = {}
    for k, (n, _) in kstats.items():
        if n and k != "copy":
            r.rewind()
            out[k] = r.g.time_kind(k, n_seq, 20)
    r.rewind()
    return out


def kernel_table(kstats, kbytes, n_layers, us_graph=None):
    """Per family: launches in the timing steps, µs per launch (graph replay of
    the family alone when given, else the events around each launch in the
    step graph), algorithmic GB/s at that duration."""
    out = {}
    for k, (n, ms) in kstats.items():
        if not n:
            continue
        ev_us = 1e3 * ms / n
        us = us_graph.get(k, ev_us) if us_graph else ev_us
        launches_per_step = per_launch(k, n_layers)
        out[k] = {"launches": n, "avg_us": round(us, 3),
                  "algorithmic_GBps": round((kbytes[k] / launches_per_step) / (us * 1e-6) / 1e9, 1)
                  if kbytes[k] else None,
                  "avg_us_events_in_step": round(ev_us, 3)}
    return out


def roofline_for(kind, kstats, kbytes, n_layers, workload, us_graph=None):
    """Algorithmic bytes per launch / average launch duration.  The duration is
    the family's launches replayed as the step graph runs them, between two HIP
    events on the model's stream (us_graph); without it, the per-launch events
    of the timing steps (which add the events' own cost to every launch)."""
    n, ms = kstats[kind]
    per_launch_bytes = kbytes[kind] / per_launch(kind, n_layers)
    avg_ms = us_graph * 1e-3 if us_graph else ms / max(n, 1)
    achieved = per_launch_bytes / (avg_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_from_profiles(kind, workload),
            "kernel": KERNEL_NAMES.get(kind, kind), "bytes_per_launch": int(per_launch_bytes),
            "avg_launch_us": round(avg_ms * 1e3, 3)}


def dominant(kstats):
    """The compute kind with the largest summed duration."""
    return max((k for k in kstats if k not in ("copy", "embed")), key=lambda k: kstats[k][1])


# The arithmetic of the GEMVs: int8 (or 4-bit) weights times the activations'
# 24-bit fixed-point digits in exact int32 block sums, the two block scales
# and the sums combined in fp32; attention, norms and softmax in fp32.
DTYPE = "int8 weights x int24 activation digits -> int32 block sums, fp32 accumulation"


def base_line(metric, tps, ms_per_step, steps, warmup, step_bytes, config, dtype=DTYPE):
    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    return {"metric": metric, "value": round(tps, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
            "achieved_hbm_GBps": round(gbps, 1), "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
            "step_bytes": int(step_bytes), "config": config}


# ---------------------------------------------------------------------------
def speculative(model, rounds: int = 12, k: int = 3) -> dict:
    """Self-speculative rounds on sequence 0 of the same model opened for four
    sequences: k = 3 drafts through the bottom 8 of 32 layers, verified by one
    pass of all layers over 4 columns; and drafts by all 32 layers (every draft
    accepted: the verify pass's own rate).  Host-clocked, each round blocks.
    The model is opened with room for every round: a round advances the
    position by at most k + 1, and the warm-up round comes on top."""
    import synth
    import token_decode_llama_amd as lm
    cfg = model.cfg
    max_ctx = cfg.ctx + (rounds + 1) * (k + 1)
    g = lm.open_model(model, lambda s, l: synth.make_kv(cfg, s, l), max_seqs=4, kv_seqs=1, max_ctx=max_ctx)
    res = {"k": k, "max_ctx": max_ctx}
    try:
        for label, d in (("draft_8_of_32", 8), ("draft_all_32", cfg.n_layers)):
            g.set_position(0, cfg.ctx)
            t = int(synth.start_tokens(cfg, 1)[0])
            acc = g.speculative_step(t, d, k)         # warm-up round
            g.set_position(0, cfg.ctx)
            n_tok = 0
            t0 = time.perf_counter()
            for _ in range(rounds):
                acc = g.speculative_step(t, d, k)
                n_tok += len(acc)
                t = int(acc[-1])
            dt = time.perf_counter() - t0
            res[label] = {"draft_layers": d, "rounds": rounds, "tokens": n_tok,
                          "tokens_per_round": round(n_tok / rounds, 3), "ms_per_round": round(1e3 * dt / rounds, 3),
                          "tokens_per_s": round(n_tok / dt, 2)}
            log(f"speculative {label}: {n_tok} tokens in {rounds} rounds, {n_tok / dt:.1f} tok/s")
    finally:
        g.close()
    res["note"] = ("random weights: the bottom layers rarely predict the full model's token, so the acceptance "
                   "rate says nothing about trained models; the all-layer draft bounds the verify pass")
    return res


def run_single(args, name: str, n_seq: int):
    """llama8b_q8 (headline, batch 1) and llama8b_q4 (four sequences)."""
    import synth
    base = synth.CONFIGS[name]
    extra = max(args.steps, args.warmup, args.timing_steps, 1)
    cfg = synth.variant(name, steps=extra)
    log(f"generating {name} ({cfg.weight_bytes() / 1e9:.2f} GB of quantized weights)")
    model = synth.make_model(cfg)
    log("loading into HBM")
    r = Runner(model, n_seq)
    r.warm(args.warmup)                                     # also captures the step graph
    ms_per_step = None
    if not args.only_kernels:
        ms_per_step = r.timed(args.steps)
        log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step")
    kstats, kbytes = r.kernel_profile(args.timing_steps)
    L = cfg.n_layers
    dom = dominant(kstats)
    ug = graph_times(r, kstats, n_seq)
    roofline = roofline_for(dom, kstats, kbytes, L, name, ug[dom])
    roofline["timing"] = ("the family's launches of one step captured alone as a HIP graph and replayed 20 "
                          "times between two HIP events on the model's stream")
    roofline["avg_launch_us_events_in_step"] = round(1e3 * kstats[dom][1] / max(kstats[dom][0], 1), 3)
    step_bytes = r.step_bytes(args.steps // 2)
    # read ceiling (the GEMVs' non-temporal 16-byte loads) over (at most) 4 GiB of the resident layer arena
    n_read = min(4 << 30, (cfg.weight_bytes() - cfg.vocab * synth.row_bytes(cfg.qtype, cfg.hidden)) // 16 * 16)
    read_ms = r.g.debug_read_bw(n_read, 5)
    if args.calibrate:
        r.g.debug_read_bw(1 << 30, 1)
        r.g.debug_dequant(0, 6, 0, 64, cfg.ffn)
        log(f"calibration: read {1 << 30} bytes; dequant wrote {64 * cfg.ffn * 4} bytes")
    qt = synth.QTYPE_NAMES[cfg.qtype]
    spec_ok = cfg.qtype in (synth.Q8_0, synth.Q4_0)      # the verify pass runs on the several-sequence path
    config = {"workload": WORKLOAD_TEXT[name], "name": name, "batch": n_seq, "ctx": base.ctx, "qtype": qt,
              "weights": "random N(0,0.02), quantized, resident in HBM"}
    metric = HEADLINE_METRIC if name == "llama8b_q8" else \
        f"decode tokens/s (aggregate over {n_seq} sequences) + achieved HBM GB/s, 8B-shape {qt} batch {n_seq}"
    if ms_per_step is not None:
        out = base_line(metric, 1000.0 * n_seq / ms_per_step, ms_per_step, args.steps, args.warmup,
                        step_bytes, config)
    else:
        out = {"metric": metric, "config": config}
    out["roofline"] = roofline
    out["read_ceiling_GBps"] = round(n_read / (read_ms * 1e-3) / 1e9, 1)
    if ms_per_step is not None and name == "llama8b_q8":
        # the engine page's own figure for this workload (section 1 table): another machine's, context only
        out["vs_baseline"] = round(out["value"] / PAGES_8B_Q8_TOKS, 2)
        out["vs_baseline_basis"] = (f"{PAGES_8B_Q8_TOKS} tok/s: the C/CUDA Llama engine page's Llama 3.1 8B Q8_0 "
                                    "decode with every layer in GPU memory, on an RTX 3090 with trained weights; "
                                    "another machine's number, quoted as context, not a target")
    if ms_per_step is not None:
        out["pct_read_ceiling"] = round(100.0 * out["achieved_hbm_GBps"] / out["read_ceiling_GBps"], 2)
        r.rewind()
        out["step_ms_percentiles"] = r.step_percentiles(min(args.steps, 32))
        r.rewind()
    out["kernels"] = kernel_table(kstats, kbytes, L, ug)
    out["inputs_sha256"] = input_digests(model, n_seq)
    # The headline fields are complete here.  The CPU baseline and the opt-in
    # side legs below only add fields: a failure in one of them becomes an
    # "error" entry of its own and never discards the headline.
    extras = n_seq == 1 and spec_ok and not args.only_kernels and args.extras
    r.close()
    if extras:
        out["speculative"] = side_leg("speculative", lambda: speculative(model))
    if not args.no_cpu_baseline and not args.only_kernels:
        log("oracle baseline")
        out["cpu_baseline"] = side_leg("cpu_baseline",
                                       lambda: public(cpu_baseline(model, cfg, n_seq, args.cpu_budget)))
    return out


def run_multi(args):
    """Three models resident together, decoded round-robin on three streams."""
    import torch
    import synth
    names = ["multi_llama1b", "multi_qwen05b", "multi_smol360m"]
    extra = max(args.steps, args.warmup, args.timing_steps, 1)
    cfgs = [synth.variant(n, steps=extra) for n in names]
    models, runners = [], []
    for c in cfgs:
        log(f"generating {c.name} ({c.weight_bytes() / 1e9:.2f} GB)")
        models.append(synth.make_model(c))
        runners.append(Runner(models[-1], 1))
    for r in runners:
        r.warm(args.warmup)
    # each model alone
    solo = {}
    for r in runners:
        solo[r.cfg.name] = r.timed(args.steps)
        r.rewind()
    # round-robin on three streams
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for r in runners:
            r.step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_round = wall_ms / args.steps
    log(f"round-robin: {ms_per_round:.4f} ms per round of 3 tokens; solo ms/step {solo}")
    for r in runners:
        r.rewind()
    round_bytes = sum(r.step_bytes(args.steps // 2) for r in runners)
    # kernel profile of the largest model (eager, alone)
    kstats, kbytes = runners[0].kernel_profile(args.timing_steps)
    dom = dominant(kstats)
    ug = graph_times(runners[0], kstats, 1)
    config = {"workload": WORKLOAD_TEXT["multi"], "name": "multi", "batch": 1, "ctx": 2048, "qtype": "Q8_0",
              "models": names, "weights": "random N(0,0.02), quantized, resident in HBM"}
    out = base_line("decode tokens/s aggregate over three concurrently resident Q8_0 models "
                    "(round-robin, one HIP stream each)", 3000.0 / ms_per_round, ms_per_round, args.steps,
                    args.warmup, round_bytes, config)
    out["per_model_solo_tokens_per_s"] = {k: round(1000.0 / v, 2) for k, v in solo.items()}
    out["roofline"] = roofline_for(dom, kstats, kbytes, cfgs[0].n_layers, "multi_llama1b", ug[dom])
    out["roofline"]["model"] = names[0]
    out["kernels"] = kernel_table(kstats, kbytes, cfgs[0].n_layers, ug)
    for r in runners:
        r.close()
    if not args.no_cpu_baseline:
        log("oracle baseline (the three models in turn)")
        per = [cpu_baseline(m, c, 1, args.cpu_budget / 3, max_steps=32) for m, c in zip(models, cfgs)]
        tot_s = sum(p["_seconds"] for p in per)
        n_tok = sum(p["_tokens"] for p in per)
        out["cpu_baseline"] = {"value": round(n_tok / tot_s, 4), "unit": "tokens/s", "cores": host_threads(),
                               "kind": "oracle",
                               "sample": "; ".join(f"{n}: {p['sample']}" for n, p in zip(names, per))}
    return out


def run_70b(args, name="llama70b_q4"):
    """(a) resident in HBM, (b) layer streaming from pinned host memory, (c) the
    engine page's split for the format (Q4_0 and Q4_K: the first 36 layers
    resident and the other 44 streamed; Q6_K: 26 and 54), (d) streamed with the
    20 most similar layers skipped."""
    import numpy as np
    import torch
    import synth
    import token_decode_llama_amd as lm
    extra = max(args.steps, args.warmup, args.timing_steps, 1)
    cfg = synth.variant(name, steps=extra)
    s, H, V = cfg.seed, cfg.hidden, cfg.vocab
    log(f"generating {name} ({cfg.weight_bytes() / 1e9:.2f} GB of quantized weights), layer by layer")
    model = synth.Model(cfg=cfg,
                        tok_embd=synth.normal_f16_bits(s, synth.tensor_id(cfg, synth.T_EMBD), V * H, 0.0,
                                                       0.02).reshape(V, H),
                        out_norm=synth.normal_f32(s, synth.tensor_id(cfg, synth.T_OUT_NORM), H, 1.0, 0.1),
                        lm_head=synth.quant_matrix(s, synth.tensor_id(cfg, synth.T_LM_HEAD), V, H, 0.02,
                                                   cfg.qtype))
    keep = not args.no_cpu_baseline

    def loader(stream):
        g = lm.Model(cfg, max_seqs=1, stream=stream)
        for l in range(cfg.n_layers):
            w = synth.make_layer(cfg, l)
            g.load_layer(l, w)
            if keep:
                model.layers.append(w)
            if l % 10 == 9:
                log(f"  layer {l + 1}/{cfg.n_layers} loaded")
        g.load_global(model.tok_embd, model.out_norm, model.lm_head)
        for l in range(cfg.n_layers):
            g.load_kv(0, l, *synth.make_kv(cfg, 0, l))
        return g

    r = Runner(model, 1, loader=loader)
    r.warm(args.warmup)
    ms_res = r.timed(args.steps)
    log(f"resident: {ms_res:.3f} ms/step")
    kstats, kbytes = r.kernel_profile(args.timing_steps)
    step_bytes = r.step_bytes(args.steps // 2)
    dom = dominant(kstats)
    ug = graph_times(r, kstats, 1)
    roof = roofline_for(dom, kstats, kbytes, cfg.n_layers, name, ug[dom])
    ktab = kernel_table(kstats, kbytes, cfg.n_layers, ug)
    # the resident step's compute time per step (eager, from the kernel events)
    compute_ms = sum(ms for k, (n, ms) in kstats.items() if k != "copy") / args.timing_steps

    log("switching to layer streaming")
    r.g.stream_mode(True)
    r.warm(1)
    n_st = args.stream_steps
    ms_st = r.timed(n_st)
    log(f"streaming: {ms_st:.3f} ms/step")
    # copy and compute event totals over streamed steps
    r.rewind()
    r.g.kernel_timing(True)
    ms_st_timed = r.timed(n_st)          # wall time of the same instrumented steps
    sk = {k: r.g.kernel_stats(k) for k in lm.KERNEL_KINDS}
    r.g.kernel_timing(False)
    copy_bytes = r.g.kernel_bytes("copy", 1)
    r.rewind()
    t_copy = sk["copy"][1] / n_st
    t_comp = sum(ms for k, (n, ms) in sk.items() if k != "copy") / n_st
    overlap = (t_copy + t_comp - ms_st_timed) / min(t_copy, t_comp) if min(t_copy, t_comp) > 0 else None
    # the serial baseline, measured: every layer copied, then computed, nothing ahead
    r.g.stream_mode(2)
    r.warm(1)
    ms_serial = r.timed(n_st)
    log(f"streaming, serial copy then compute: {ms_serial:.3f} ms/step")
    r.g.stream_mode(True)
    r.rewind()
    qt = synth.QTYPE_NAMES[cfg.qtype]
    k_h = HYBRID_RESIDENT[name]
    config = {"workload": WORKLOAD_TEXT[name], "name": name, "batch": 1, "ctx": cfg.ctx, "qtype": qt,
              "weights": "random N(0,0.02), quantized; (a) resident in HBM, (b) streamed per layer from "
                         f"pinned host memory, (c) first {k_h} layers resident, the other "
                         f"{cfg.n_layers - k_h} streamed"}
    out = base_line(f"decode tokens/s + achieved HBM GB/s, 70B-shape {qt} batch 1, weights resident in HBM",
                    1000.0 / ms_res, ms_res, args.steps, args.warmup, step_bytes, config)
    out["roofline"] = roof
    out["kernels"] = ktab
    out["streaming"] = {
        "value": round(1000.0 / ms_st, 4), "unit": "tokens/s", "steps": n_st, "ms_per_step": round(ms_st, 2),
        "host_link_GBps": round(copy_bytes / (ms_st * 1e-3) / 1e9, 2),
        "copy_only_GBps": round(copy_bytes / (t_copy * 1e-3) / 1e9, 2) if t_copy else None,
        "layer_blob_bytes": int(copy_bytes / cfg.n_layers),
        "sum_copy_ms": round(t_copy, 2), "sum_compute_ms": round(t_comp, 3),
        "instrumented_wall_ms": round(ms_st_timed, 2),
        "serial_copy_then_compute_ms": round(t_copy + t_comp, 2),
        "serial_measured_ms_per_step": round(ms_serial, 2),
        "serial_measured_tokens_per_s": round(1000.0 / ms_serial, 4),
        "speedup_over_serial": round(ms_serial / ms_st, 3),
        "overlap_fraction": round(overlap, 4) if overlap is not None else None,
        "overlap_definition": "(sum copy + sum compute - wall) / min(sum copy, sum compute), per step, all "
                              "three from the same steps with HIP events around every copy and kernel",
        "resident_compute_ms_eager": round(compute_ms, 3)}
    # (c) hybrid residency: the pages' 70B split for this format (Q4_K_M: 36 of
    # 80 layers in GPU memory; Q6_K: 26); and what the tier sizing rule gives
    # for a 24 GiB card
    log(f"hybrid: {k_h} of {cfg.n_layers} layers resident")
    r.g.set_residency(k_h)
    r.warm(1)
    ms_h = r.timed(n_st)
    copy_h = r.g.kernel_bytes("copy", 1)
    log(f"hybrid: {ms_h:.3f} ms/step")
    out["hybrid"] = {
        "value": round(1000.0 / ms_h, 4), "unit": "tokens/s", "steps": n_st, "ms_per_step": round(ms_h, 2),
        "n_resident": k_h, "n_streamed": cfg.n_layers - k_h,
        "host_link_GBps": round(copy_h / (ms_h * 1e-3) / 1e9, 2),
        "tier_a_for_24GiB": r.g.plan_residency(hbm_bytes=24 << 30, host_bytes=1 << 40)}
    # (d) layer skip, streamed: the similarity of every layer's input and output
    # recorded over 2 steps, then the 20 most similar of 80 layers skipped (the
    # pages' 70B figure skips 20 of 80); skipped layers are not copied
    r.g.set_residency(0)
    r.rewind()
    r.g.layer_similarity(True)
    for _ in range(2):
        r.step()
    torch.cuda.synchronize()
    r.g.layer_similarity(False)
    mean, _ = r.g.get_layer_similarity()
    order = np.sort(mean)[::-1]
    n_skip = 20
    thr = float((order[n_skip - 1] + order[n_skip]) / 2)
    skipped = r.g.skip_similar_layers(thr)
    r.warm(1)
    ms_sk = r.timed(n_st)
    copy_sk = r.g.kernel_bytes("copy", 1)
    log(f"streaming, {skipped} layers skipped: {ms_sk:.3f} ms/step")
    out["layer_skip"] = {
        "value": round(1000.0 / ms_sk, 4), "unit": "tokens/s", "steps": n_st, "ms_per_step": round(ms_sk, 2),
        "mode": "all layers streamed", "n_skipped": skipped, "threshold": round(thr, 6),
        "similarity_min_max": [round(float(np.nanmin(mean)), 6), round(float(np.nanmax(mean)), 6)],
        "host_link_GBps": round(copy_sk / (ms_sk * 1e-3) / 1e9, 2),
        "calibration": "mean input/output cosine similarity per layer over 2 greedy steps; the list skips the "
                       "layers above a threshold set between the 20th and 21st largest mean"}
    r.g.set_layer_skip(None)
    r.close()
    if keep:
        log("oracle baseline (bounded sample)")
        out["cpu_baseline"] = public(cpu_baseline(model, cfg, 1, args.cpu_budget, max_steps=2))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: the workload's own)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama8b_q8",
                    choices=["llama8b_q8", "llama8b_q4", "multi", "llama70b_q4", "llama8b_q4k",
                             "llama8b_q5k", "llama8b_q6k", "llama70b_q4k", "llama70b_q6k"])
    ap.add_argument("--timing-steps", type=int, default=8,
                    help="eager steps with per-kernel HIP events for the roofline")
    ap.add_argument("--stream-steps", type=int, default=16, help="timed steps in layer-streaming mode (70B)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extras", action="store_true",
                    help="also time self-speculative rounds (batch-1 Q8_0/Q4_0 workloads)")
    ap.add_argument("--only-kernels", action="store_true",
                    help="skip the timed loop: run the per-kernel timing steps only (for profilers)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run two calibration dispatches of known traffic for HBM counters: "
                         "a plain read of 1 GiB (k_read_bw) and a dequant of 64 down-projection rows "
                         "that writes 64*ffn*4 bytes (k_dequant)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="no GPU: reduce rocprofv3 output of this script under DIR (trace/, fetch/, write/) "
                         "to profiles/kernels_<workload>.md and profiles/pmc_<workload>.json")
    ap.add_argument("--command", action="append", default=[],
                    help="(with --summarize) a command that produced DIR, recorded in the summary")
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize, args.workload, args.command)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(the per-GPU throughput is the --gpus 1 figure)", file=sys.stderr)
        sys.exit(2)
    if args.steps is None:
        args.steps = {"llama8b_q8": 64, "llama8b_q4": 32, "multi": 32, "llama70b_q4": 16, "llama8b_q4k": 64,
                      "llama8b_q5k": 64, "llama8b_q6k": 64, "llama70b_q4k": 16, "llama70b_q6k": 16}[args.workload]

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.workload == "llama8b_q8":
        out = run_single(args, "llama8b_q8", 1)
    elif args.workload == "llama8b_q4":
        out = run_single(args, "llama8b_q4", 4)
    elif args.workload in ("llama8b_q4k", "llama8b_q5k", "llama8b_q6k"):
        out = run_single(args, args.workload, 1)
    elif args.workload == "multi":
        out = run_multi(args)
    else:
        out = run_70b(args, args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
