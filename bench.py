#!/usr/bin/env python3
"""Decode-layer benchmark on one MI355X: us per layer step and achieved HBM GB/s.

A step is one pass of the whole hot path over one batch of synthetic tokens
(b = 1 by default, d = 7168): attention input projection 7168 -> 12288,
output projection 8192 -> 7168 with residual add and RMSNorm, router scores
over E = 384 experts with top-8 renormalised softmax, latent projection
7168 -> 7168, the 8 routed SwiGLU experts (I = 2048) behind the token
permutation and the shared expert (folded into the routed kernels; the
two-stream form and the side-stream prefetch are timed beside the step).
Weights are bf16, synthetic and seeded; they and the inputs are resident in
HBM before timing starts.

Cold-cache discipline: steps rotate over --layers independent copies of the
layer's weights (about 35 GB each) and a pool of 16 token batches, so no
weight a step reads is still in the 256 MB MALL from an earlier step.

Timing: W eager warm-up steps, then a pass of K eager steps with an event
after each step and trace events around every launch of the dominant kernel
(the routed gate/up kernel, on the stream it runs on) for its average
duration; then the timed region proper: exactly K steps captured in one HIP
graph and replayed once, between events on the replay stream, synchronised on
both sides. ROCm does not allow timing events inside a captured graph, which
is why the kernel is timed in the eager pass.

Value = algorithmic bytes per step / time per step (weights touched once plus
activations in and out), in GB/s; peak = 8 TB/s (MI355X HBM3E).

Prints one JSON line on stdout; progress goes to stderr.
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

PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_moe_up_b1_traffic.json")
DOMINANT_SOURCES = ["moe_router_topk_amd/csrc/moe_b1.hip", "moe_router_topk_amd/csrc/k3_gemv.h",
                    "moe_router_topk_amd/csrc/k3_device.h"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ byte accounting
def moe_bytes(cfg, b: int, n_active: int) -> int:
    """Algorithmic bytes of one MoE block pass: each weight once, plus the
    activations each kernel boundary hands over (written once, read once)."""
    d, E, I, Is, dl, k = cfg.d, cfg.E, cfg.I, cfg.I_s, cfg.d_lat, cfg.k
    weights = 2 * (E * d + dl * d + 3 * Is * d + n_active * (2 * I * dl + d * I))
    if cfg.zipf_bias:
        weights += 4 * E
    acts = (2 * b * d                      # x
            + 2 * (4 * b * E)              # logits out and in
            + 2 * (8 * b * k)              # ids + weights out and in
            + 2 * (2 * b * dl)             # z out and in
            + 2 * (2 * b * k * I)          # routed h out and in
            + 2 * (2 * b * Is)             # shared h out and in
            + 2 * (4 * b * d)              # y_s out and in
            + 2 * b * d)                   # y out
    return weights + acts


def chain_bytes(cc, b: int) -> int:
    weights = 2 * (cc.n_in * cc.d + cc.d * cc.k_o + cc.d)
    acts = (2 * b * cc.d                   # x
            + 2 * b * cc.n_in + 2 * b * cc.k_o   # q out, a in
            + 2 * (2 * b * cc.d)           # residual in and out
            + 2 * (4 * b * cc.d)           # fp32 h out and in
            + 2 * b * cc.d)                # normalised hidden state out
    return weights + acts


def gateup_bytes(cfg, b: int, n_active: int) -> int:
    """Per launch of the kernel traced as the routed experts' gate/up pass:
    n_active experts' [2I x d_lat] weights, the z rows it reads and the h rows
    it writes. At batch 1 that kernel (k_moe_up_b1) also selects the experts:
    + the logits it reads, the ids and weights it writes."""
    dl, I, E, k = cfg.d_lat, cfg.I, cfg.E, cfg.k
    n = 2 * n_active * 2 * I * dl + 2 * b * dl + 2 * b * k * I
    if b == 1:
        n += 4 * E + 8 * k
    return n


def gateup_kernel_name(b: int) -> str:
    if b == 1:
        return "k_moe_up_b1<true> (expert selection + routed gate/up + SwiGLU)"
    if b <= 4:
        return "routed gate/up + SwiGLU (dot2 rows for light experts, MFMA tiles for heavy)"
    return "routed gate/up + SwiGLU, every expert on MFMA tiles (k_sk_gemm_stream)"


def sources_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_per_launch():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None when it is missing or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != sources_digest(DOMINANT_SOURCES):
        return None
    return t.get("traffic_bytes_per_launch")


PMC_RUNS = {
    "fetch": ("FETCH_SIZE", "--steps 5 --warmup 2 --eager-only --layers 2"),
    "write": ("WRITE_SIZE", "--steps 5 --warmup 2 --eager-only --layers 2"),
    "copy_fetch": ("FETCH_SIZE", "--copy-mb 256"),
    "copy_write": ("WRITE_SIZE", "--copy-mb 256"),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_MB = 256


def pmc_values(run_dir: str, counter: str, name_part: str):
    """Per-dispatch values (KiB) of one counter for kernels whose name holds
    name_part, from a rocprofv3 --pmc csv directory."""
    import csv
    import glob
    vals = []
    for f in sorted(glob.glob(os.path.join(run_dir, "*counter_collection.csv"))):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]))
    return vals


def write_traffic_summary(pmc_dir: str) -> int:
    """Reduce the four counter runs under pmc_dir (pmc_fetch, pmc_write,
    pmc_copy_fetch, pmc_copy_write, made by the commands recorded in the
    output) to HBM bytes per launch of the dominant kernel at b = 1."""
    import synth
    name = "k_moe_up_b1<true"
    fetch = pmc_values(os.path.join(pmc_dir, "pmc_fetch"), "FETCH_SIZE", name)
    write = pmc_values(os.path.join(pmc_dir, "pmc_write"), "WRITE_SIZE", name)
    cf = pmc_values(os.path.join(pmc_dir, "pmc_copy_fetch"), "FETCH_SIZE", COPY_KERNEL)
    cw = pmc_values(os.path.join(pmc_dir, "pmc_copy_write"), "WRITE_SIZE", COPY_KERNEL)
    if not (fetch and write and cf and cw):
        print("bench.py: counter runs missing under " + pmc_dir, file=sys.stderr)
        return 2
    copied = COPY_MB << 20
    # the copy reads and writes `copied` bytes; take its largest dispatch
    fetch_scale = copied / (max(cf) * 1024)
    write_scale = copied / (max(cw) * 1024)
    f_kib = sum(fetch) / len(fetch)
    w_kib = sum(write) / len(write)
    traffic = int(round(f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale))
    algo = gateup_bytes(synth.MOE_CONFIGS["b1"], 1, synth.MOE_CONFIGS["b1"].k)
    out = {
        "kernel": "k3::k_moe_up_b1<true> (expert selection + routed gate/up + SwiGLU), "
                  "batch 1, d=7168, E=384, k=8, I=2048",
        "commands": [
            f"rocprofv3 --pmc {ctr} --output-format csv -d {pmc_dir}/pmc_{key} -o c -- "
            f"python3 -u bench.py {args}" for key, (ctr, args) in PMC_RUNS.items()
        ] + [f"python3 bench.py --traffic-summary {pmc_dir}"],
        "dispatches_averaged": {"FETCH_SIZE": len(fetch), "WRITE_SIZE": len(write)},
        "fetch_kib_per_dispatch": round(f_kib, 1),
        "write_kib_per_dispatch": round(w_kib, 1),
        "copy_calibration": {
            "bytes_copied": copied, "kernel": COPY_KERNEL,
            "fetch_kib": round(max(cf), 1), "write_kib": round(max(cw), 1),
            "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
        },
        "traffic_bytes_per_launch": traffic,
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": round(traffic / algo, 4),
        "source_sha256": sources_digest(DOMINANT_SOURCES),
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")
    print(json.dumps(out))
    return 0


def print_counter_summary(pmc_dir: str) -> int:
    """Per-kernel means (per dispatch) of every counter in the rocprofv3 --pmc
    csv files under pmc_dir, printed as a markdown table."""
    import csv
    import glob
    acc = {}
    for f in sorted(glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"),
                              recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].split("(")[0]
                if "k3::" not in name:
                    continue
                key = (name, r["Counter_Name"])
                acc.setdefault(key, []).append(float(r["Counter_Value"]))
    if not acc:
        print("bench.py: no k3 counter rows under " + pmc_dir, file=sys.stderr)
        return 2
    counters = sorted({c for _, c in acc})
    print("| Kernel | dispatches | " + " | ".join(counters) + " |")
    print("|---|---|" + "---|" * len(counters))
    for name in sorted({n for n, _ in acc}):
        vals = [acc.get((name, c)) for c in counters]
        n = max(len(v) for v in vals if v)
        cells = [f"{sum(v) / len(v):.4g}" if v else "" for v in vals]
        print(f"| `{name}` | {n} | " + " | ".join(cells) + " |")
    return 0


# ------------------------------------------------------------------ timing helpers
def read_ceiling(torch, k3, t, nbytes: int, reps: int = 7) -> float:
    """GB/s of k3_stream_read over the first nbytes of t: the median of reps
    event-timed reads."""
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        k3.k3_stream_read(t, nbytes)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return nbytes / (pct(ts, 0.5) * 1e-3) / 1e9


def capture(torch, fn, n: int):
    """Capture fn(i) for i < n into one graph."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def replay_timed(torch, g, n: int):
    """One replay of an n-step graph between events on the replay stream,
    synchronised on both sides: (ms per step, wall seconds)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n, time.perf_counter() - t0


def eager_timed(torch, k3, fn, n: int):
    """n host-launched steps with an event after each and the routed gate/up
    kernel bracketed by trace events: (ms per step, per-step ms sorted,
    gate/up ms per launch)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    kb = [k3.HipEvent() for _ in range(n)]
    ke = [k3.HipEvent() for _ in range(n)]
    torch.cuda.synchronize()
    ev[0].record()
    try:
        for i in range(n):
            k3.k3_trace_events("moe_experts", kb[i], ke[i])
            fn(i)
            ev[i + 1].record()
    finally:
        k3.k3_trace_events("moe_experts", None, None)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))
    kern = [kb[i].elapsed_ms(ke[i]) for i in range(n)]
    return ev[0].elapsed_time(ev[n]) / n, per, kern


def pct(v, q):
    return v[min(len(v) - 1, int(q * len(v)))]


# ------------------------------------------------------------------ main
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--zipf", type=float, default=0.0,
                    help="Zipf exponent of the router bias for the main step (0: none)")
    ap.add_argument("--layers", type=int, default=2, help="weight copies rotated per step")
    ap.add_argument("--prefetch", action="store_true",
                    help="run the side-stream prefetch inside the timed step")
    ap.add_argument("--cu-shared", type=int, default=0, help="CU budget of the shared expert")
    ap.add_argument("--prefetch-cu", type=int, default=32, help="CU budget of the prefetch")
    ap.add_argument("--no-sweep", action="store_true", help="skip the b = 1..64 sweep")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager-only", action="store_true",
                    help="time host-launched steps only (no graph, sweep or CPU leg); "
                         "for profiler counter runs")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    ap.add_argument("--traffic-summary", metavar="DIR", default="",
                    help="no GPU work: reduce the rocprofv3 counter runs under DIR to the "
                         "dominant kernel's HBM bytes per launch (written under profiles/)")
    ap.add_argument("--counter-summary", metavar="DIR", default="",
                    help="no GPU work: per-kernel means of every counter in the rocprofv3 "
                         "--pmc csv files under DIR, as a markdown table")
    args = ap.parse_args()
    if args.traffic_summary:
        return write_traffic_summary(args.traffic_summary)
    if args.counter_summary:
        return print_counter_summary(args.counter_summary)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; there is no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        return 2
    if not 1 <= args.steps <= 2000:
        print("bench.py: --steps must be in 1..2000", file=sys.stderr)
        return 2

    import torch

    import synth
    import moe_router_topk_amd as k3
    from moe_router_topk_amd.layer import DecodeLayer

    k3.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_mb:
        n = args.copy_mb * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_mb} MiB x3")
        return 0

    cfg = synth.MOE_CONFIGS["b1"]
    cc = synth.CHAIN_CONFIG
    b = args.batch
    t_gen = time.perf_counter()
    layers = []
    for li in range(args.layers):
        mw = synth.make_moe_weights(cfg, device=dev, layer=li)
        cw = synth.make_chain_weights(cc, device=dev, layer=li)
        layers.append(DecodeLayer(mw, cfg.k, b_max=64, chain=cw, eps=cc.eps,
                                  cu_shared=args.cu_shared, prefetch_cu=args.prefetch_cu))
        log(f"layer {li}: weights generated")
    if args.zipf > 0:
        zbias = synth.zipf_router_bias(cfg.E, args.zipf, cfg.seed).to(dev)
        for lay in layers:
            lay.moe["bias"] = zbias
        cfg = synth.MOE_CONFIGS["b64zipf"]  # the same layer with the bias counted
    NX = 16
    pool = [synth.make_chain_inputs(cc, 64, device=dev, index=i) for i in range(NX)]
    torch.cuda.synchronize()
    log(f"weights + inputs ready in {time.perf_counter() - t_gen:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")
    prefetch = args.prefetch

    # the measured streaming-read ceiling: 4 GiB of expert weights read once
    # with the weight streams' non-temporal loads (k3_stream_read)
    ceil_bytes = min(4 << 30, layers[0].moe["w13"].numel() * 2)
    ceiling = read_ceiling(torch, k3, layers[0].moe["w13"], ceil_bytes)
    log(f"streaming-read ceiling: {ceiling:.0f} GB/s over {ceil_bytes / 2**30:.1f} GiB")

    def step(i, bb=b):
        lay = layers[i % len(layers)]
        inp = pool[i % NX]
        return lay.step(inp["x"][:bb], inp["r"][:bb], prefetch=prefetch)

    # ---- warm-up (eager) and routing statistics
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n_act = []
    for i in range(NX):
        step(i)
        ids = layers[i % len(layers)].ids[:b]
        n_act.append(int(torch.unique(ids).numel()))
    torch.cuda.synchronize()
    log(f"warm-up done; distinct experts per step: {sorted(set(n_act))}")

    # ---- eager pass: per-step events and the dominant kernel's launches
    K = args.steps
    eager_ms, per, kern_ms = eager_timed(torch, k3, step, K)
    kern_avg = sum(kern_ms) / K

    # ---- timed region: exactly K steps in one graph, one replay
    if args.eager_only:
        ms, wall = eager_ms, float("nan")
        args.no_sweep = args.no_cpu_baseline = True
    else:
        g = capture(torch, step, K)
        ms, wall = replay_timed(torch, g, K)
        del g
    mean_act = sum(n_act[i % NX] for i in range(K)) / K
    bytes_step = moe_bytes(cfg, b, mean_act) + chain_bytes(cc, b)
    gbs = bytes_step / (ms * 1e-3) / 1e9
    log(f"layer step b={b}: {ms * 1e3:.1f} us/step in the graph, {gbs:.0f} GB/s "
        f"({100 * gbs / PEAK_GBS:.1f}% of peak); eager {eager_ms * 1e3:.1f} us/step "
        f"(median {pct(per, 0.5) * 1e3:.1f}, p90 {pct(per, 0.9) * 1e3:.1f}); "
        f"wall {wall * 1e3:.1f} ms for {K} steps")
    gu_bytes = gateup_bytes(cfg, b, mean_act)
    gu_gbs = gu_bytes / (kern_avg * 1e-3) / 1e9
    log(f"routed gate/up kernel: {kern_avg * 1e3:.1f} us avg over {K} launches, "
        f"{gu_gbs:.0f} GB/s")

    # ---- MoE block alone (the block the 70%-of-peak target names)
    def block(i, bb=b):
        lay = layers[i % len(layers)]
        return lay.moe_block(pool[i % NX]["x"][:bb])

    for i in range(4):
        block(i)
    if args.eager_only:
        moe_ms = eager_timed(torch, k3, block, K)[0]
    else:
        g = capture(torch, block, K)
        moe_ms, _ = replay_timed(torch, g, K)
        del g
    moe_gbs = moe_bytes(cfg, b, mean_act) / (moe_ms * 1e-3) / 1e9
    log(f"MoE block b={b}: {moe_ms * 1e3:.1f} us, {moe_gbs:.0f} GB/s "
        f"({100 * moe_gbs / PEAK_GBS:.1f}% of peak)")

    # the other configurations, for comparison (graph-timed like the step)
    def step_alt(i):
        lay = layers[i % len(layers)]
        return lay.step(pool[i % NX]["x"][:b], pool[i % NX]["r"][:b], prefetch=not prefetch)

    step_alt(0)
    g = capture(torch, step_alt, K)
    alt_ms, _ = replay_timed(torch, g, K)
    del g

    def block_streams(i, bb=b):
        lay = layers[i % len(layers)]
        return lay.moe_block_streams(pool[i % NX]["x"][:bb])

    block_streams(0)
    g = capture(torch, block_streams, K)
    streams_ms, _ = replay_timed(torch, g, K)
    del g
    log(f"step with prefetch {'off' if prefetch else 'on'}: {alt_ms * 1e3:.1f} us; "
        f"MoE block as two-stream composition: {streams_ms * 1e3:.1f} us")

    extra = {"moe_block_us": round(moe_ms * 1e3, 2), "moe_block_GBps": round(moe_gbs, 1),
             ("step_us_prefetch_off" if prefetch else "step_us_prefetch_on"):
                 round(alt_ms * 1e3, 2),
             "moe_block_two_stream_us": round(streams_ms * 1e3, 2),
             "moe_block_frac_of_peak": round(moe_gbs / PEAK_GBS, 4),
             "moe_block_frac_of_read_ceiling": round(moe_gbs / ceiling, 4),
             "eager_step_us": round(eager_ms * 1e3, 2),
             "eager_step_us_median": round(pct(per, 0.5) * 1e3, 2),
             "eager_step_us_p10": round(pct(per, 0.1) * 1e3, 2),
             "eager_step_us_p90": round(pct(per, 0.9) * 1e3, 2),
             "bytes_per_step": int(bytes_step), "n_active_mean": mean_act}

    # ---- sweep: MoE block and layer step at b = 4, 8, 16, 32 (uniform) and 64 (Zipf
    # bias); chain b = 1..64
    if not args.no_sweep:
        sweep = []
        S = 40
        bias = synth.zipf_router_bias(cfg.E, 1.1, cfg.seed).to(dev)
        for bb, zipf in ((4, False), (8, False), (16, False), (32, False), (64, True)):
            for lay in layers:
                lay.moe["bias"] = bias if zipf else None
            acts = []
            for i in range(NX):
                block(i, bb)
                acts.append(int(torch.unique(layers[i % len(layers)].ids[:bb]).numel()))
            g = capture(torch, lambda i: block(i, bb), S)
            ts, _ = replay_timed(torch, g, S)
            del g
            us = ts * 1e3
            na = sum(acts[i % NX] for i in range(S)) / S
            by = moe_bytes(synth.MOE_CONFIGS["b64zipf" if zipf else "b16"], bb, na)
            sweep.append({"what": "moe_block", "b": bb, "routing": "zipf1.1" if zipf else "uniform",
                          "us": round(us, 1), "n_active_mean": na,
                          "GBps": round(by / us / 1e3, 1),
                          "frac_of_peak": round(by / us / 1e3 / PEAK_GBS, 4),
                          "frac_of_read_ceiling": round(by / us / 1e3 / ceiling, 4)})
            log(f"MoE block b={bb} {'zipf' if zipf else 'uniform'}: {us:.1f} us, "
                f"n_active {na:.1f}, {by / us / 1e3:.0f} GB/s")
            # the whole layer step at this batch: chain, then the block on its output
            acts = []
            for i in range(NX):
                step(i, bb)
                acts.append(int(torch.unique(layers[i % len(layers)].ids[:bb]).numel()))
            g = capture(torch, lambda i: step(i, bb), S)
            ts, _ = replay_timed(torch, g, S)
            del g
            us = ts * 1e3
            na = sum(acts[i % NX] for i in range(S)) / S
            by = moe_bytes(synth.MOE_CONFIGS["b64zipf" if zipf else "b16"], bb, na) + \
                chain_bytes(cc, bb)
            entry = {"what": "layer_step", "b": bb,
                     "routing": "zipf1.1" if zipf else "uniform", "us": round(us, 1),
                     "n_active_mean": na, "GBps": round(by / us / 1e3, 1),
                     "frac_of_peak": round(by / us / 1e3 / PEAK_GBS, 4),
                     "frac_of_read_ceiling": round(by / us / 1e3 / ceiling, 4)}
            if not args.no_cpu_baseline:
                # the oracle beside it: one layer step at this batch on the host cores
                cfg_b = synth.MOE_CONFIGS["b64zipf" if zipf else "b16"]
                oms, othr, oby = oracle_step(layers[0], cfg_b, cc, pool[0], bb)
                entry["oracle"] = {"ms_per_step": round(oms, 1), "cores": othr,
                                   "GBps": round(oby / oms / 1e6, 3), "steps": 1}
                log(f"oracle layer step b={bb}: {oms:.0f} ms on {othr} threads")
            sweep.append(entry)
            log(f"layer step b={bb} {'zipf' if zipf else 'uniform'}: {us:.1f} us, "
                f"n_active {na:.1f}, {by / us / 1e3:.0f} GB/s")
        for lay in layers:
            lay.moe["bias"] = None

        def chain(i, bb):
            lay = layers[i % len(layers)]
            inp = pool[i % NX]
            return lay.attn_chain(inp["x"][:bb], inp["r"][:bb])

        for bb in synth.CHAIN_BATCHES:
            chain(0, bb)
            g = capture(torch, lambda i: chain(i, bb), S)
            ts, _ = replay_timed(torch, g, S)
            del g
            us = ts * 1e3
            by = chain_bytes(cc, bb)
            sweep.append({"what": "chain", "b": bb, "us": round(us, 1),
                          "GBps": round(by / us / 1e3, 1),
                          "frac_of_peak": round(by / us / 1e3 / PEAK_GBS, 4),
                          "frac_of_read_ceiling": round(by / us / 1e3 / ceiling, 4)})
            log(f"chain b={bb}: {us:.1f} us, {by / us / 1e3:.0f} GB/s")
        extra["sweep"] = sweep

    # ---- CPU baseline: the oracle, timed on this host's cores
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, layers[0], cfg, cc, pool, b, args.cpu_seconds)

    out = {
        "metric": "MoE decode layer us/step and achieved HBM GB/s (% of peak), batch 1-64",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "frac_of_peak": round(gbs / PEAK_GBS, 4),
        "frac_of_read_ceiling": round(gbs / ceiling, 4),
        "read_ceiling": {"GBps": round(ceiling, 1), "bytes": int(ceil_bytes),
                         "kernel": "k3_stream_read: non-temporal 128-bit loads, one workgroup "
                                   "per compute unit"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 weights and tokens, rotated over "
                f"{args.layers} weight copies and {NX} token batches)",
        "config": {
            "workload": (f"decode layer step at batch {b}: attention in-proj 7168->12288, "
                         "o-proj 8192->7168 + residual + RMSNorm, router E=384 top-8 "
                         "renormalised softmax, latent 7168->7168, 8 routed + 1 shared "
                         "SwiGLU experts I=2048 (gate/up [4096x7168], down [7168x2048]), "
                         "side-stream prefetch " + ("on" if prefetch else "off")
                         + (f", Zipf({args.zipf}) router bias" if args.zipf > 0 else "")),
            "batch": b, "d": cfg.d, "E": cfg.E, "top_k": cfg.k, "I": cfg.I,
            "prefetch": prefetch, "hip_graph": not args.eager_only,
            "layers_rotated": args.layers,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": gateup_kernel_name(b),
            "achieved": round(gu_gbs, 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gu_gbs / PEAK_GBS, 4),
            "frac_of_read_ceiling": round(gu_gbs / ceiling, 4),
            "traffic": traffic_per_launch() if b == 1 else None,
            "bytes_per_launch": int(gu_bytes),
            "avg_launch_us": round(kern_avg * 1e3, 2),
        },
        "cpu_baseline": cpu,
    }
    out.update(extra)
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(torch, layer, cfg, cc, pool, b, seconds):
    """Time the oracle (plain fp64 C, all host cores) on whole layer steps at
    batch b, as many as fit in about `seconds` (at least one)."""
    import numpy as np

    import oracle

    L = oracle.lib()
    threads = oracle.threads()
    host = {k: (v.cpu() if v is not None else None) for k, v in layer.moe.items()
            if k not in ("w13", "w2")}
    ch = {k: v.cpu() for k, v in layer.chain_w.items()}
    experts = {}

    def fetch(e):
        if e not in experts:
            experts[e] = (layer.moe["w13"][e].cpu(), layer.moe["w2"][e].cpu())
        return experts[e]

    done, spent, i, nbytes = 0, 0.0, 0, 0
    while done < 2000 and (done == 0 or spent < seconds):
        inp = pool[i % len(pool)]
        x, r = inp["x"][:b].cpu(), inp["r"][:b].cpu()
        # host copies of what this step reads (outside the timed part)
        hm = oracle.chain(x, r, ch["w_in"], ch["w_o"], ch["gamma"], cc.eps)["y"]
        ids, _ = oracle.topk_softmax(oracle.router_logits(hm, host["w_router"]), cfg.k)
        for e in np.unique(ids):
            fetch(int(e))
        t0 = time.perf_counter()
        c = oracle.chain(x, r, ch["w_in"], ch["w_o"], ch["gamma"], cc.eps)
        oracle.moe_block(c["y"], host, cfg.k, expert_weights=fetch)
        dt = time.perf_counter() - t0
        nbytes += moe_bytes(cfg, b, len(np.unique(ids))) + chain_bytes(cc, b)
        spent += dt
        done += 1
        i += 1
    sec = spent / done
    log(f"oracle: {done} steps, {sec * 1e3:.1f} ms/step on {threads} threads")
    del L
    return {"value": round(nbytes / spent / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "ms_per_step": round(sec * 1e3, 2),
            "sample": f"{done} whole layer steps at batch {b} (chain + MoE block, "
                      f"{cfg.k} routed experts each), fp64 C oracle with OpenMP"}


def oracle_step(layer, cfg, cc, inp, b):
    """One whole layer step of the oracle (plain fp64 C, all host cores) at
    batch b: (ms, threads, bytes of the step). The experts it reads are copied
    to the host before the clock starts."""
    import numpy as np

    import oracle

    threads = oracle.threads()
    host = {k: (v.cpu() if v is not None else None) for k, v in layer.moe.items()
            if k not in ("w13", "w2")}
    ch = {k: v.cpu() for k, v in layer.chain_w.items()}
    x, r = inp["x"][:b].cpu(), inp["r"][:b].cpu()
    hm = oracle.chain(x, r, ch["w_in"], ch["w_o"], ch["gamma"], cc.eps)["y"]
    ids, _ = oracle.topk_softmax(oracle.router_logits(hm, host["w_router"], host["bias"]),
                                 cfg.k)
    experts = {int(e): (layer.moe["w13"][int(e)].cpu(), layer.moe["w2"][int(e)].cpu())
               for e in np.unique(ids)}
    t0 = time.perf_counter()
    c = oracle.chain(x, r, ch["w_in"], ch["w_o"], ch["gamma"], cc.eps)
    oracle.moe_block(c["y"], host, cfg.k, expert_weights=lambda e: experts[e])
    dt = time.perf_counter() - t0
    nbytes = moe_bytes(cfg, b, len(experts)) + chain_bytes(cc, b)
    return dt * 1e3, threads, nbytes


if __name__ == "__main__":
    sys.exit(main())
