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
TRACE_FILE = os.path.join(ROOT, "profiles", "layer_step_b1_kernel_trace.json")
TRACE_MD = os.path.join(ROOT, "profiles", "layer_step_b1_kernel_stats.md")
NX = 16  # token batches rotated through the steps
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
    it writes. At batch 1 that kernel (k_moe_up_b1) also selects the experts
    and, ahead of the routed rows, streams the shared expert's gate/up rows:
    + the logits it reads, the ids and weights it writes, the shared
    [2 I_s x d] weights, the x row it reads and the h_s row it writes."""
    dl, I, E, k = cfg.d_lat, cfg.I, cfg.E, cfg.k
    n = 2 * n_active * 2 * I * dl + 2 * b * dl + 2 * b * k * I
    if b == 1:
        n += 4 * E + 8 * k
        n += 2 * 2 * cfg.I_s * cfg.d + 2 * cfg.d + 2 * cfg.I_s
    return n


def gateup_kernel_name(b: int) -> str:
    if b == 1:
        return "k_moe_up_b1<true> (shared gate/up, expert selection, routed gate/up + SwiGLU)"
    if b <= 4:
        return "routed gate/up + SwiGLU (dot2 rows for light experts, MFMA tiles for heavy)"
    return "routed gate/up + SwiGLU, every expert on MFMA tiles (k_sk_gemm_stream)"


def sources_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_trace():
    """The committed rocprofv3 kernel-trace summary of the default step, or
    {} when it is missing or the dominant kernel's sources changed since."""
    try:
        with open(TRACE_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    if t.get("source_sha256") != sources_digest(DOMINANT_SOURCES):
        return {}
    return t


# the kernels of one batch-1 layer step, once each, in launch order
STEP_B1_KERNELS = ["k_gemv<7, 1,", "k_oproj_gemv<", "k_rls_gemv<7, 1, true",
                   "k_moe_up_b1<true", "k_down_b1<"]


def write_trace_summary(trace_dir: str, warmup: int, steps: int, out_json: str = TRACE_FILE,
                        out_md: str = TRACE_MD) -> int:
    """Reduce the kernel trace of a default bench run (rocprofv3 --kernel-trace,
    csv) to per-kernel statistics over all dispatches and over the timed
    region: the K steps of the one graph replay the line's time comes from.
    Each step kernel runs once per step, and before the timed replay come the
    warm-up steps, the NX routing-statistics steps and the K eager steps, so
    dispatches [warmup + NX + K, warmup + NX + 2K) of each are the replay's."""
    import csv
    import glob
    import statistics as st
    files = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"),
                             recursive=True))
    if not files:
        print("bench.py: no kernel_trace.csv under " + trace_dir, file=sys.stderr)
        return 2
    rows = []
    for fn in files:
        with open(fn, newline="") as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    allk = {}
    for r in rows:
        name = r["Kernel_Name"].split("(")[0]
        if "k3::" in name:
            allk.setdefault(name, []).append(r)
    i0 = warmup + NX + steps
    region = {}
    for pat in STEP_B1_KERNELS:
        hits = [n for n in allk if pat in n]
        if len(hits) != 1 or len(allk[hits[0]]) < i0 + steps:
            print(f"bench.py: step kernel {pat} not found {i0 + steps} times", file=sys.stderr)
            return 2
        region[hits[0]] = allk[hits[0]][i0:i0 + steps]

    def dur(r):
        return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0

    first = region[[n for n in region if STEP_B1_KERNELS[0] in n][0]][0]
    last = region[[n for n in region if STEP_B1_KERNELS[-1] in n][0]][-1]
    span_us = (int(last["End_Timestamp"]) - int(first["Start_Timestamp"])) / 1000.0
    dom = [n for n in region if STEP_B1_KERNELS[3] in n][0]
    dom_d = [dur(r) for r in region[dom]]
    cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o kt -- "
           f"python3 -u bench.py --steps {steps} --warmup {warmup} --no-sweep "
           f"--no-cpu-baseline")
    out = {
        "command": cmd,
        "summary_command": f"python3 bench.py --trace-summary {trace_dir} --steps {steps} "
                           f"--warmup {warmup}",
        "timed_region_steps": steps,
        "timed_region_us_per_step": round(span_us / steps, 2),
        "dominant_kernel": dom,
        "dominant_timed_region_avg_us": round(sum(dom_d) / len(dom_d), 2),
        "dominant_timed_region_median_us": round(st.median(dom_d), 2),
        "dominant_all_dispatches_avg_us": round(
            sum(dur(r) for r in allk[dom]) / len(allk[dom]), 2),
        "source_sha256": sources_digest(DOMINANT_SOURCES),
    }
    with open(out_json, "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")
    lines = [
        "# Kernel trace of the batch-1 layer step (rocprofv3)",
        "",
        "Command (on the GPU box, from the repository root):",
        "",
        "    " + cmd,
        "    " + out["summary_command"],
        "",
        f"Timed region: the {steps} graph-replayed steps the bench line's time comes from "
        f"(dispatches {i0}..{i0 + steps - 1} of each step kernel; warm-up {warmup}, "
        f"{NX} routing-statistics steps and {steps} eager steps come first). Trace span "
        f"from the first step's input projection to the last step's down projection: "
        f"{span_us / steps:.2f} us per step.",
        "",
        "| Kernel (timed region) | dispatches | avg us | median us | min us | max us |",
        "|---|---|---|---|---|---|",
    ]
    for n in region:
        d = [dur(r) for r in region[n]]
        lines.append(f"| `{n}` | {len(d)} | {sum(d) / len(d):.2f} | {st.median(d):.2f} | "
                     f"{min(d):.2f} | {max(d):.2f} |")
    lines += ["", "| Kernel (every dispatch of the run: eager and graph-replayed) | dispatches "
              "| avg us | median us |", "|---|---|---|---|"]
    for n, rs in sorted(allk.items(), key=lambda kv: -sum(dur(r) for r in kv[1])):
        d = [dur(r) for r in rs]
        lines.append(f"| `{n}` | {len(d)} | {sum(d) / len(d):.2f} | {st.median(d):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(out))
    return 0


def host_info() -> dict:
    """What the oracle's timings ran on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        nproc = os.cpu_count()
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "nproc": nproc,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


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
        "kernel": "k3::k_moe_up_b1<true> (shared gate/up, expert selection, routed gate/up + SwiGLU), "
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
    ap.add_argument("--no-sweep", action="store_true", help="skip the b = 2..64 sweep")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager-only", action="store_true",
                    help="host-launched steps on one stream only: no HIP graph is captured, "
                         "no side stream runs, no sweep or CPU leg; for profiler counter runs")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    ap.add_argument("--traffic-summary", metavar="DIR", default="",
                    help="no GPU work: reduce the rocprofv3 counter runs under DIR to the "
                         "dominant kernel's HBM bytes per launch (written under profiles/)")
    ap.add_argument("--counter-summary", metavar="DIR", default="",
                    help="no GPU work: per-kernel means of every counter in the rocprofv3 "
                         "--pmc csv files under DIR, as a markdown table")
    ap.add_argument("--mall-probe", action="store_true",
                    help="only time the o-projection cold, after k3_prefetch of its weights "
                         "and warm (what the prefetch leaves in the MALL)")
    ap.add_argument("--router-fusion", action="store_true",
                    help="only time the batch-1 router + top-k as two kernels (default) and "
                         "as one kernel whose last workgroup selects (K3_VARIANT_LASTWG)")
    ap.add_argument("--shard-probe", action="store_true",
                    help="only time the kernels at one GPU's share under tensor parallelism "
                         "over 8 GPUs (experts I = 256, input projection 1536 rows, "
                         "o-projection K = 1024)")
    ap.add_argument("--trace-summary", metavar="DIR", default="",
                    help="no GPU work: reduce the rocprofv3 kernel trace of a default run "
                         "(same --steps/--warmup) to per-kernel statistics of its timed "
                         "region (written under profiles/)")
    args = ap.parse_args()
    if args.traffic_summary:
        return write_traffic_summary(args.traffic_summary)
    if args.counter_summary:
        return print_counter_summary(args.counter_summary)
    if args.trace_summary:
        return write_trace_summary(args.trace_summary, args.warmup, args.steps)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; there is no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        return 2
    if not 1 <= args.steps <= 2000:
        print("bench.py: --steps must be in 1..2000", file=sys.stderr)
        return 2
    if args.eager_only:
        args.no_sweep = args.no_cpu_baseline = True
        if args.prefetch:
            print("bench.py: --eager-only runs one stream; drop --prefetch", file=sys.stderr)
            return 2

    import torch

    import synth
    import moe_router_topk_amd as k3
    from moe_router_topk_amd.layer import DecodeLayer

    k3.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.mall_probe:
        print(json.dumps(mall_probe(torch, k3, synth)), flush=True)
        return 0
    if args.router_fusion:
        print(json.dumps(router_fusion(torch, k3, synth)), flush=True)
        return 0
    if args.shard_probe:
        print(json.dumps(shard_probe(torch, k3, synth)), flush=True)
        return 0

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

    extra = {"moe_block_us": round(moe_ms * 1e3, 2), "moe_block_GBps": round(moe_gbs, 1),
             "moe_block_frac_of_peak": round(moe_gbs / PEAK_GBS, 4),
             "moe_block_frac_of_read_ceiling": round(moe_gbs / ceiling, 4),
             "eager_step_us": round(eager_ms * 1e3, 2),
             "eager_step_us_median": round(pct(per, 0.5) * 1e3, 2),
             "eager_step_us_p10": round(pct(per, 0.1) * 1e3, 2),
             "eager_step_us_p90": round(pct(per, 0.9) * 1e3, 2),
             "bytes_per_step": int(bytes_step), "n_active_mean": mean_act}

    # the other configurations, for comparison (graph-timed like the step);
    # both use a second stream, so a counter run (--eager-only) skips them
    if not args.eager_only:
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
        extra[("step_us_prefetch_off" if prefetch else "step_us_prefetch_on")] = \
            round(alt_ms * 1e3, 2)
        extra["moe_block_two_stream_us"] = round(streams_ms * 1e3, 2)

    # ---- the tiny workload (d = 256, E = 8, top-2, I = 128): launch-bound, its
    # weights sit in the caches; us only
    if not args.no_sweep:
        tcfg = synth.MOE_CONFIGS["tiny"]
        tw = synth.make_moe_weights(tcfg, device=dev)
        tl = DecodeLayer(tw, tcfg.k, b_max=1)
        tx = [synth.make_tokens(tcfg, device=dev, index=i, b=1) for i in range(NX)]
        tl.moe_block(tx[0])
        g = capture(torch, lambda i: tl.moe_block(tx[i % NX]), K)
        tiny_ms, _ = replay_timed(torch, g, K)
        del g
        extra["tiny"] = {"what": "moe_block", "b": 1, "d": tcfg.d, "E": tcfg.E,
                         "top_k": tcfg.k, "I": tcfg.I, "us": round(tiny_ms * 1e3, 2),
                         "note": "launch-bound (about 725 KB of weights, cache-resident); "
                                 "no GB/s claim"}
        log(f"tiny MoE block b=1: {tiny_ms * 1e3:.2f} us")

    # ---- sweep: MoE block and layer step at b = 2, 4 and the verify batches
    # 8 r (r = 1..8) with uniform routing, b = 64 with the Zipf(1.1) router
    # bias; chain b = 1..64. The oracle runs beside some of them on the host.
    oracle_runs = []
    hw = None if args.no_cpu_baseline else HostWeights(layers[0])
    main_bias = layers[0].moe["bias"]
    if not args.no_sweep:
        sweep = []
        S = 40
        zbias64 = synth.zipf_router_bias(cfg.E, 1.1, cfg.seed).to(dev)
        cases = [(bb, False) for bb in SWEEP_UNIFORM] + [(64, True)]
        if not args.no_cpu_baseline:
            # host copies first (no copies while the GPU is timed); the
            # single-thread oracle steps then run in host threads beside the
            # GPU sweep
            log("oracle: preparing host copies for the sweep batches")
            oracle_runs = [OracleStep(hw, cfg.k, cc, pool[0], bb, zbias64 if zipf else None,
                                      synth.MOE_CONFIGS["b64zipf" if zipf else "b16"])
                           for bb, zipf in ORACLE_CASES]
            threads = start_single_thread_runs(oracle_runs, reps=3)
        for bb, zipf in cases:
            for lay in layers:
                lay.moe["bias"] = zbias64 if zipf else None
            cfg_b = synth.MOE_CONFIGS["b64zipf" if zipf else "b16"]
            acts, hist = [], {}
            for i in range(NX):
                block(i, bb)
                ids_i = layers[i % len(layers)].ids[:bb]
                acts.append(int(torch.unique(ids_i).numel()))
                cnt = torch.bincount(ids_i.reshape(-1).long(), minlength=cfg.E)
                for c, nexp in zip(*torch.unique(cnt[cnt > 0], return_counts=True)):
                    hist[int(c)] = hist.get(int(c), 0) + int(nexp)
            g = capture(torch, lambda i: block(i, bb), S)
            ts, _ = replay_timed(torch, g, S)
            del g
            us = ts * 1e3
            na = sum(acts[i % NX] for i in range(S)) / S
            by = moe_bytes(cfg_b, bb, na)
            routing = "zipf1.1" if zipf else "uniform"
            entry = {"what": "moe_block", "b": bb, "routing": routing, "us": round(us, 1),
                     "n_active_mean": na, "GBps": round(by / us / 1e3, 1),
                     "frac_of_peak": round(by / us / 1e3 / PEAK_GBS, 4),
                     "frac_of_read_ceiling": round(by / us / 1e3 / ceiling, 4),
                     "tokens_per_expert_hist": {str(c): round(n / NX, 2)
                                                for c, n in sorted(hist.items())}}
            if bb % 8 == 0 and not zipf:
                entry["verify_requests"] = bb // 8
            sweep.append(entry)
            log(f"MoE block b={bb} {routing}: {us:.1f} us, n_active {na:.1f}, "
                f"{by / us / 1e3:.0f} GB/s")
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
            by = moe_bytes(cfg_b, bb, na) + chain_bytes(cc, bb)
            sweep.append({"what": "layer_step", "b": bb, "routing": routing, "us": round(us, 1),
                          "n_active_mean": na, "GBps": round(by / us / 1e3, 1),
                          "frac_of_peak": round(by / us / 1e3 / PEAK_GBS, 4),
                          "frac_of_read_ceiling": round(by / us / 1e3 / ceiling, 4)})
            log(f"layer step b={bb} {routing}: {us:.1f} us, n_active {na:.1f}, "
                f"{by / us / 1e3:.0f} GB/s")
        for lay in layers:
            lay.moe["bias"] = main_bias

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
        if oracle_runs:
            for t in threads:
                t.join()
            # all host cores, once the single-thread runs are done
            for o in oracle_runs:
                o.time_all_cores(reps=3)
            for o in oracle_runs:
                for e in sweep:
                    if (e["what"] == "layer_step" and e["b"] == o.b
                            and (e["routing"] == "zipf1.1") == (o.bias is not None)):
                        e["oracle"] = o.report()
                        log(f"oracle layer step b={o.b}: {o.report()}")
        extra["sweep"] = sweep

    # ---- CPU baseline: the oracle, timed on this host's cores
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, hw, cfg, cc, pool, b, args.cpu_seconds,
                           tiny=extra.get("tiny"))

    tr = committed_trace() if b == 1 and not args.zipf else {}
    rocprof_us = tr.get("dominant_timed_region_avg_us")
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
            "traffic": traffic_per_launch() if b == 1 and not args.zipf else None,
            "bytes_per_launch": int(gu_bytes),
            "avg_launch_us": round(kern_avg * 1e3, 2),
            "avg_launch_us_source": "HIP events on the kernel's stream around each of the "
                                    f"{K} eager launches of this run (frac uses this)",
            "avg_launch_us_rocprof_all_dispatches": tr.get("dominant_all_dispatches_avg_us"),
            "avg_launch_us_in_graph_rocprof": rocprof_us,
            "frac_in_graph_rocprof": (round(gu_bytes / (rocprof_us * 1e-6) / 1e9 / PEAK_GBS, 4)
                                      if rocprof_us else None),
            "rocprof_source": "profiles/layer_step_b1_kernel_trace.json: rocprofv3 kernel "
                              "trace of this command without the sweep; all dispatches of the "
                              "kernel, and those of the timed graph replay",
        },
        "cpu_baseline": cpu,
    }
    out.update(extra)
    print(json.dumps(out), flush=True)
    return 0


def mall_probe(torch, k3, synth, reps=7) -> dict:
    """What k3_prefetch leaves in the MALL for the operator that follows. The
    o-projection (W_o, 117 MB) is timed with HIP events: cold (after 1 GiB of
    allocating reads of other memory), after k3_prefetch of all or the first
    half of W_o, and warm (right after itself); then 117 MB reads of W_o
    themselves, allocating (k3_prefetch) and non-temporal (k3_stream_read),
    cold and after an allocating read. Medians of reps, in us."""
    import statistics as st
    dev = "cuda:0"
    cc = synth.CHAIN_CONFIG
    cw = synth.make_chain_weights(cc, device=dev)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    wo_bytes = cw["w_o"].numel() * 2
    out = {"what": "o-projection W_o [7168 x 8192] bf16 (117.4 MB) after MALL preparation",
           "flush": "k3_prefetch over 1 GiB of other memory before every mode"}

    def timed(fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    for b in (1, 16):
        a = synth.randn_bf16((b, cc.k_o), 1.0, 0, "pf_a", b, device=dev)
        r = synth.randn_bf16((b, cc.d), 1.0, 0, "pf_r", b, device=dev)
        ws = torch.empty(k3.workspace_size("oproj_residual", b=b, K=cc.k_o, d=cc.d),
                         dtype=torch.uint8, device=dev)
        yn = torch.empty((b, cc.d), dtype=torch.bfloat16, device=dev)

        def oproj():
            k3.k3_oproj_residual(a, cw["w_o"], r, cw["gamma"], cc.eps, y_norm=yn, workspace=ws)

        res = {}
        for _ in range(reps):
            for mode in ("cold", "prefetched", "prefetched_half", "warm"):
                k3.k3_prefetch(flush)
                if mode == "prefetched":
                    k3.k3_prefetch(cw["w_o"])
                elif mode == "prefetched_half":
                    k3.k3_prefetch(cw["w_o"], nbytes=wo_bytes // 2)
                elif mode == "warm":
                    oproj()
                torch.cuda.synchronize()
                res.setdefault(mode, []).append(timed(oproj))
        out[f"oproj_b{b}_us"] = {m: round(st.median(v), 1) for m, v in res.items()}
        log(f"o-proj b={b}: {out[f'oproj_b{b}_us']}")
    t = {"prefetch_cold": [], "prefetch_after_prefetch": [], "stream_read_cold": [],
         "stream_read_after_prefetch": []}
    for _ in range(reps):
        for mode in t:
            k3.k3_prefetch(flush)
            if mode.endswith("after_prefetch"):
                k3.k3_prefetch(cw["w_o"])
            torch.cuda.synchronize()
            if mode.startswith("prefetch"):
                t[mode].append(timed(lambda: k3.k3_prefetch(cw["w_o"])))
            else:
                t[mode].append(timed(lambda: k3.k3_stream_read(cw["w_o"])))
    out["w_o_read_us"] = {m: round(st.median(v), 1) for m, v in t.items()}
    log(f"117 MB reads of W_o: {out['w_o_read_us']}")
    return out


def router_fusion(torch, k3, synth, n=100, reps=7) -> dict:
    """The batch-1 router scores + top-k (384 experts x 7168, top-8) two ways:
    the default projection kernel followed by the top-k kernel, and the forced
    last-workgroup variant (one kernel: every workgroup publishes its logits
    with a release fence and takes a ticket; the last one acquires and
    selects). Each is captured as n calls (two weight copies alternating, so
    the 5.5 MB of router rows are not cache-resident) and replayed reps times,
    alternating; medians in us per call."""
    import statistics as st
    dev = "cuda:0"
    cfg = synth.MOE_CONFIGS["b1"]
    ws_ = [synth.make_moe_weights(cfg, device=dev, layer=li) for li in range(2)]
    xs = [synth.make_tokens(cfg, device=dev, index=i, b=1) for i in range(4)]
    nbytes = k3.workspace_size("router_topk", b=1, E=cfg.E)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    ids = torch.empty((1, cfg.k), dtype=torch.int32, device=dev)
    wts = torch.empty((1, cfg.k), dtype=torch.float32, device=dev)

    def call(i):
        k3.k3_router_topk(xs[i % 4], ws_[i % 2]["w_router"], None, cfg.k, topk_ids=ids,
                          topk_w=wts, workspace=ws)

    graphs = {}
    for name in ("two_kernels", "last_workgroup"):
        k3.k3_force_variant("router_topk", "lastwg" if name == "last_workgroup" else "none")
        for i in range(8):
            call(i)
        graphs[name] = capture(torch, call, n)
    k3.k3_force_variant("router_topk", "none")
    t = {name: [] for name in graphs}
    for _ in range(reps):
        for name, g in graphs.items():
            t[name].append(replay_timed(torch, g, n)[0] * 1e3)
    out = {"what": "batch-1 router (384 x 7168 bf16) + top-8 selection, graph-replayed",
           "calls_per_replay": n,
           "us_per_call": {name: round(st.median(v), 2) for name, v in t.items()}}
    log(f"router + top-k at b=1: {out['us_per_call']}")
    return out


def shard_probe(torch, k3, synth, n=50, reps=5) -> dict:
    """One GPU's share of the layer under tensor parallelism over 8 GPUs, as
    the kernels would run it before their collectives (not run here): the
    routed experts and the shared expert at I = I_s = 256, the input
    projection's 1536 of 12288 rows, the o-projection's 1024 of 8192 K
    columns (+ residual + norm). Graph-replayed calls; weight copies rotate
    so that each call reads its weights from HBM (the dense shares: 20
    copies, 440 and 294 MB; the experts: two layers, tokens rotating).
    Medians in us per call, GB/s of algorithmic bytes."""
    import statistics as st
    dev = "cuda:0"
    cfg = synth.MOE_CONFIGS["tp8_shard"]
    cc = synth.CHAIN_CONFIG
    mw = [synth.make_moe_weights(cfg, device=dev, layer=li) for li in range(2)]
    cw = synth.make_chain_weights(cc, device=dev)
    w_in = [cw["w_in"][:1536].clone() for _ in range(20)]
    w_o = [cw["w_o"][:, :1024].contiguous() for _ in range(20)]
    del cw["w_in"], cw["w_o"]
    xs = [synth.make_tokens(cfg, device=dev, index=i, b=64) for i in range(8)]
    bias = synth.zipf_router_bias(cfg.E, 1.1, cfg.seed).to(dev)
    out = {"what": "kernels at one GPU's TP8 share, before their collectives",
           "calls_per_replay": n}

    def timed(fn):
        for i in range(4):
            fn(i)
        g = capture(torch, fn, n)
        return st.median(replay_timed(torch, g, n)[0] * 1e3 for _ in range(reps))

    expert_bytes = 2 * (2 * cfg.I * cfg.d + cfg.d * cfg.I)
    for b, zipf in ((1, False), (16, False), (64, True)):
        ids_all, wts_all, zs = [], [], []
        for i in range(8):
            x = xs[i][:b]
            ids, wts = k3.k3_router_topk(x, mw[i % 2]["w_router"], bias if zipf else None, cfg.k)
            ids_all.append(ids)
            wts_all.append(wts)
            zs.append(k3.k3_proj_skinny(x, mw[i % 2]["w_lat"]))
        torch.cuda.synchronize()
        n_act = st.mean(int(torch.unique(t).numel()) for t in ids_all)
        y = torch.empty((b, cfg.d), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(k3.workspace_size("moe_experts", b=b, d_in=cfg.d, E=cfg.E, k=cfg.k,
                                           I=cfg.I, d_out=cfg.d), dtype=torch.uint8, device=dev)
        us = timed(lambda i: k3.k3_moe_experts(zs[i % 8], ids_all[i % 8], wts_all[i % 8],
                                               mw[i % 2]["w13"], mw[i % 2]["w2"], y=y,
                                               workspace=ws))
        by = n_act * expert_bytes
        key = f"routed_experts_b{b}" + ("_zipf" if zipf else "")
        out[key] = {"us": round(us, 2), "n_active": round(n_act, 1),
                    "GBps": round(by / us / 1e3, 1)}
        log(f"TP8 share, routed experts b={b}: {out[key]}")
    for b in (1, 16, 64):
        y_s = torch.empty((b, cfg.d), dtype=torch.float32, device=dev)
        ws = torch.empty(k3.workspace_size("shared_expert", b=b, d=cfg.d, I=cfg.I_s),
                         dtype=torch.uint8, device=dev)
        us = timed(lambda i: k3.k3_shared_expert(xs[i % 8][:b], mw[i % 2]["w13_s"],
                                                 mw[i % 2]["w2_s"], y_s=y_s, workspace=ws))
        out[f"shared_expert_b{b}"] = {"us": round(us, 2),
                                      "GBps": round(expert_bytes / us / 1e3, 1)}
        q = torch.empty((b, 1536), dtype=torch.bfloat16, device=dev)
        wsp = torch.empty(k3.workspace_size("proj_skinny", b=b, K=cc.d, N=1536),
                          dtype=torch.uint8, device=dev)
        us = timed(lambda i: k3.k3_proj_skinny(xs[i % 8][:b], w_in[i % 20], y=q, workspace=wsp))
        out[f"in_proj_1536_b{b}"] = {"us": round(us, 2),
                                     "GBps": round(2 * 1536 * cc.d / us / 1e3, 1)}
        a = synth.randn_bf16((b, 1024), 1.0, 0, "shard_a", b, device=dev)
        r = synth.randn_bf16((b, cc.d), 1.0, 0, "shard_r", b, device=dev)
        yn = torch.empty((b, cc.d), dtype=torch.bfloat16, device=dev)
        wso = torch.empty(k3.workspace_size("oproj_residual", b=b, K=1024, d=cc.d),
                          dtype=torch.uint8, device=dev)
        us = timed(lambda i: k3.k3_oproj_residual(a, w_o[i % 20], r, cw["gamma"], cc.eps,
                                                  y_norm=yn, workspace=wso))
        out[f"o_proj_k1024_b{b}"] = {"us": round(us, 2),
                                     "GBps": round(2 * cc.d * 1024 / us / 1e3, 1)}
        log(f"TP8 share b={b}: shared {out[f'shared_expert_b{b}']}, in-proj "
            f"{out[f'in_proj_1536_b{b}']}, o-proj {out[f'o_proj_k1024_b{b}']}")
    return out


# sweep batches with uniform routing: 2, 4 and the verify batches 8 r (a
# speculative-decoding step verifies 8 tokens per request, r = 1..8)
SWEEP_UNIFORM = (2, 4, 8, 16, 24, 32, 40, 48, 56, 64)
# where the oracle is timed beside the sweep (batch, Zipf bias)
ORACLE_CASES = ((2, False), (4, False), (8, False), (16, False), (32, False), (64, True))


class HostWeights:
    """Host copies of one layer's weights for the oracle; experts are copied
    the first time one is named."""

    def __init__(self, layer):
        self.layer = layer
        self.dense = {k: v.cpu() for k, v in layer.moe.items()
                      if k not in ("w13", "w2", "bias") and v is not None}
        self.chain = {k: v.cpu() for k, v in layer.chain_w.items()}
        self.experts = {}

    def expert(self, e):
        if e not in self.experts:
            self.experts[e] = (self.layer.moe["w13"][e].cpu(), self.layer.moe["w2"][e].cpu())
        return self.experts[e]


class OracleStep:
    """One whole layer step of the oracle (plain fp64 C) at batch b: the
    chain, then the MoE block on its output. Everything it reads is on the
    host before any clock starts (the experts its own routing picks)."""

    def __init__(self, hw, k, cc, inp, b, bias, cfg_b):
        import numpy as np

        import oracle
        self.hw, self.k, self.cc, self.b, self.cfg_b = hw, k, cc, b, cfg_b
        self.bias = None if bias is None else bias.cpu()
        self.x, self.r = inp["x"][:b].cpu(), inp["r"][:b].cpu()
        ch = hw.chain
        hm = oracle.chain(self.x, self.r, ch["w_in"], ch["w_o"], ch["gamma"], cc.eps)["y"]
        ids, _ = oracle.topk_softmax(
            oracle.router_logits(hm, hw.dense["w_router"], self.bias), k)
        self.act = [int(e) for e in np.unique(ids)]
        for e in self.act:
            hw.expert(e)
        self.nbytes = moe_bytes(cfg_b, b, len(self.act)) + chain_bytes(cc, b)
        self.single, self.multi, self.threads = [], [], None

    def run(self) -> float:
        import oracle
        ch, host = self.hw.chain, dict(self.hw.dense)
        host["bias"] = self.bias
        t0 = time.perf_counter()
        c = oracle.chain(self.x, self.r, ch["w_in"], ch["w_o"], ch["gamma"], self.cc.eps)
        oracle.moe_block(c["y"], host, self.k, expert_weights=self.hw.expert)
        return time.perf_counter() - t0

    def time_all_cores(self, reps):
        import oracle
        self.threads = oracle.threads()
        self.multi = [self.run() for _ in range(reps)]

    def report(self) -> dict:
        import statistics as st
        out = {"bytes": int(self.nbytes), "n_active": len(self.act)}
        if self.multi:
            ms = st.median(self.multi) * 1e3
            out.update({"ms_per_step": round(ms, 1), "cores": self.threads,
                        "GBps": round(self.nbytes / ms / 1e6, 3), "runs": len(self.multi)})
        if self.single:
            ms1 = st.median(self.single) * 1e3
            out.update({"ms_per_step_1thread": round(ms1, 1),
                        "GBps_1thread": round(self.nbytes / ms1 / 1e6, 3),
                        "runs_1thread": len(self.single)})
        out["note"] = ("median of the runs; the single-thread runs of all sweep batches ran "
                       "concurrently, one host thread each, beside the GPU sweep")
        return out


def start_single_thread_runs(runs, reps):
    """One host thread per oracle step, each timing it reps times on one core."""
    import threading

    import oracle

    def work(o):
        oracle.set_threads(1)
        o.single = [o.run() for _ in range(reps)]

    ts = [threading.Thread(target=work, args=(o,), daemon=True) for o in runs]
    for t in ts:
        t.start()
    return ts


def cpu_baseline(torch, hw, cfg, cc, pool, b, seconds, tiny=None):
    """Time the oracle (plain fp64 C) on whole layer steps at batch b: as many
    as fit in about `seconds` on all host cores, and the median of three on
    one core (also for the tiny workload's MoE block when it was timed)."""
    import statistics as st
    import threading

    import numpy as np

    import oracle

    threads = oracle.threads()
    steps = [OracleStep(hw, cfg.k, cc, pool[i], b, hw.layer.moe.get("bias"), cfg)
             for i in range(NX)]
    done, spent, nbytes = 0, 0.0, 0
    while done < 2000 and (done == 0 or spent < seconds):
        o = steps[done % NX]
        spent += o.run()
        nbytes += o.nbytes
        done += 1
    sec = spent / done
    log(f"oracle: {done} steps, {sec * 1e3:.1f} ms/step on {threads} threads")
    single = []

    def one():
        oracle.set_threads(1)
        single.extend(steps[i].run() for i in range(3))

    t = threading.Thread(target=one)
    t.start()
    t.join()
    sec1 = st.median(single)
    out = {"value": round(nbytes / spent / 1e9, 3), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "ms_per_step": round(sec * 1e3, 2),
           "ms_per_step_1thread": round(sec1 * 1e3, 2),
           "GBps_1thread": round(float(np.mean([s.nbytes for s in steps[:3]])) / sec1 / 1e9, 3),
           "host": host_info(),
           "sample": f"{done} whole layer steps at batch {b} (chain + MoE block, "
                     f"{cfg.k} routed experts each) on all {threads} threads, and the median "
                     "of 3 on one thread; fp64 C oracle with OpenMP, a plain-loop "
                     "reference, not a tuned CPU implementation"}
    if tiny is not None:
        import synth
        tcfg = synth.MOE_CONFIGS["tiny"]
        tw = {k: (v.cpu() if v is not None else None)
              for k, v in synth.make_moe_weights(tcfg, device="cuda").items()}
        tx = synth.make_tokens(tcfg, device="cuda", index=0, b=1).cpu()

        def tiny_run():
            t0 = time.perf_counter()
            oracle.moe_block(tx, tw, tcfg.k)
            return time.perf_counter() - t0

        multi = [tiny_run() for _ in range(3)]
        one_t = []

        def tiny_one():
            oracle.set_threads(1)
            one_t.extend(tiny_run() for _ in range(3))

        t = threading.Thread(target=tiny_one)
        t.start()
        t.join()
        tiny["oracle"] = {"ms": round(st.median(multi) * 1e3, 3), "cores": threads,
                          "ms_1thread": round(st.median(one_t) * 1e3, 3), "runs": 3}
    return out


if __name__ == "__main__":
    sys.exit(main())
