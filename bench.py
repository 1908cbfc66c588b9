#!/usr/bin/env python3
"""Throughput of the chunked KDA forward on one MI355X (prints one JSON line).

A step is one full forward (prepare kernel + state kernel, i.e. one kda_fwd call) over one
synthetic batch already resident in HBM. Default workload: B=1, T=4096, H=HV=16, K=V=128, bf16
io ("h16_t4096"). The timed region is exactly --steps kda_fwd calls bracketed by
torch.cuda.synchronize(); before each step a 1 GiB device copy (a write of 1 GiB) evicts L2 and
the 256 MB MALL and a 512 MiB read leaves clean lines there, and each step is timed alone with
HIP events on its stream, so the step reads its inputs from HBM; the reported time is the
median step. Each kernel's average duration for
the roofline figures comes from a second pass of --steps flushed rounds, the two stages
launched separately (kda_fwd_prepare, kda_fwd_state: the same kernels), --kernel-reps launches
of each back to back between HIP events on the stream they run on.

With --backward the step is one kda_bwd call instead (gradients of every input from seeded
d_o and dht), reported under its own metric; the default line is the forward.

Extra fields beyond the driver contract:
  roofline        dominant kernel: achieved algorithmic throughput / MI355X peak
  roofline_path   the whole forward against the HBM roof (algorithmic bytes / step time)
  kernels         per-kernel average durations and algorithmic work
  warm_cache      back-to-back steps without flushes (the working set stays in the MALL)
  flush_dirty     steps after the write-only flush (its dirty lines still in the MALL)
  chunk16_run     the same workload with 16-token chunks, timed the same way
  cpu_baseline    the fp64 C oracle on the host cores over a bounded sample
"""
from __future__ import annotations

import argparse
import re
import hashlib
import glob
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA fwd tokens/s (all heads) @H=16,T=4096,K=V=128 bf16; HBM GB/s, MFMA %"
METRIC_BWD = "KDA bwd tokens/s (all heads); gradients of q, k, v, g, beta, h0 (fp32)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}   # dense; fp16 == bf16


def algorithmic_work(inp, C):
    """Algorithmic bytes and FLOPs of one forward with chunks of C tokens, split by the kernel
    that must do them.

    Bytes (what the method must move): the prepare kernel reads q, k (once per q/k head), v, g,
    beta; the state kernel writes o and reads/writes the per-(sequence, value head) states.
    FLOPs per C-token chunk of one value head (multiply-add = 2): state kernel
    6 C K V + 2 C^2 V + K V (w S, qd S, kr^T delta, Mqk delta, decay); prepare kernel
    L + Mqk + w + u (2 C^2 K + 2 C^2 K + 2 C^2 K + 2 C^2 V) plus the inverse (the Neumann
    product of each 16 x 16 diagonal block, 6 products of 16 x 16 x 16, and for C = 32 the
    block substitution, 2 more).
    """
    w = inp.w
    es = 2 if w.dtype == "bf16" else 4
    T_total = inp.T_total
    H, HV, K, V = w.H, w.HV, w.K, w.V
    N = inp.N
    n_chunk_heads = sum((b - a + C - 1) // C for a, b in inp.seq_bounds()) * HV
    prep_bytes = T_total * (H * 2 * K * es + HV * (V * es + K * es + es))
    state_bytes = T_total * HV * V * es + N * HV * K * V * 4 * (1 + (inp.h0 is not None))
    state_flops = n_chunk_heads * (6 * C * K * V + 2 * C * C * V + K * V)
    inv_flops = ((C // 16) * 6 * 2 * 16 ** 3 + (C // 16 - 1) * 2 * 2 * 16 ** 3) if C >= 16 else 0
    prep_flops = n_chunk_heads * (2 * C * C * (3 * K + V) + inv_flops)
    return dict(prep_bytes=prep_bytes, state_bytes=state_bytes, prep_flops=prep_flops,
                state_flops=state_flops, n_chunk_heads=n_chunk_heads)


def source_digest() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "chunked_kimi_delta_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when it is
    missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_digest") != source_digest():
        return None
    return d.get("hbm_bytes_per_launch")


def summarize_trace(d: str, command: str) -> str:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run (CSV output): per kernel the
    statistics of every dispatch, and, for this script's forward kernels, the average over the
    first launch of each stage after a cache flush next to the average over the launches that
    follow it back to back."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    out = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", command, "```", "",
           "| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f}% |")
    tp = os.path.join(d, "run_kernel_trace.csv")
    # the backward's runs have no cache-flushed steps: no split for them
    if os.path.exists(tp) and not any("bwd_" in r["Name"] for r in rows):
        tr = sorted(csv.DictReader(open(tp)), key=lambda r: int(r["Start_Timestamp"]))
        first, again = {}, {}
        seen = set()
        for r in tr:
            name = r["Kernel_Name"]
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            if "kda::" not in name:
                seen = set()                  # the flush's copy and read kernels
                continue
            # each kernel name once per stage call (the state stage of the two-segment pass
            # is two kernels)
            (again if name in seen else first).setdefault(name, []).append(dur)
            seen.add(name)
        out += ["", "Forward kernels by launch kind: the first launch of each stage after a "
                    "cache flush (the timed steps' kernels), and the launches that follow it "
                    "back to back before the next flush (warm steps and the per-kernel timing "
                    "pass's repeats):", "",
                "| kernel | first after a flush: calls | avg (us) | repeats: calls | avg (us) |",
                "|---|---|---|---|---|"]
        for name in sorted(set(first) | set(again)):
            f, w = first.get(name, []), again.get(name, [])
            fa = f"{statistics.mean(f):.2f}" if f else "-"
            wa = f"{statistics.mean(w):.2f}" if w else "-"
            out.append(f"| `{name}` | {len(f)} | {fa} | {len(w)} | {wa} |")
    out += ["", f"kernel sources digest: `{source_digest()}`", ""]
    return "\n".join(out)


def summarize_traffic(fetch_dir: str, write_dir: str, workload: str, command: str) -> dict:
    """Per-launch HBM bytes of each libkda_fwd kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads
    for a device copy of known size (__amd_rocclr_copyBuffer): the 1 GiB cache-flushing copies
    the timed steps run between them (their source does not fit any cache, so the copy reads
    and writes 1 GiB of HBM)."""
    import csv
    copy_bytes = 1 << 30
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        vals = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024)
        # the flush copies are the largest copy dispatches (inputs uploaded to the device show
        # up as smaller ones); their median calibrates the counter
        copy = sorted(x for k, v in vals.items() if "copyBuffer" in k for x in v)
        copy = [x for x in copy if x > 0.25 * copy[-1]] if copy else []
        if not copy:
            raise SystemExit(f"no calibration copy kernel in {d}")
        scale = copy_bytes / statistics.median(copy)
        for k, v in vals.items():
            if "kda::" not in k:
                continue
            # the stage a kernel belongs to: the state stage of the two-segment pass is two
            # kernels (the pass and its correction), each launched once per stage call
            stage = ("prepare" if "prepare" in k else
                     "recurrent" if "recurrent" in k else "state")
            e = res.setdefault(f"kda_{stage}", {})
            e[counter.lower() + "_raw_bytes"] = (e.get(counter.lower() + "_raw_bytes", 0.0) +
                                                 statistics.mean(v))
            e[counter.lower() + "_scale"] = round(scale, 4)
            e[counter.lower() + "_bytes"] = (e.get(counter.lower() + "_bytes", 0.0) +
                                             statistics.mean(v) * scale)
            e.setdefault("kernels", {}).setdefault(k, {})[counter.lower() + "_bytes"] = (
                statistics.mean(v) * scale)
    for k, e in res.items():
        e["hbm_bytes_per_launch"] = e["fetch_size_bytes"] + e["write_size_bytes"]
        e.update(kernel=k, workload=workload, source_digest=source_digest(), command=command)
    return res


def backward_work(inp):
    """Algorithmic bytes of one backward: read q, k (per q/k head), v, g, beta, d_o in the io
    dtype and the fp32 initial state and dht; write fp32 dq, dk, dv, dg, dbeta and dh0."""
    w = inp.w
    es = 2 if w.dtype == "bf16" else 4
    T_total, N = inp.T_total, inp.N
    H, HV, K, V = w.H, w.HV, w.K, w.V
    rd = T_total * (H * 2 * K * es + HV * (2 * V * es + K * es + es))
    rd += N * HV * K * V * 4 * (1 + (inp.h0 is not None))
    wr = T_total * (H * 2 * K * 4 + HV * (V + K + 1) * 4) + N * HV * K * V * 4
    return rd + wr


def backward_flops(inp):
    """Algorithmic FLOPs of one backward (multiply-add = 2) with 16-token chunks, per chunk of
    one value head (C = 16): the states chain (w S, kr^T delta: 2 C K V), the gradient chain
    (kr Lam, qd^T dO, w^T dDelta: 3 C K V, Mqk^T dO: C^2 V), the local products (w S, kr Lam,
    dO S^T, delta Lam^T, dDelta S^T: 5 C K V; A v, Mqk^T dO, dO delta^T, dDelta v^T, A^T dDelta:
    5 C^2 V) and the record (Gram, Mqk, w, u: C^2 (3 K + V) + C^2 V, the Neumann product)."""
    w = inp.w
    C, K, V = 16, w.K, w.V
    n = sum((b - a + C - 1) // C for a, b in inp.seq_bounds()) * w.HV
    mac = 10 * C * K * V + 6 * C * C * V + C * C * (3 * K + V) + 6 * 16 ** 3 + C * C * V
    return 2 * mac * n


def cpu_baseline_bwd(inp, gr, min_seconds: float):
    """The fp64 C backward oracle (unchanged) on the host cores: the whole workload's gradients
    (every unit), repeated until at least `min_seconds` of wall time have passed (bounded at
    1000 repetitions); then the same on one thread for a third of that time."""
    import workloads as W
    from oracle.native import kda_oracle_bwd_c
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    cores = max(1, min(affinity, BOX_CPU_SHARE))
    f = W.as_f32_numpy
    args = [f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.scale,
            None if inp.h0 is None else inp.h0.numpy(),
            None if inp.cu_seqlens is None else inp.cu_seqlens.numpy(),
            f(gr.d_o), None if gr.dht is None else gr.dht.numpy()]
    def run(threads, seconds):
        reps, t0 = 0, time.perf_counter()
        while True:
            kda_oracle_bwd_c(*args, n_threads=threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 1000:
                return reps, el
    reps, el = run(cores, min_seconds)
    reps1, el1 = run(1, min_seconds / 3)
    return {"value": round(reps * inp.T_total / el, 2), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"full {inp.w.name} backward (all {inp.w.HV} heads, fp64 C reverse "
                      f"recurrence), repeated {reps}x in {el:.1f} s",
            "value_1_thread": round(reps1 * inp.T_total / el1, 2),
            "cpu_model": cpu_model(), "affinity_cpus": affinity,
            "threads_note": f"{cores} threads: the CPU share of a one-GPU box "
                            f"(min of the affinity mask and {BOX_CPU_SHARE}); the tasks are "
                            f"(sequence, q/k head) pairs"}


def run_backward(a, torch, W, kda):
    w = W.WORKLOADS[a.workload]
    inp = W.make_inputs(w, seed=0)
    gr = W.make_grads(inp, seed=0)
    dev = torch.device("cuda:0")
    d = lambda x: None if x is None else x.to(dev).contiguous()
    plan = kda.KdaBwdPlan(d(inp.q), d(inp.k), d(inp.v), d(inp.g), d(inp.beta), d(gr.d_o),
                          d(gr.dht), scale=inp.scale, cu_seqlens=d(inp.cu_seqlens),
                          initial_state=d(inp.h0))
    stream = torch.cuda.current_stream(dev)
    for _ in range(a.warmup):
        plan(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        plan(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    nb = backward_work(inp)
    gbs = nb / (ms * 1e-3) / 1e9
    nf = backward_flops(inp)
    tfs = nf / (ms * 1e-3) / 1e12
    cpu = cpu_baseline_bwd(inp, gr, a.cpu_seconds) if a.cpu_seconds > 0 else None
    out = {
        "metric": METRIC_BWD, "value": round(inp.T_total / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": inp.q.shape[1], "H": w.H, "HV": w.HV,
                   "K": w.K, "V": w.V, "chunk": 16, "io": w.dtype,
                   "tokens_per_step": inp.T_total, "parallelism": "single-gpu"},
        "roofline": {"kernel": "kda_bwd (all launches of one call)", "bound": "mfma",
                     "achieved": round(tfs, 2), "peak": MFMA_PEAK_TFLOPS["fp32"],
                     "unit": "TFLOP/s", "frac": round(tfs / MFMA_PEAK_TFLOPS["fp32"], 5),
                     "traffic": None, "alg_flops_per_step": nf},
        "roofline_path": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 5),
                          "alg_bytes_per_step": nb},
        "kernel_timing": "per-kernel durations: rocprofv3 --kernel-trace of this command",
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def summarize_mfma(d: str, command: str) -> str:
    """Markdown summary of a rocprofv3 --pmc run with SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE
    and the SQ_INSTS_VALU_MFMA_MOPS_* counters: per kernel, the matrix-core busy share and the
    MFMA FLOPs issued (MOPS x 512, the counters' own unit). The busy share is the busy cycles
    summed over all 1,024 SIMDs divided by 1,024 times the kernel's active cycles; the collected
    GRBM_GUI_ACTIVE is the sum of the eight XCDs' counters, so the active cycles are that / 8
    (with it, the share matches the issued FLOPs over the kernel time at the dense peak)."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
    per = {}
    for r in rows:
        e = per.setdefault(r["Kernel_Name"], {})
        e.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = ["# rocprofv3 matrix-core counters", "", "Command:", "", "```", command, "```", "",
           "| kernel | dispatches | MFMA busy | MFMA GFLOP / dispatch (f16, bf16, f32) |",
           "|---|---|---|---|"]
    for k, e in per.items():
        if "kda::" not in k:
            continue
        m = lambda c: statistics.mean(e[c]) if c in e else 0.0
        busy = m("SQ_VALU_MFMA_BUSY_CYCLES") / (m("GRBM_GUI_ACTIVE") / 8 * 1024) * 100
        fl = [m(f"SQ_INSTS_VALU_MFMA_MOPS_{t}") * 512 / 1e9 for t in ("F16", "BF16", "F32")]
        out.append(f"| `{k}` | {len(e.get('GRBM_GUI_ACTIVE', []))} | {busy:.1f}% | "
                   + ", ".join(f"{x:.3f}" for x in fl) + " |")
    out += ["", f"kernel sources digest: `{source_digest()}`", ""]
    return "\n".join(out)


def summarize_counters(dirs, command: str) -> str:
    """Markdown summary of rocprofv3 --pmc runs of SQ_* instruction and cycle counters (one or
    more passes, CSV output): per libkda_fwd kernel the mean per dispatch and, for counts, the
    mean per wave (SQ_WAVES). Cycle counters in the SQ_*_CYCLES / SQ_WAIT / SQ_ACTIVE family
    count in units of four cycles (quad cycles); they are shown as read."""
    import csv
    per = {}
    for d in dirs:
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if "kda::" not in r["Kernel_Name"]:
                continue
            e = per.setdefault(r["Kernel_Name"], {})
            e.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = ["# rocprofv3 instruction and cycle counters", "", "Command (one run per pass):", "",
           "```", command, "```", ""]
    for k, e in per.items():
        waves = statistics.mean(e["SQ_WAVES"]) if "SQ_WAVES" in e else None
        out += [f"## `{k}`", "", "| counter | mean per dispatch | per wave |", "|---|---|---|"]
        for c in sorted(e):
            m = statistics.mean(e[c])
            pw = f"{m / waves:.1f}" if waves and c != "SQ_WAVES" and c != "GRBM_GUI_ACTIVE" else ""
            out.append(f"| {c} | {m:.6g} | {pw} |")
        out.append("")
    out += [f"kernel sources digest: `{source_digest()}`", ""]
    return "\n".join(out)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Host threads the oracle runs on: the CPU share of a one-GPU machine (16 CPUs), or fewer when the
# process may run on fewer. The affinity mask of a box can list every CPU of the host, which
# the other GPUs' jobs share.
BOX_CPU_SHARE = 16


def cpu_baseline(inp, min_seconds: float):
    """The fp64 C oracle (unchanged) on the host cores: the whole workload, repeated until at
    least `min_seconds` of wall time have passed (bounded at 1000 repetitions); then the same
    on one thread for a third of that time, to show the scaling."""
    import workloads as W
    from oracle.native import kda_oracle_c
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    cores = max(1, min(affinity, BOX_CPU_SHARE))
    f = W.as_f32_numpy
    args = [f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta)]
    h0 = None if inp.h0 is None else inp.h0.numpy()
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    def run(threads, seconds):
        reps, t0 = 0, time.perf_counter()
        while True:
            kda_oracle_c(*args, inp.scale, h0, cu, n_threads=threads, want_o=True)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 1000:
                return reps, el
    reps, el = run(cores, min_seconds)
    reps1, el1 = run(1, min_seconds / 3)
    return {"value": round(reps * inp.T_total / el, 2), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"full {inp.w.name} forward (all {inp.w.HV} heads, fp64 C recurrence), "
                      f"repeated {reps}x in {el:.1f} s",
            "value_1_thread": round(reps1 * inp.T_total / el1, 2),
            "cpu_model": cpu_model(), "affinity_cpus": affinity,
            "threads_note": f"{cores} threads: the CPU share of a one-GPU box "
                            f"(min of the affinity mask and {BOX_CPU_SHARE})"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="h16_t4096")
    ap.add_argument("--prestage", choices=["none", "softplus", "bounded"], default="none",
                    help="raw inputs with the fused pre-stage (q/k L2 norm, beta sigmoid and "
                         "this gate activation) inside the kernels")
    ap.add_argument("--chunk", type=int, default=0,
                    help="tokens per serial state step (16, 32; 0 = library default)")
    ap.add_argument("--kernel-reps", type=int, default=8,
                    help="launches of each stage per event span in the per-kernel timing pass")
    ap.add_argument("--warm-steps", type=int, default=50,
                    help="extra back-to-back steps without flushes, reported as warm (0: skip)")
    ap.add_argument("--compare-chunk16", type=int, default=1,
                    help="also time the 16-token chunk path of the same workload (0: skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum wall time of the oracle CPU baseline (0: skip)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 --stats output dir and exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<kernel>_<workload>.txt from two --pmc runs")
    ap.add_argument("--command", default="", help="the profiling command, for the summaries")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 --pmc matrix-core run and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="print a markdown summary of rocprofv3 --pmc SQ counter runs and exit")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (kda_bwd) instead of the forward")
    a = ap.parse_args()

    if a.summarize_trace:
        print(summarize_trace(a.summarize_trace, a.command))
        return
    if a.summarize_counters:
        print(summarize_counters(a.summarize_counters, a.command))
        return
    if a.summarize_mfma:
        print(summarize_mfma(a.summarize_mfma, a.command))
        return
    if a.summarize_traffic:
        res = summarize_traffic(a.summarize_traffic[0], a.summarize_traffic[1], a.workload,
                                a.command)
        for k, e in res.items():
            path = os.path.join(ROOT, "profiles", f"traffic_{k}_{a.workload}.txt")
            with open(path, "w") as f:
                json.dump(e, f, indent=1)
                f.write("\n")
            print(path, json.dumps(e))
        return

    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {a.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import chunked_kimi_delta_amd as kda

    if a.backward:
        run_backward(a, torch, W, kda)
        return

    w = W.WORKLOADS[a.workload]
    pre = {}
    if a.prestage != "none":
        raw = W.make_raw_inputs(w, seed=0)
        inp = raw.inp
        pre = dict(use_qk_l2norm=True, use_beta_sigmoid=True, gate=a.prestage,
                   A_log=raw.A_log.to("cuda:0"), dt_bias=raw.dt_bias.to("cuda:0"))
    else:
        inp = W.make_inputs(w, seed=0)
    dev = torch.device("cuda:0")
    d = lambda x: None if x is None else x.to(dev).contiguous()
    plan = kda.KdaFwdPlan(d(inp.q), d(inp.k), d(inp.v), d(inp.g), d(inp.beta),
                          cu_seqlens=d(inp.cu_seqlens), initial_state=d(inp.h0), chunk=a.chunk,
                          **pre)
    # the chunk the library picks for chunk 0 (include/kda_fwd.h): the token recurrence for a
    # dense batch of at most 16 tokens per sequence, else 32 (bf16 io) or 16 (fp32 io)
    chunk = a.chunk or (1 if inp.cu_seqlens is None and inp.q.shape[1] <= 16 else
                        32 if w.dtype == "bf16" else 16)
    stream = torch.cuda.current_stream(dev)

    # Every timed step starts with the caches flushed: a 1 GiB device copy (a write of 1 GiB)
    # evicts every line of the step's working set from L2 and the 256 MB MALL; a 512 MiB read
    # of a third buffer then replaces the copy's dirty lines with clean ones, so the step reads
    # its inputs from HBM without also paying for writing the flush's own data back. Each step
    # is timed alone with HIP events on the stream it runs on; the flush lies outside them.
    flush_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)
    flush_clean = torch.zeros(1 << 29, dtype=torch.uint8, device=dev)

    def flush_dirty():
        flush_dst.copy_(flush_src)

    def flush():
        flush_dst.copy_(flush_src)
        flush_clean.max()

    def flushed_steps(call, n, flush=flush):
        evs = []
        for _ in range(n):
            flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(stream)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    for _ in range(a.warmup):
        flush()
        plan(stream)
    torch.cuda.synchronize()

    # the box's own copy bandwidth, for context next to the 8 TB/s peak: the flush's 1 GiB
    # device copy (reads and writes 1 GiB of HBM; neither buffer fits any cache), HIP events
    # around each of five copies, median
    cps = []
    for _ in range(5):
        flush_clean.max()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        flush_dst.copy_(flush_src)
        c1.record(stream)
        cps.append((c0, c1))
    torch.cuda.synchronize()
    copy_ms = statistics.median(c0.elapsed_time(c1) for c0, c1 in cps)
    copy_gbs = 2 * (1 << 30) / (copy_ms * 1e-3) / 1e9

    # the timed region: exactly --steps forwards, each after a cache flush
    t0 = time.perf_counter()
    step_ms = flushed_steps(plan, a.steps)
    t1 = time.perf_counter()
    ms_per_step = statistics.median(step_ms)
    srt = sorted(step_ms)
    pct = lambda f: round(srt[min(len(srt) - 1, int(f * len(srt)))], 5)
    step_dist = {"p10_ms": pct(0.1), "p50_ms": pct(0.5), "p90_ms": pct(0.9),
                 "wall_s_with_flushes": round(t1 - t0, 4),
                 "note": "per-step HIP-event durations of the timed (flushed) steps"}

    # per-kernel durations: after each flush, --kernel-reps launches of the prepare stage, then
    # as many of the state stage, back to back between HIP events on their stream (both stages
    # are idempotent: the same inputs give the same workspace, the same workspace the same o
    # and final state). An event recorded between two kernels adds several microseconds of GPU
    # time, so a span of one launch would overstate the kernel; over R launches it adds 1/R.
    R = max(1, a.kernel_reps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    for i in range(a.steps):
        flush()
        ev[i][0].record(stream)
        for _ in range(R):
            plan.prepare(stream)
        ev[i][1].record(stream)
        for _ in range(R):
            plan.state(stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    prep_ms = statistics.mean(ev[i][0].elapsed_time(ev[i][1]) for i in range(a.steps)) / R
    state_ms = statistics.mean(ev[i][1].elapsed_time(ev[i][2]) for i in range(a.steps)) / R

    # warm cache, labelled as such: --warm-steps back-to-back forwards with the working set
    # (inputs, workspace, outputs) left in the MALL, timed by the host clock
    warm = None
    if a.warm_steps > 0:
        torch.cuda.synchronize()
        tw0 = time.perf_counter()
        for _ in range(a.warm_steps):
            plan(stream)
        torch.cuda.synchronize()
        warm_ms = (time.perf_counter() - tw0) * 1e3 / a.warm_steps
        warm = {"ms_per_step": round(warm_ms, 5),
                "tokens_per_s": round(inp.T_total / (warm_ms * 1e-3), 1),
                "steps": a.warm_steps,
                "note": "warm cache: back-to-back steps, no flush, host clock around all of them"}

    # the same steps after the write-only flush (the flush's dirty lines still in the MALL)
    dirty_ms = statistics.median(flushed_steps(plan, max(5, a.steps // 5), flush=flush_dirty))
    dirty = {"ms_per_step_median": round(dirty_ms, 5),
             "tokens_per_s": round(inp.T_total / (dirty_ms * 1e-3), 1),
             "note": "each step after the 1 GiB copy alone: the MALL still holds the copy's "
                     "dirty lines, which the step's own traffic has to write back"}

    # the chunk-16 run of the same workload (the FlashKDA tile), timed the same way
    c16 = None
    if a.compare_chunk16 and chunk in (32, 64):
        plan16 = kda.KdaFwdPlan(d(inp.q), d(inp.k), d(inp.v), d(inp.g), d(inp.beta),
                                cu_seqlens=d(inp.cu_seqlens), initial_state=d(inp.h0),
                                chunk=16, **pre)
        for _ in range(3):
            plan16(stream)
        ms16 = statistics.median(flushed_steps(plan16, a.steps))
        c16 = {"chunk": 16, "ms_per_step": round(ms16, 5),
               "tokens_per_s": round(inp.T_total / (ms16 * 1e-3), 1),
               "note": "same workload and timing (flushed, median), 16-token chunks"}
        del plan16
    del flush_src, flush_dst, flush_clean

    work = algorithmic_work(inp, chunk)
    # The method's algorithmic FLOPs are counted with 16-token chunks, the chunk length the
    # pages' kernels use; longer chunks issue more (the 2 C^2 V term) for the same result.
    work16 = algorithmic_work(inp, 16)
    es = "bf16" if w.dtype == "bf16" else "fp32"
    if chunk != 1:
        kernels = {
            "kda_prepare": {"avg_ms": round(prep_ms, 5), "bound": "hbm",
                            "alg_bytes": work["prep_bytes"], "alg_flops": work16["prep_flops"],
                            "issued_flops_this_chunk": work["prep_flops"],
                            "achieved_GBs": round(work["prep_bytes"] / (prep_ms * 1e-3) / 1e9,
                                                  1)},
            "kda_state": {"avg_ms": round(state_ms, 5), "bound": "mfma",
                          "alg_bytes": work["state_bytes"], "alg_flops": work16["state_flops"],
                          "issued_flops_this_chunk": work["state_flops"],
                          "achieved_TFLOPs": round(work16["state_flops"] / (state_ms * 1e-3)
                                                   / 1e12, 2),
                          "launches": "the state stage (kda_fwd_state): one kernel, or, for a "
                                      "dense 32-token batch whose state slices fill at most "
                                      "half of the CUs, the two-segment pass and its "
                                      "correction kernel"},
        }
    if chunk == 1:
        # the token recurrence is one kernel (the prepare launch is empty): everything it reads
        # and writes (inputs, o, the states) is its algorithmic traffic
        rb = work["prep_bytes"] + work["state_bytes"]
        kernels = {"kda_recurrent": {"avg_ms": round(state_ms, 5), "bound": "hbm",
                                     "alg_bytes": rb,
                                     "achieved_GBs": round(rb / (state_ms * 1e-3) / 1e9, 1)}}
        ach = rb / (state_ms * 1e-3) / 1e9
        roof = {"kernel": "kda_recurrent", "bound": "hbm", "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 5),
                "traffic": committed_traffic("kda_recurrent", w.name)}
    elif state_ms >= prep_ms:
        ach = work16["state_flops"] / (state_ms * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[es]
        roof = {"kernel": "kda_state", "bound": "mfma", "achieved": round(ach, 3),
                "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 5),
                "traffic": committed_traffic("kda_state", w.name),
                "alg_flops_per_launch": work16["state_flops"]}
    else:
        ach = work["prep_bytes"] / (prep_ms * 1e-3) / 1e9
        roof = {"kernel": "kda_prepare", "bound": "hbm", "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 5),
                "traffic": committed_traffic("kda_prepare", w.name),
                "alg_bytes_per_launch": work["prep_bytes"]}
    path_bytes = work["prep_bytes"] + work["state_bytes"]
    path_gbs = path_bytes / (ms_per_step * 1e-3) / 1e9
    roof_path = {"bound": "hbm", "achieved": round(path_gbs, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": round(path_gbs / HBM_PEAK_GBS, 5),
                 "alg_bytes_per_step": path_bytes,
                 "copy_GBs": round(copy_gbs, 1), "frac_of_copy": round(path_gbs / copy_gbs, 5),
                 "note": "whole forward, algorithmic bytes / flushed median step time; copy_GBs "
                         "is a 1 GiB device copy on the same GPU (read + write bytes / time)"}
    if c16 is not None:
        c16["roofline_path_frac"] = round(path_bytes / (c16["ms_per_step"] * 1e-3) / 1e9
                                          / HBM_PEAK_GBS, 5)

    cpu = None
    if a.cpu_seconds > 0 and not pre:
        cpu = cpu_baseline(inp, a.cpu_seconds)

    value = inp.T_total / (ms_per_step * 1e-3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": inp.q.shape[1], "H": w.H, "HV": w.HV,
                   "K": w.K, "V": w.V, "chunk": chunk, "tokens_per_step": inp.T_total,
                   "parallelism": "single-gpu", "prestage": a.prestage,
                   "timing": "median of per-step HIP-event times, each step after a cache "
                             "flush (1 GiB copy, then a 512 MiB read so the MALL holds clean, "
                             "unrelated lines)",
                   "chunk_note": ("the library's default chunk for bf16 io (32 tokens); the "
                                  "16-token run of the same workload is in chunk16_run"
                                  if chunk == 32 else ""),
                   "arithmetic": ("fp32 VALU token recurrence" if chunk == 1 else
                                  "bf16/fp16 MFMA with fp32 accumulation, fp32 inverse")},
        "roofline": roof, "roofline_path": roof_path, "kernels": kernels,
        "kernel_timing": f"avg_ms: a second pass of --steps rounds, each after a cache flush: "
                         f"{R} back-to-back launches of one stage between HIP events on its "
                         f"stream, then {R} of the other; span / {R}",
        "step_distribution": step_dist, "warm_cache": warm, "flush_dirty": dirty,
        "chunk16_run": c16,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
