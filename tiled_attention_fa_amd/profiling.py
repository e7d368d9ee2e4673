"""rocprofv3 evidence for the benchmark workloads: kernel times, HBM traffic,
instruction mix and shader clock, summarised into profiles/.

    python -m tiled_attention_fa_amd.profiling run --workload W --out DIR
        Runs, one rocprofv3 pass per child process (this process never
        touches the GPU), each under a time limit, from /tmp, every pass
        over bench.py --workload W --steps 20 --warmup 5 (its defaults):
          kernel trace + stats
          --pmc FETCH_SIZE
          --pmc WRITE_SIZE
          --pmc SQ_* (8 counters, one pass)
        and, once per DIR, the same two traffic counters over a plain 1 GiB
        device copy (bench.py --copy-calibration 1024), which scales the
        counters' KiB to bytes.
    python -m tiled_attention_fa_amd.profiling summarize --workload W --out DIR
        Parses those CSV files and writes profiles/traffic_W.json (read by
        bench.py for roofline.traffic and the clock) and
        profiles/W_counters.md (the figures and the commands that made them).
    With --batch B / --seq-len S (both actions) the workload runs at that
    shape; the summary is then profiles/W_B<B>_S<S>_counters.md, with the
    compulsory HBM bytes of the shape beside the counters (a shape whose
    inputs fit the L2 checks the copy calibration on the library's own
    access pattern), and no traffic file.

    python -m tiled_attention_fa_amd.profiling bench --set SET --out DIR
    python -m tiled_attention_fa_amd.profiling bench-summary --set SET --out DIR
        Plain bench.py runs (no profiler), one child process each under a
        time limit, their JSON lines kept in DIR/bench/, then one table in
        profiles/: SET = workloads (every workload at its own shape:
        workloads_all_bench.md), seqlen (causal fwd+bwd from S = 1024 to
        32768: causal_by_seqlen.md) or variants (static against persistent
        schedule, recomputed against stored dS for dQ, each twice, in
        alternation: schedule_and_dq_variants.md).

    python -m tiled_attention_fa_amd.profiling stalls --workload W --out DIR
    python -m tiled_attention_fa_amd.profiling stalls-summary --workload W --out DIR
        Two more --pmc passes over the same bench.py run (STALL_PASSES): where
        the waves spend their time (waiting for a dependency, waiting to
        issue, issuing VALU or LDS instructions) and how busy the matrix
        cores and the LDS are; then profiles/W_stalls.md, per kernel.

    python -m tiled_attention_fa_amd.profiling wgtrace --workload W --out DIR
    python -m tiled_attention_fa_amd.profiling wgtrace-summary --workload W --out DIR
        bench.py --wg-trace (no profiler): after the timed steps, one more
        step whose forward records every query tile's start and end (the
        100 MHz clock), compute unit and size; then
        profiles/W_wgtrace.md: span, balance over compute units and XCDs,
        the gaps between workgroups, and the fit duration = fixed + per
        step x steps.

Kernels are grouped by the bench.py timing keys (fwd, bwd_delta, bwd_dkdv,
bwd_dq, block_mask).  Durations and counters are taken over the dispatches
of bench.py's timed steps (a kernel launched once per step: its last 20).
The shader clock under a kernel is SQ_BUSY_CYCLES / 32 (the counter is
summed over the 32 shader engines) over each dispatch's own duration in the
SQ run, averaged; the matrix-core busy fraction is SQ_VALU_MFMA_BUSY_CYCLES
over (kernel cycles x 1024 SIMDs).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BENCH = os.path.join(ROOT, "bench.py")
PROFILES = os.path.join(ROOT, "profiles")

SQ_COUNTERS = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
               "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_SALU"]
# Wave-time and LDS/matrix-core counters, 8 SQ counters per pass (the most
# one pass can hold); SQ_BUSY_CYCLES in both gives each dispatch's cycles.
STALL_PASSES = {
    "stallA": ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY",
               "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_BUSY_CYCLES"],
    "stallB": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_DATA_FIFO_FULL",
               "SQ_LDS_CMD_FIFO_FULL", "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_INSTS_MFMA", "SQ_BUSY_CYCLES"],
}
COMPUTE_UNITS = 256
SHADER_ENGINES = 32
SIMDS = 1024
COPY_MIB = 1024
# Every profiled run and every bench-table run: bench.py's default step counts.
BENCH_STEPS, BENCH_WARMUP = 20, 5


def kernel_key(name: str) -> str | None:
    """bench.py's timing key of a library kernel, or None for other kernels."""
    if "miattn::" not in name:
        return None
    for pat, key in (("bwd_delta", "bwd_delta"), ("bwd_dkdv", "bwd_dkdv"), ("bwd_dq", "bwd_dq"),
                     ("block_mask", "block_mask"), ("fp8_quantize", "fp8_quantize"), ("fwd", "fwd"),
                     ("bias_grad", "bwd_bias_grad")):
        if pat in name:
            return key
    return None


def source_sha() -> str:
    """Same hash as bench.py: of the kernel sources the counters were taken on."""
    h = hashlib.sha256()
    d = os.path.join(HERE, "csrc")
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def _bench_args(workload: str, steps: int, warmup: int, shape=(0, 0)) -> list[str]:
    extra = []
    if shape[0]:
        extra += ["--batch", str(shape[0])]
    if shape[1]:
        extra += ["--seq-len", str(shape[1])]
    return [sys.executable, BENCH, "--workload", workload, "--no-cpu-baseline", "--steps", str(steps),
            "--warmup", str(warmup), *extra]


def label(workload: str, shape=(0, 0)) -> str:
    """Name of a profiled case: the workload, plus its shape when overridden."""
    if not any(shape):
        return workload
    return workload + "".join(f"_{t}{v}" for t, v in zip("BS", shape) if v)


def passes(workload: str, out: str, shape=(0, 0)) -> list[tuple[str, list[str]]]:
    """(name, argv) of every rocprofv3 pass of one workload: each runs
    bench.py's default step counts, so the timed dispatches are bench.py's."""
    wdir = os.path.join(out, label(workload, shape))
    fmt = ["--output-format", "csv", "-o", "run"]
    args = _bench_args(workload, BENCH_STEPS, BENCH_WARMUP, shape)
    res = [("trace", ["rocprofv3", "--kernel-trace", "--stats", *fmt, "-d", os.path.join(wdir, "trace"), "--", *args])]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        res.append((c, ["rocprofv3", "--pmc", c, *fmt, "-d", os.path.join(wdir, c), "--", *args]))
    res.append(("sq", ["rocprofv3", "--pmc", *SQ_COUNTERS, *fmt, "-d", os.path.join(wdir, "sq"), "--", *args]))
    return res


def stall_passes(workload: str, out: str, shape=(0, 0)) -> list[tuple[str, list[str]]]:
    wdir = os.path.join(out, label(workload, shape))
    fmt = ["--output-format", "csv", "-o", "run"]
    args = _bench_args(workload, BENCH_STEPS, BENCH_WARMUP, shape)
    return [(name, ["rocprofv3", "--pmc", *ctrs, *fmt, "-d", os.path.join(wdir, name), "--", *args])
            for name, ctrs in STALL_PASSES.items()]


def calibration_passes(out: str) -> list[tuple[str, list[str]]]:
    fmt = ["--output-format", "csv", "-o", "run"]
    return [(f"copy_{c}", ["rocprofv3", "--pmc", c, *fmt, "-d", os.path.join(out, f"copy_{c}"), "--",
                           sys.executable, BENCH, "--copy-calibration", str(COPY_MIB)])
            for c in ("FETCH_SIZE", "WRITE_SIZE")]


def run(workload: str, out: str, limit: int, shape=(0, 0), stalls: bool = False) -> None:
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    name_of = label(workload, shape)
    if stalls:
        todo = stall_passes(workload, out, shape)
    else:
        todo = passes(workload, out, shape)
        if not os.path.isdir(os.path.join(out, "copy_WRITE_SIZE")):
            todo = calibration_passes(out) + todo
    env = dict(os.environ, TMPDIR="/tmp")
    for name, argv in todo:
        print(f"profiling: {name_of} {name}", flush=True)
        # The pass's own time limit (a counter request the hardware cannot
        # serve makes rocprofv3 hang instead of failing).
        r = subprocess.run(["timeout", "-s", "KILL", str(limit), *argv], cwd="/tmp", env=env,
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        with open(os.path.join(out, f"{name_of}_{name}.log" if not name.startswith("copy") else f"{name}.log"),
                  "w") as f:
            f.write(r.stdout)
        if r.returncode != 0:
            sys.exit(f"rocprofv3 pass {name} of {name_of} ended with status {r.returncode}")


def _csv(pattern: str) -> list[dict]:
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise FileNotFoundError(pattern)
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _timed(seq: list) -> list:
    """The dispatches of bench.py's timed steps: a kernel launched once per
    step has BENCH_WARMUP + BENCH_STEPS dispatches and keeps the last
    BENCH_STEPS; kernels launched outside the step loop keep all."""
    return seq[-BENCH_STEPS:] if len(seq) >= BENCH_STEPS + BENCH_WARMUP else seq


def _dispatches(d: str) -> dict[str, list[dict[str, float]]]:
    """Per kernel name, in dispatch order: each dispatch's counters (summed
    over the rows rocprofv3 splits them into) and its duration in ns."""
    per: dict[str, dict[int, dict[str, float]]] = {}
    for r in _csv(os.path.join(d, "**", "*counter_collection.csv")):
        disp = per.setdefault(r["Kernel_Name"], {}).setdefault(int(r.get("Dispatch_Id") or r["Correlation_Id"]), {})
        c = r["Counter_Name"]
        disp[c] = disp.get(c, 0.0) + float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            disp["_dur_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return {n: [ds[i] for i in sorted(ds)] for n, ds in per.items()}


def _dispatch_sums(d: str) -> dict[str, dict[str, float]]:
    """Per kernel name and counter: mean over the timed dispatches."""
    res = {}
    for name, seq in _dispatches(d).items():
        seq = _timed(seq)
        keys = {c for x in seq for c in x if not c.startswith("_")}
        res[name] = {c: sum(x.get(c, 0.0) for x in seq) / len(seq) for c in keys}
        clocks = [x["SQ_BUSY_CYCLES"] / SHADER_ENGINES / x["_dur_ns"] for x in seq
                  if x.get("_dur_ns", 0) > 0 and "SQ_BUSY_CYCLES" in x]
        if clocks:
            res[name]["_clock_ghz"] = sum(clocks) / len(clocks)
    return res


def trace_stats(d: str) -> dict[str, dict[str, float]]:
    """Per kernel name: durations of the timed dispatches (average, min,
    max, in us) and the average over every dispatch."""
    per: dict[str, list[tuple[int, float]]] = {}
    for r in _csv(os.path.join(d, "**", "*kernel_trace.csv")):
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["Dispatch_Id"]), (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3))
    res = {}
    for name, v in per.items():
        allv = [t for _, t in sorted(v)]
        tv = _timed(allv)
        res[name] = {"calls": len(allv), "timed_calls": len(tv), "avg_us": sum(tv) / len(tv), "min_us": min(tv),
                     "max_us": max(tv), "avg_all_us": sum(allv) / len(allv), "total_us": sum(allv)}
    return res


def calibration(out: str) -> dict:
    f = _dispatch_sums(os.path.join(out, "copy_FETCH_SIZE"))
    w = _dispatch_sums(os.path.join(out, "copy_WRITE_SIZE"))
    copy = [n for n in f if "copy" in n.lower()]
    if not copy:
        raise RuntimeError("no copy kernel in the calibration run")
    name = max(copy, key=lambda n: f[n].get("FETCH_SIZE", 0.0))
    nbytes = COPY_MIB << 20
    fk, wk = f[name]["FETCH_SIZE"], w[name]["WRITE_SIZE"]
    return {"copy_kernel": name, "copy_bytes": nbytes, "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
            "fetch_factor": nbytes / (fk * 1024.0), "write_factor": nbytes / (wk * 1024.0)}


def compulsory_bytes(workload: str, shape=(0, 0)) -> dict[str, int]:
    """HBM bytes each forward kernel must move at least, per launch: Q, K, V
    read once, O and LSE written once (bf16 / fp32 elements as the workload
    stores them)."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import synth  # the workload shapes only
    w = synth.WORKLOADS[workload]
    B, S = shape[0] or w.B, shape[1] or w.S
    el = 4 if w.dtype == "f32" else 2
    q = B * w.Hq * S * w.D * el
    kv = 2 * B * w.Hkv * S * w.D * el
    return {"read": q + kv, "written": q + (B * w.Hq * S * 4 if w.lse else 0)}


def summarize(workload: str, out: str, shape=(0, 0)) -> dict:
    wdir = os.path.join(out, label(workload, shape))
    cal = calibration(out)
    fetch = _dispatch_sums(os.path.join(wdir, "FETCH_SIZE"))
    write = _dispatch_sums(os.path.join(wdir, "WRITE_SIZE"))
    sq = _dispatch_sums(os.path.join(wdir, "sq"))
    tr = trace_stats(os.path.join(wdir, "trace"))
    kernels: dict[str, dict] = {}
    for name, st in sorted(tr.items(), key=lambda kv: -kv[1]["total_us"]):
        key = kernel_key(name)
        if key is None:
            continue
        k = {"kernel_name": name, "calls": st["calls"], "timed_calls": st["timed_calls"], "avg_us": st["avg_us"],
             "min_us": st["min_us"], "max_us": st["max_us"], "avg_all_us": st["avg_all_us"]}
        if name in fetch and name in write:
            fk, wk = fetch[name]["FETCH_SIZE"], write[name]["WRITE_SIZE"]
            k.update(fetch_kib=fk, write_kib=wk,
                     bytes_per_launch=int(round(fk * 1024.0 * cal["fetch_factor"] + wk * 1024.0 * cal["write_factor"])))
        if name in sq:
            c = {x: v for x, v in sq[name].items() if not x.startswith("_")}
            cycles = c.get("SQ_BUSY_CYCLES", 0.0) / SHADER_ENGINES
            k["sq"] = c
            if cycles > 0:
                # The clock of the counter run's own dispatches (their cycles
                # over their durations); the trace run's average otherwise.
                k["clock_ghz"] = sq[name].get("_clock_ghz", cycles / (st["avg_us"] * 1e3))
                k["mfma_busy"] = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cycles * SIMDS)
            if c.get("SQ_INSTS_MFMA", 0) > 0:
                k["valu_per_mfma"] = c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"]
                k["lds_per_mfma"] = c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"]
        if key in kernels:  # several kernels under one key (the block-mask builder): the longest
            if kernels[key]["avg_us"] >= k["avg_us"]:
                continue
        kernels[key] = k
    out_abs = os.path.abspath(out)
    rec = {"workload": workload, "label": label(workload, shape), "source_sha": source_sha(), "calibration": cal,
           "kernels": kernels,
           "commands": {n: " ".join("python3" if x == sys.executable else x for x in a)
                        .replace(out_abs, "<out>").replace(ROOT, "<repo>")
                        for n, a in passes(workload, out_abs, shape) + calibration_passes(out_abs)}}
    if any(shape):
        rec["compulsory"] = compulsory_bytes(workload, shape)
    return rec


def write_summary(rec: dict) -> tuple[str | None, str]:
    w = rec["workload"]
    name = rec.get("label", w)
    os.makedirs(PROFILES, exist_ok=True)
    jpath = None
    if name == w:  # bench.py's traffic file belongs to the workload's own shape
        jpath = os.path.join(PROFILES, f"traffic_{w}.json")
        slim = {"workload": w, "source_sha": rec["source_sha"], "calibration": rec["calibration"],
                "kernels": {k: {x: v for x, v in d.items() if x != "sq"} for k, d in rec["kernels"].items()}}
        with open(jpath, "w") as f:
            json.dump(slim, f, indent=1)
    lines = [f"# Counters and kernel trace: {name}", "",
             "Commands (on the GPU host, from /tmp with TMPDIR=/tmp; `<repo>` is the repository root, `<out>` the "
             "output folder); `python -m tiled_attention_fa_amd.profiling run` issues exactly these:", "", "```"]
    lines += [rec["commands"][n] for n in ("trace", "FETCH_SIZE", "WRITE_SIZE", "sq", "copy_FETCH_SIZE",
                                            "copy_WRITE_SIZE")]
    cal = rec["calibration"]
    lines += ["```", "",
              f"Calibration: a {cal['copy_bytes'] >> 20} MiB device copy (`{cal['copy_kernel']}`) reads "
              f"FETCH_SIZE = {cal['fetch_kib_per_dispatch']:.0f} KiB and WRITE_SIZE = {cal['write_kib_per_dispatch']:.0f}"
              f" KiB per dispatch: KiB are scaled by {cal['fetch_factor']:.3f} (fetch) and {cal['write_factor']:.3f}"
              " (write) to bytes.", "",
              f"Durations: the kernel trace's timed dispatches (a kernel launched once per step: the last "
              f"{BENCH_STEPS} of {BENCH_WARMUP} + {BENCH_STEPS}, the dispatches bench.py times; others: all), with the "
              "average over every dispatch beside them. Counters: the mean over the same dispatches of each counter "
              "run; the clock is each dispatch's SQ_BUSY_CYCLES / 32 over its own duration in the SQ run.", "",
              "| key | kernel | timed / all calls | avg (us) | min (us) | max (us) | avg all (us) | HBM read MB "
              "| HBM written MB | clock (GHz) | MFMA busy | VALU / MFMA | LDS / MFMA | LDS bank conflicts |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for key, k in rec["kernels"].items():
        rd = k.get("fetch_kib", 0.0) * 1024 * cal["fetch_factor"] / 1e6
        wr = k.get("write_kib", 0.0) * 1024 * cal["write_factor"] / 1e6
        sq = k.get("sq", {})

        def fmt(x, p=2):
            return "-" if x is None else f"{x:.{p}f}"
        lines.append(f"| {key} | `{k['kernel_name']}` | {k.get('timed_calls', k['calls'])} / {k['calls']} | "
                     f"{k['avg_us']:.1f} | {k['min_us']:.1f} | {k['max_us']:.1f} | {k.get('avg_all_us', k['avg_us']):.1f} | "
                     f"{rd:.1f} | {wr:.1f} | {fmt(k.get('clock_ghz'))} | "
                     f"{fmt(k.get('mfma_busy'))} | {fmt(k.get('valu_per_mfma'), 1)} | {fmt(k.get('lds_per_mfma'), 2)} | "
                     f"{sq.get('SQ_LDS_BANK_CONFLICT', 0):.0f} |")
    if "compulsory" in rec:
        c = rec["compulsory"]
        lines += ["", f"Compulsory bytes of the forward at this shape (Q, K, V read once; O and LSE written once): "
                  f"{c['read'] / 1e6:.2f} MB read, {c['written'] / 1e6:.2f} MB written."]
    lines += ["", f"Kernel sources of these figures: hash `{rec['source_sha']}` (bench.py uses the traffic and clock "
              "only while the sources hash the same)."]
    mpath = os.path.join(PROFILES, f"{name}_counters.md")
    with open(mpath, "w") as f:
        f.write("\n".join(lines) + "\n")
    return jpath, mpath


# ---------------------------------------------------------------- bench tables
SEQLEN_SHAPES = [(16, 1024), (8, 2048), (4, 4096), (2, 8192), (1, 16384), (1, 32768)]
VARIANT_WORKLOADS = ["causal_fwd_bwd", "causal_prefill", "gqa_causal", "gqa_window", "doc_packed"]


def bench_runs(which: str) -> list[tuple[str, list[str]]]:
    """(label, bench.py arguments) of every run of one table, in run order."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import synth  # the workload names only
    base = ["--no-cpu-baseline", "--steps", str(BENCH_STEPS), "--warmup", str(BENCH_WARMUP)]
    if which == "workloads":
        return [(w, ["--workload", w, *base]) for w in synth.WORKLOADS]
    if which == "seqlen":
        return [(f"causal_fwd_bwd_B{b}_S{n}", ["--workload", "causal_fwd_bwd", "--batch", str(b), "--seq-len", str(n),
                                                *base]) for b, n in SEQLEN_SHAPES]
    if which == "variants":
        runs = []
        for rep in (1, 2):
            for w in VARIANT_WORKLOADS:
                for sched in ("static", "persistent"):
                    runs.append((f"{w}_schedule-{sched}_{rep}", ["--workload", w, "--schedule", sched, *base]))
            for dq in ("recompute", "stored"):
                runs.append((f"causal_fwd_bwd_dq-{dq}_{rep}", ["--workload", "causal_fwd_bwd", "--bwd-dq", dq, *base]))
        return runs
    raise ValueError(which)


def run_benches(which: str, out: str, limit: int) -> None:
    d = os.path.join(os.path.abspath(out), "bench")
    os.makedirs(d, exist_ok=True)
    for lab, args in bench_runs(which):
        print(f"bench: {lab}", flush=True)
        r = subprocess.run(["timeout", "-s", "KILL", str(limit), sys.executable, BENCH, *args], cwd=ROOT,
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        with open(os.path.join(d, f"{lab}.json"), "w") as f:
            f.write(r.stdout)
        if r.returncode != 0:
            sys.exit(f"bench.py {' '.join(args)} ended with status {r.returncode}")


def _bench_line(path: str) -> dict:
    for line in reversed(open(path).read().splitlines()):
        if line.startswith("{"):
            return json.loads(line)
    raise ValueError(f"no JSON line in {path}")


def _kernel_ms(rec: dict) -> str:
    return ", ".join(f"{k} {v:.3f}" for k, v in rec.get("kernel_ms", {}).items())


def write_bench_table(which: str, out: str) -> str:
    d = os.path.join(out, "bench")
    runs = bench_runs(which)
    recs = [(lab, args, _bench_line(os.path.join(d, f"{lab}.json"))) for lab, args in runs]
    cmd = "python3 bench.py " + " ".join(runs[0][1])
    lines = []
    if which == "workloads":
        lines += ["# All workloads, one MI355X", "",
                  "Command (repository root on the GPU host), one run per workload (the first shown; "
                  "`python -m tiled_attention_fa_amd.profiling bench --set workloads` runs them all):", "",
                  "```", cmd, "```", "",
                  "Timed region: the listed kernels per step with inputs resident in HBM (`block_mask` is the mask "
                  "builder, counted in the step for the document workload). TFLOP/s = 4·D per admissible pair "
                  "(forward) + 10·D (backward), over Hq.", "",
                  "| workload | shape | mask | mod | pass | dtype | admissible pairs | ms / step | TFLOP/s | kernel ms "
                  "| dominant kernel | its frac of 2516.6 |",
                  "|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for lab, _, r in recs:
            c = r["config"]
            mask = c["mask"] + (f" w={c['window']}" if c.get("window") else "")
            lines.append(f"| {lab} | B{c['B']} Hq{c['Hq']} Hkv{c['Hkv']} S{c['S']} D{c['D']} | {mask} | {c['mod']} | "
                         f"{c['pass']} | {r['dtype']} | {c['admissible_pairs']:,} | {r['ms_per_step']:.4f} | "
                         f"{r['value']:.1f} | {_kernel_ms(r)} | {r['roofline']['kernel']} | "
                         f"{r['roofline']['frac']:.3f} |")
        name = "workloads_all_bench.md"
    elif which == "seqlen":
        lines += ["# Causal forward + backward by sequence length, H=16, D=128, bf16, one MI355X", "",
                  "Command (repository root on the GPU host), B x S = 16384 tokens up to S = 16384, then B = 1 "
                  "(the first shown):", "", "```", cmd, "```", "",
                  "TFLOP/s count admissible pairs only (4 D forward, 10 D backward). Kernel times are HIP-event "
                  f"averages over {BENCH_STEPS} steps after {BENCH_WARMUP} warm-up steps.", "",
                  "dQ ms includes the row pass (rowsum(dO * O)) fused into the dQ kernel; a separate row-pass "
                  "launch, where a run has one, is listed as delta ms.", "",
                  "| S | B | fwd+bwd TFLOP/s | fwd TFLOP/s | bwd TFLOP/s | fwd ms | delta ms | dK/dV ms | dQ ms |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for lab, _, r in recs:
            c, k = r["config"], r["kernel_ms"]
            delta = f"{k['bwd_delta']:.3f}" if "bwd_delta" in k else "-"
            lines.append(f"| {c['S']} | {c['B']} | {r['value']:.1f} | {r['fwd_tflops']:.1f} | {r['bwd_tflops']:.1f} | "
                         f"{k['fwd']:.3f} | {delta} | {k['bwd_dkdv']:.3f} | {k['bwd_dq']:.3f} |")
        name = "causal_by_seqlen.md"
    else:
        lines += ["# Schedule and dQ variants, one MI355X", "",
                  "Each workload with the static schedule (default) and the persistent work-queue schedule "
                  "(`--schedule persistent`), and the causal fwd+bwd with dQ recomputed (default) or read from the "
                  "dS blocks the dK/dV kernel stores (`--bwd-dq stored`); two rounds of all runs in alternation on "
                  "one box. Command of the first run:", "", "```", cmd, "```", "",
                  "| run | workload | schedule | dQ | ms / step | TFLOP/s | kernel ms |", "|---|---|---|---|---|---|---|"]
        for lab, _, r in recs:
            c = r["config"]
            lines.append(f"| {lab} | {c['workload']} | {c['schedule']} | {c.get('bwd_dq', '-')} | "
                         f"{r['ms_per_step']:.4f} | {r['value']:.1f} | {_kernel_ms(r)} |")
        name = "schedule_and_dq_variants.md"
    path = os.path.join(PROFILES, name)
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


# ---------------------------------------------------------------- workgroup traces
def run_wgtrace(workload: str, out: str, limit: int, shape=(0, 0)) -> str:
    d = os.path.join(os.path.abspath(out), "wgtrace")
    os.makedirs(d, exist_ok=True)
    path = os.path.join(d, label(workload, shape) + ".npy")
    args = _bench_args(workload, BENCH_STEPS, BENCH_WARMUP, shape) + ["--wg-trace", path]
    print(f"wgtrace: {label(workload, shape)}", flush=True)
    r = subprocess.run(["timeout", "-s", "KILL", str(limit), *args], cwd=ROOT, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True)
    with open(os.path.join(d, label(workload, shape) + ".log"), "w") as f:
        f.write(r.stdout)
    if r.returncode != 0:
        sys.exit(f"bench.py --wg-trace for {workload} ended with status {r.returncode}")
    return path


def _quantile(xs: list, q: float) -> float:
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(q * (len(xs) - 1) + 0.5))]


def wgtrace_stats(recs: list[dict]) -> dict:
    """Balance and cost figures of one traced launch (records of
    binding.decode_wg_trace)."""
    t_min = min(r["start_us"] for r in recs)
    span = max(r["end_us"] for r in recs) - t_min
    dur = [r["end_us"] - r["start_us"] for r in recs]
    by_cu: dict[int, list[dict]] = {}
    for r in recs:
        by_cu.setdefault(r["cu"], []).append(r)
    # Workgroups resident on a compute unit at once (the launch's occupancy).
    conc = 1
    gaps = []
    cu_end = []
    for tiles in by_cu.values():
        ev = sorted([(t["start_us"], 1) for t in tiles] + [(t["end_us"], -1) for t in tiles], key=lambda e: (e[0], e[1]))
        c = 0
        for _, d in ev:
            c += d
            conc = max(conc, c)
        ends = sorted(t["end_us"] for t in tiles)
        for t in tiles:  # time from the last end before this start (a freed slot) to this start
            prev = [e for e in ends if e <= t["start_us"]]
            if prev:
                gaps.append(t["start_us"] - prev[-1])
        cu_end.append(max(ends) - t_min)
    ideal = sum(dur) / (len(by_cu) * conc)
    # Least squares: duration = fixed + per_step * steps.
    n = len(recs)
    sx = sum(r["steps"] for r in recs)
    sy = sum(dur)
    sxx = sum(r["steps"] ** 2 for r in recs)
    sxy = sum(r["steps"] * d for r, d in zip(recs, dur))
    den = n * sxx - sx * sx
    per_step = (n * sxy - sx * sy) / den if den else 0.0
    fixed = (sy - per_step * sx) / n
    ss_tot = sum((d - sy / n) ** 2 for d in dur)
    ss_res = sum((d - fixed - per_step * r["steps"]) ** 2 for r, d in zip(recs, dur))
    xcds = {}
    for r, d in zip(recs, dur):
        x = xcds.setdefault(r["xcd"], {"tiles": 0, "busy_us": 0.0, "steps": 0, "end_us": 0.0})
        x["tiles"] += 1
        x["busy_us"] += d
        x["steps"] += r["steps"]
        x["end_us"] = max(x["end_us"], r["end_us"] - t_min)
    for x in xcds.values():
        x["us_per_step"] = x["busy_us"] / max(1, x["steps"])
    return {"tiles": n, "rows": recs[0]["rows"], "span_us": span, "compute_units": len(by_cu),
            "per_cu_concurrency": conc, "ideal_span_us": ideal,
            "cu_end_us": {"min": min(cu_end), "median": _quantile(cu_end, 0.5), "max": max(cu_end)},
            "gap_us": {"median": _quantile(gaps, 0.5), "p90": _quantile(gaps, 0.9), "n": len(gaps)} if gaps else None,
            "fit": {"fixed_us": fixed, "per_step_us": per_step, "r2": 1 - ss_res / ss_tot if ss_tot else 1.0},
            "xcd_match": sum(1 for r in recs if r["xcd"] == r["P"] % 8) / n,
            "xcds": dict(sorted(xcds.items()))}


def _wgtrace_table(title: str, st: dict, unit: str) -> list[str]:
    f = st["fit"]
    lines = [f"## {title}", "", "| figure | value |", "|---|---|",
             f"| tiles ({st['rows']} {unit} each) | {st['tiles']} |",
             f"| compute units seen, workgroups resident per unit | {st['compute_units']}, {st['per_cu_concurrency']} |",
             f"| span, first start to last end (us) | {st['span_us']:.1f} |",
             f"| ideal span: summed tile time / (units x resident) (us) | {st['ideal_span_us']:.1f} "
             f"({st['ideal_span_us'] / st['span_us']:.3f} of the span) |",
             f"| last end per compute unit, min / median / max (us) | {st['cu_end_us']['min']:.1f} / "
             f"{st['cu_end_us']['median']:.1f} / {st['cu_end_us']['max']:.1f} |"]
    if st["gap_us"]:
        lines.append(f"| slot freed to next start on that unit, median / p90 (us; {st['gap_us']['n']} starts) | "
                     f"{st['gap_us']['median']:.2f} / {st['gap_us']['p90']:.2f} |")
    lines += [f"| tile duration = fixed + per step x steps: fixed, per step (us), R^2 | {f['fixed_us']:.2f}, "
              f"{f['per_step_us']:.3f}, {f['r2']:.3f} |",
              f"| tiles whose XCD is their schedule index mod 8 | {st['xcd_match']:.3f} |", "",
              "| XCD | tiles | summed tile time (us) | steps | us per step | last end (us) |",
              "|---|---|---|---|---|---|"]
    for x, v in st["xcds"].items():
        lines.append(f"| {x} | {v['tiles']} | {v['busy_us']:.0f} | {v['steps']} | {v['us_per_step']:.3f} | "
                     f"{v['end_us']:.1f} |")
    return lines + [""]


def write_wgtrace_summary(workload: str, out: str, shape=(0, 0)) -> str:
    import numpy as np
    from . import binding
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import synth  # the workload shapes only
    lab = label(workload, shape)
    base = os.path.join(out, "wgtrace", lab)
    args = _bench_args(workload, BENCH_STEPS, BENCH_WARMUP, shape)
    cmd = " ".join("python3" if x == sys.executable else x for x in args).replace(ROOT, "<repo>")
    lines = [f"# Workgroup traces: {lab}", "",
             "Command (repository root on the GPU host; `python -m tiled_attention_fa_amd.profiling wgtrace` runs it):",
             "", "```", cmd + " --wg-trace <out>/wgtrace/" + lab + ".npy", "```", "",
             "After the timed steps, one more step runs with fa_mask_params.wg_trace: every workgroup records "
             "the GPU's 100 MHz clock at its start and end, its compute unit (XCC_ID, HW_ID) and its steps "
             "(forward: key steps of 64 keys; dK/dV: query steps of 32 rows; dQ: key steps of 64 keys).", ""]
    lines += _wgtrace_table("Forward", wgtrace_stats(binding.decode_wg_trace(np.load(base + ".npy"))), "query rows")
    if os.path.exists(base + ".bwd.npy"):
        w = synth.WORKLOADS[workload]
        B, S = shape[0] or w.B, shape[1] or w.S
        n_kv = B * w.Hkv * -(-S // binding.BLOCK)
        rec = np.load(base + ".bwd.npy")
        lines += _wgtrace_table("Backward dK/dV", wgtrace_stats(binding.decode_wg_trace(rec[:n_kv])), "keys")
        dq = binding.decode_wg_trace(rec[n_kv:])
        lines += _wgtrace_table("Backward dQ", wgtrace_stats(dq), "query rows")
    path = os.path.join(PROFILES, f"{lab}_wgtrace.md")
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    return path


def stall_stats(workload: str, out: str, shape=(0, 0)) -> dict[str, dict[str, float]]:
    """Per bench.py timing key: the stall passes' counters over the timed
    dispatches, as fractions.  The wave-time counters (SQ_WAVE_CYCLES,
    SQ_WAIT_*, SQ_ACTIVE_INST_*) are summed over all waves in one unit, so
    each is taken as a fraction of SQ_WAVE_CYCLES; the matrix-core counters
    are per SIMD and the LDS ones per compute unit, taken over the
    dispatch's cycles (SQ_BUSY_CYCLES / shader engines) times the SIMDs or
    compute units."""
    wdir = os.path.join(out, label(workload, shape))
    a = _dispatch_sums(os.path.join(wdir, "stallA"))
    b = _dispatch_sums(os.path.join(wdir, "stallB"))
    res = {}
    for name in a:
        key = kernel_key(name)
        if key is None or name not in b:
            continue
        x, y = a[name], b[name]
        wave = x["SQ_WAVE_CYCLES"]
        cyc_b = y["SQ_BUSY_CYCLES"] / SHADER_ENGINES
        res[key] = {
            "kernel_name": name,
            "wait_dependency": x["SQ_WAIT_ANY"] / wave,
            "wait_issue": x["SQ_WAIT_INST_ANY"] / wave,
            "wait_issue_lds": x["SQ_WAIT_INST_LDS"] / wave,
            "active_any": x["SQ_ACTIVE_INST_ANY"] / wave,
            "active_valu": x["SQ_ACTIVE_INST_VALU"] / wave,
            "active_lds": x["SQ_ACTIVE_INST_LDS"] / wave,
            "mfma_busy": y["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc_b * SIMDS),
            "mfma_coexec": y["SQ_VALU_MFMA_COEXEC_CYCLES"] / y["SQ_VALU_MFMA_BUSY_CYCLES"]
            if y["SQ_VALU_MFMA_BUSY_CYCLES"] else 0.0,
            "lds_active": y["SQ_LDS_IDX_ACTIVE"] / (cyc_b * COMPUTE_UNITS),
            "lds_cmd_fifo_full": y["SQ_LDS_CMD_FIFO_FULL"] / (cyc_b * COMPUTE_UNITS),
            "lds_data_fifo_full": y["SQ_LDS_DATA_FIFO_FULL"] / (cyc_b * COMPUTE_UNITS),
            "lds_bytes_per_cu_cycle": 64.0 * y["SQ_INSTS_LDS_LOAD_BANDWIDTH"] / (cyc_b * COMPUTE_UNITS),
            "lds_bytes_per_mfma": 64.0 * y["SQ_INSTS_LDS_LOAD_BANDWIDTH"] / y["SQ_INSTS_MFMA"]
            if y.get("SQ_INSTS_MFMA") else 0.0,
        }
    return res


def write_stall_summary(workload: str, out: str, shape=(0, 0)) -> str:
    st = stall_stats(workload, out, shape)
    lab = label(workload, shape)
    extra = "".join(f" --{k} {v}" for k, v in (("batch", shape[0]), ("seq-len", shape[1])) if v)
    lines = [f"# Where the waves spend their time: {lab}", "",
             "Commands (repository root on the GPU host; rocprofv3 from /tmp, one counter pass each):", "", "```"]
    for name, ctrs in STALL_PASSES.items():
        lines.append(f"rocprofv3 --pmc {' '.join(ctrs)} --output-format csv -o run -d <out>/{lab}/{name} -- "
                     f"python3 <repo>/bench.py --workload {workload} --no-cpu-baseline --steps {BENCH_STEPS} "
                     f"--warmup {BENCH_WARMUP}{extra}")
    lines += ["```", "",
              f"Averages over the {BENCH_STEPS} timed dispatches of each kernel. Wave time (fractions of "
              "SQ_WAVE_CYCLES, summed over all waves; the categories overlap): waiting on a dependency "
              "(SQ_WAIT_ANY), waiting to issue (SQ_WAIT_INST_ANY; of it, LDS instructions: SQ_WAIT_INST_LDS), "
              "working on any, VALU and LDS instructions (SQ_ACTIVE_INST_*). Matrix cores: SQ_VALU_MFMA_BUSY_CYCLES "
              f"over the dispatch's cycles x {SIMDS} SIMDs, and the share of those cycles in which a VALU "
              "instruction also issued (SQ_VALU_MFMA_COEXEC_CYCLES). LDS: SQ_LDS_IDX_ACTIVE and the FIFO-full "
              f"counters over cycles x {COMPUTE_UNITS} compute units, loaded bytes (64 x "
              "SQ_INSTS_LDS_LOAD_BANDWIDTH) per compute unit and cycle and per MFMA.", "",
              "| kernel | wait dependency | wait issue | of it LDS | active any | active VALU | active LDS | MFMA busy "
              "| MFMA co-exec VALU | LDS active | LDS cmd FIFO full | LDS data FIFO full | LDS B / CU cycle "
              "| LDS B / MFMA |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for key, v in sorted(st.items()):
        lines.append(f"| {key} | {v['wait_dependency']:.2f} | {v['wait_issue']:.2f} | {v['wait_issue_lds']:.2f} | "
                     f"{v['active_any']:.2f} | {v['active_valu']:.2f} | {v['active_lds']:.2f} | {v['mfma_busy']:.2f} | "
                     f"{v['mfma_coexec']:.2f} | {v['lds_active']:.2f} | {v['lds_cmd_fifo_full']:.3f} | "
                     f"{v['lds_data_fifo_full']:.3f} | {v['lds_bytes_per_cu_cycle']:.1f} | "
                     f"{v['lds_bytes_per_mfma']:.0f} |")
    lines += ["", f"Kernel sources of these figures: hash `{source_sha()}`.", ""]
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"{lab}_stalls.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("action", choices=["run", "summarize", "bench", "bench-summary", "wgtrace", "wgtrace-summary",
                                       "stalls", "stalls-summary"])
    ap.add_argument("--workload")
    ap.add_argument("--set", choices=["workloads", "seqlen", "variants"])
    ap.add_argument("--out", required=True)
    ap.add_argument("--limit", type=int, default=150, help="seconds per rocprofv3 pass")
    ap.add_argument("--batch", type=int, default=0, help="run the workload at this batch size")
    ap.add_argument("--seq-len", type=int, default=0, help="run the workload at this sequence length")
    args = ap.parse_args()
    shape = (args.batch, args.seq_len)
    if args.action in ("bench", "bench-summary"):
        if not args.set:
            ap.error("--set is required")
        if args.action == "bench":
            run_benches(args.set, args.out, max(args.limit, 300))
        else:
            print(write_bench_table(args.set, args.out))
        return
    if not args.workload:
        ap.error("--workload is required")
    if args.action == "wgtrace":
        run_wgtrace(args.workload, args.out, max(args.limit, 300), shape)
        return
    if args.action == "wgtrace-summary":
        print(write_wgtrace_summary(args.workload, args.out, shape))
        return
    if args.action == "stalls":
        run(args.workload, args.out, args.limit, shape, stalls=True)
        return
    if args.action == "stalls-summary":
        print(write_stall_summary(args.workload, args.out, shape))
        return
    if args.action == "run":
        run(args.workload, args.out, args.limit, shape)
    else:
        print(*[p for p in write_summary(summarize(args.workload, args.out, shape)) if p])


if __name__ == "__main__":
    main()
