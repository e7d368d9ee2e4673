#!/usr/bin/env python3
"""Benchmark of libmiattn on one MI355X.

Default workload: causal attention forward + backward, B=2, Hq=Hkv=16,
S=8192, D=128, bf16, seeded N(0,1) inputs already resident in HBM.  One
step = fa_fwd (with LSE) then the backward: the dQ kernel with the row pass
(rowsum(dO * O)) fused in, then dK/dV; with --bwd-dq stored the row pass,
dK/dV, then dQ from the stored dS.  Throughput counts admissible-pair FLOPs only (4 D per pair forward,
10 D backward) and is compared with the dense bf16 MFMA peak.

Per-kernel times come from HIP events recorded between the launches on the
stream the library launches on.  The CPU baseline times the fp64 oracle on a
bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--seq-len S] [--batch B] [--oracle full]
Prints one JSON line.  With --seq-len / --batch the profile-derived fields
(roofline.traffic, clock) are null: the committed counters are for the
workload's own shape.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOPS (unmasked FLOPs) + % of bf16 MFMA peak, S=8192 D=128"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_FP8_TFLOPS = 5033.2    # 256 CU x 2.4 GHz x 8192 dense fp8 flop/clk/CU
PEAK_HBM_GBS = 8000.0
MASK_NAMES = {0: "none", 1: "causal", 2: "sliding_window", 3: "document"}
MOD_NAMES = {0: "none", 1: "alibi", 2: "softcap", 3: "local_boost"}


def source_sha() -> str:
    """Hash of the kernel sources: traffic figures taken from another build are void."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "tiled_attention_fa_amd", "csrc")
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_profile(workload: str, kernel: str) -> dict:
    """The committed rocprofv3 figures of one kernel (HBM bytes per launch,
    average shader clock), or {} when there are none for this kernel or the
    sources changed since they were taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return {}
    rec = json.load(open(p))
    k = rec.get("kernels", {}).get(kernel)
    if not k or rec.get("source_sha") != source_sha():
        return {}
    return k


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, or None."""
    return measured_profile(workload, kernel).get("bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def affinity_cores() -> int:
    """Host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return os.cpu_count() or 1


class _OracleJob:
    """The oracle's work for whole (batch, head) pairs of one workload: the
    inputs are generated once per process from the workload's seeds."""

    def __init__(self, w):
        import oracle
        import synth
        from tiled_attention_fa_amd.binding import default_scale

        self.w = w
        self.q, self.k, self.v, self.extras = synth.workload_inputs(w)
        doc = self.extras.get("doc_ids")
        self.var = oracle.Variant(mask=w.mask, window=w.window, mod=w.mod, softcap=w.softcap,
                                  boost_radius=w.boost_radius, boost_factor=w.boost_factor,
                                  doc_ids=None if doc is None else doc.numpy())
        self.scale = default_scale(w.D)

    def head_flops(self) -> float:
        """Admissible-pair FLOPs of one (batch, head): 4 D per pair forward, + 10 D backward."""
        from tiled_attention_fa_amd import flops
        w = self.w
        per_head = flops.pairs_per_row_batch(w.mask, w.S, w.S, w.window, self.extras.get("doc_lengths"))
        return float(per_head * ((4 + 10) * w.D if w.backward else 4 * w.D))

    def run(self, b: int, h: int) -> None:
        import oracle
        w, q, k, v = self.w, self.q, self.k, self.v
        hk = h // (w.Hq // w.Hkv)
        if w.backward:
            oracle.backward_head(q[b, h], k[b, hk], v[b, hk], self.extras["do"][b, h], self.scale, self.var,
                                 b, h, w.Hq)
        else:
            oracle.forward(q[b:b + 1, h:h + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1], self.scale, self.var)


def cpu_baseline(w, heads: int):
    """The oracle (numpy fp64, as committed) on `heads` whole (batch, head)
    pairs of the workload with the BLAS library's threads, plus one head on a
    single core (pairs per second per core); returns the dict for the JSON line."""
    from threadpoolctl import threadpool_limits

    job = _OracleJob(w)
    threads = _blas_threads()
    info = {"cpu_model": cpu_model(), "affinity_cores": affinity_cores()}
    if w.dtype == "fp8":
        return {**_cpu_baseline_fp8(w, job.q, job.k, job.v, job.var, job.scale, max(1, heads // 16), threads),
                **info}  # ~20 s a head
    todo = [(0, h) for h in range(min(heads, w.Hq))]
    t0 = time.perf_counter()
    for b, h in todo:
        job.run(b, h)
    dt = time.perf_counter() - t0
    hf = job.head_flops()
    pairs_per_head = hf / ((4 + 10) * w.D if w.backward else 4 * w.D)
    # One more head on one core: the per-core rate, free of BLAS threading.
    with threadpool_limits(1):
        t1 = time.perf_counter()
        job.run(0, min(heads, w.Hq) % w.Hq)
        dt1 = time.perf_counter() - t1
    return {"value": hf * len(todo) / dt / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "seconds": dt, **info,
            "per_core": {"pairs_per_s": pairs_per_head / dt1, "tflops": hf / dt1 / 1e12, "seconds": dt1,
                         "sample": "one more (batch, head) pair, BLAS limited to one thread"},
            "sample": f"{'forward+backward' if w.backward else 'forward'} of {len(todo)} of {w.B * w.Hq} "
                      f"(batch, head) pairs at full S={w.S}, numpy float64 with {threads} BLAS threads; "
                      f"value = admissible-pair FLOPs of that sample / its time"}


def _full_worker(args):
    """One process of the full oracle run: BLAS on one thread, a share of the heads."""
    name, heads = args
    import synth
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        job = _OracleJob(synth.WORKLOADS[name])
        t0 = time.perf_counter()
        for b, h in heads:
            job.run(b, h)
        return time.perf_counter() - t0


def oracle_full(name: str, procs: int) -> dict:
    """Every (batch, head) pair of the workload through the oracle, one
    single-threaded process per core (no threads inside the oracle)."""
    import multiprocessing as mp

    import synth
    w = synth.WORKLOADS[name]
    if w.dtype == "fp8":
        raise SystemExit("--oracle full covers the bf16 and fp32 workloads")
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    procs = max(1, min(procs, len(heads)))
    shares = [heads[i::procs] for i in range(procs)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(procs) as pool:
        busy = pool.map(_full_worker, [(name, sh) for sh in shares])
    wall = time.perf_counter() - t0
    hf = _OracleJob(w).head_flops()
    return {"workload": name, "kind": "oracle", "mode": "full", "heads": len(heads), "processes": procs,
            "cpu_model": cpu_model(), "affinity_cores": affinity_cores(), "wall_s": round(wall, 2),
            "busy_s_per_process": [round(x, 2) for x in busy], "tflops": hf * len(heads) / wall / 1e12,
            "pairs_per_s_per_core": hf / ((4 + 10) * w.D if w.backward else 4 * w.D) * len(heads) / sum(busy)}


def _cpu_baseline_fp8(w, q, k, v, var, scale, heads, threads):
    """The FP8 oracle (quantization and the FP8 forward emulation, numpy
    float64) on `heads` whole heads, rows in chunks of 2048."""
    import numpy as np
    import torch

    import synth
    from oracle import fp8 as ofp8
    from tiled_attention_fa_amd import flops

    s = synth.signs(w.D, synth.FP8_SIGN_SEED).numpy()

    def f64(t):
        return t.to(torch.float64).numpy()
    t0 = time.perf_counter()
    for h in range(heads):
        hk = h // (w.Hq // w.Hkv)
        q8, qs = ofp8.block_quantize(f64(q[0, h])[None], s)
        k8, ks = ofp8.block_quantize(f64(k[0, hk])[None], s)
        v8, vs = ofp8.block_quantize(f64(v[0, hk])[None])
        for r0 in range(0, w.S, 2048):
            ofp8.fp8_forward(q8, k8, v8, qs, ks, vs, scale, var, rows=np.arange(r0, min(w.S, r0 + 2048)))
    dt = time.perf_counter() - t0
    per_head = flops.pairs_per_row_batch(w.mask, w.S, w.S, w.window, None)
    return {"value": per_head * heads * 4 * w.D / dt / 1e12, "unit": "TFLOPS", "cores": int(threads),
            "kind": "oracle", "seconds": dt,
            "sample": f"FP8 quantization + FP8 forward emulation of {heads} of {w.B * w.Hq} (batch, head) pairs "
                      f"at full S={w.S}, numpy float64 with {threads} BLAS threads; value = admissible-pair "
                      f"FLOPs of that sample / its time"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="causal_fwd_bwd")
    ap.add_argument("--seq-len", type=int, default=0, help="run the workload at this sequence length instead")
    ap.add_argument("--batch", type=int, default=0, help="run the workload at this batch size instead")
    ap.add_argument("--cpu-heads", type=int, default=16, help="heads of the oracle CPU baseline sample")
    ap.add_argument("--oracle", choices=["sample", "full"], default="sample",
                    help="full: only run the oracle over every head of the workload, one single-threaded "
                         "process per host core (up to --oracle-procs), print one JSON line, no GPU work")
    ap.add_argument("--oracle-procs", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd-dq", choices=["stored", "recompute"], default="recompute",
                    help="stored: the backward workspace has room for dS (fa_bwd_ds_workspace_bytes) where the "
                         "mask allows, so the dQ launch reads dS instead of recomputing it")
    ap.add_argument("--schedule", choices=["static", "persistent"], default="static",
                    help="persistent: the forward takes its query tiles from a work queue "
                         "(fa_mask_params.work_queue)")
    ap.add_argument("--wg-trace", default="", metavar="FILE.npy",
                    help="after the timed steps, run one more step whose forward records each query tile's "
                         "start, end, compute unit and size (fa_mask_params.wg_trace) and save the records; "
                         "with a backward, its dK/dV and dQ records go to FILE.bwd.npy")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times) and exit: the reference for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs on one GPU (no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.oracle == "full":
        print(json.dumps({"oracle_full": oracle_full(args.workload, min(args.oracle_procs, affinity_cores()))}),
              flush=True)
        return

    import torch

    import synth
    import tiled_attention_fa_amd as fa
    from tiled_attention_fa_amd import flops

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return
    fa.lib()
    if args.workload not in synth.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; choose from {sorted(synth.WORKLOADS)}")
    w = synth.WORKLOADS[args.workload]
    reshaped = bool(args.seq_len or args.batch)
    if reshaped:
        w = dataclasses.replace(w, S=args.seq_len or w.S, B=args.batch or w.B)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, extras = synth.workload_inputs(w)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    do = extras["do"].to(dev) if w.backward else None
    doc = extras["doc_ids"].to(dev) if "doc_ids" in extras else None
    kw = dict(mask=w.mask, window=w.window, doc_ids=doc, mod=w.mod, softcap=w.softcap,
              boost_radius=w.boost_radius, boost_factor=w.boost_factor)
    stream = torch.cuda.current_stream()
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if w.backward else None
    ws_bytes = fa.fa_bwd_workspace_bytes(w.B, w.Hq, w.S, w.D)
    if w.backward and args.bwd_dq == "stored":
        ws_bytes = max(ws_bytes, fa.fa_bwd_ds_workspace_bytes(w.B, w.Hq, w.S, w.S, w.D, w.mask))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    use_bm = w.mask == fa.MASK_DOCUMENT
    bm = fa.build_block_mask(w.mask, w.B, w.S, w.S, window=w.window, doc_ids=doc) if use_bm else None
    wq = fa.new_work_queue(dev) if args.schedule == "persistent" else None

    # Backward launches in stream order, each timed by its own pair of events.
    if args.bwd_dq == "stored":
        bwd_calls = [("bwd_delta", fa.FA_BWD_DELTA), ("bwd_dkdv", fa.FA_BWD_DKDV), ("bwd_dq", fa.FA_BWD_DQ)]
    else:
        bwd_calls = [("bwd_dq", fa.FA_BWD_DELTA | fa.FA_BWD_DQ), ("bwd_dkdv", fa.FA_BWD_DKDV)]
    names = (["block_mask"] if use_bm else []) + ["fwd"] + ([n for n, _ in bwd_calls] if w.backward else [])
    is_fp8 = w.dtype == "fp8"
    if is_fp8:
        # Quantized once, outside the timed region (as the FP8 tables of the
        # pages exclude the quantization time); Q and K with incoherent processing.
        signs = synth.signs(w.D, synth.FP8_SIGN_SEED).to(dev)
        q8, qs = fa.quantize_fp8(q, signs)
        k8, ks = fa.quantize_fp8(k, signs)
        v8, vs = fa.quantize_fp8(v)
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)

    def step(evs):
        i = 0
        if evs:
            evs[i].record(stream)
        if is_fp8:
            fa.forward_fp8(q8, k8, v8, qs, ks, vs, mask=w.mask, window=w.window, out=out, lse=lse,
                           return_lse=w.lse)
            if evs:
                evs[1].record(stream)
            return
        if use_bm:
            fa.build_block_mask(w.mask, w.B, w.S, w.S, window=w.window, doc_ids=doc, into=bm)
            i += 1
            if evs:
                evs[i].record(stream)
        fa.forward(q, k, v, out=out, lse=lse, return_lse=w.lse or w.backward, block_mask=bm, work_queue=wq,
                   wg_trace=trace_buf[0], **kw)
        i += 1
        if evs:
            evs[i].record(stream)
        if w.backward:
            for _, ph in bwd_calls:
                fa.backward(q, k, v, out, do, lse, block_mask=bm, workspace=ws, grads=grads, phases=ph,
                            wg_trace=trace_buf[1], **kw)
                i += 1
                if evs:
                    evs[i].record(stream)

    trace_buf = [None, None]  # forward, backward: set for the one traced step after the timed ones
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        step(evs[s])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps
    if args.wg_trace:
        # One more step, untimed, its forward recording where and when each
        # query tile ran (fa_mask_params.wg_trace; static schedule only).
        if is_fp8 or wq is not None:
            sys.exit("--wg-trace covers the bf16/fp32 forward with the static schedule")
        import numpy as np
        trace_buf[0] = fa.new_wg_trace(w.B, w.Hq, w.S, dev)
        if w.backward:
            trace_buf[1] = fa.new_wg_trace(w.B, w.Hq, w.S, dev, Hkv=w.Hkv, Skv=w.S)
        step(None)
        torch.cuda.synchronize()
        np.save(args.wg_trace, trace_buf[0].cpu().numpy())
        if w.backward:  # dK/dV records, then dQ records
            np.save(args.wg_trace[:-4] + ".bwd.npy" if args.wg_trace.endswith(".npy") else args.wg_trace + ".bwd.npy",
                    trace_buf[1].cpu().numpy())
        trace_buf[0] = trace_buf[1] = None
    per_step = {n: sorted(e[i].elapsed_time(e[i + 1]) for e in evs) for i, n in enumerate(names)}
    kernel_ms = {n: sum(t) / args.steps for n, t in per_step.items()}

    npairs = flops.pairs(w.mask, w.B, w.Hq, w.S, w.S, w.window, extras.get("doc_lengths"))
    f_fwd = flops.fwd_flops(npairs, w.D)
    f_bwd = flops.bwd_flops(npairs, w.D) if w.backward else 0.0
    tflops = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    # Algorithmic FLOPs per launch: the forward kernel does the two forward
    # contractions; the dK/dV kernel the recomputed Q K^T, dO V^T, P^T dO and
    # dS^T Q; the dQ kernel is credited with dS K only (its recomputation of
    # Q K^T and dO V^T repeats work the dK/dV kernel already counts).
    algo = {"fwd": f_fwd, "bwd_dkdv": 8.0 * w.D * npairs, "bwd_dq": 2.0 * w.D * npairs}
    dominant = max((n for n in names if n in algo), key=lambda n: kernel_ms[n])
    peak = PEAK_FP8_TFLOPS if is_fp8 else PEAK_BF16_TFLOPS  # a contraction takes its own dtype's peak
    achieved = algo[dominant] / (kernel_ms[dominant] * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3"}.get(w.dtype, "f32"),
        "data": "synthetic: seeded N(0,1) tensors of the workload's shape",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "D": w.D,
                   "mask": MASK_NAMES[w.mask], "mod": MOD_NAMES[w.mod], "window": w.window,
                   "pass": "fwd+bwd" if w.backward else "fwd", "lse": bool(w.lse or w.backward),
                   "admissible_pairs": npairs, "schedule": args.schedule,
                   **({"bwd_dq": args.bwd_dq, "workspace_bytes": ws_bytes} if w.backward else {})},
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        **({"pct_of_fp8_peak": round(100.0 * tflops / PEAK_FP8_TFLOPS, 2)} if is_fp8 else {}),
        "fwd_tflops": round(f_fwd / (kernel_ms["fwd"] * 1e-3) / 1e12, 2),
        "bwd_tflops": round(f_bwd / (sum(kernel_ms[n] for n in names if n.startswith("bwd")) * 1e-3) / 1e12, 2)
        if w.backward else None,
        "kernel_ms": {n: round(t, 4) for n, t in kernel_ms.items()},
        "kernel_ms_median": {n: round(statistics.median(t), 4) for n, t in per_step.items()},
        "kernel_ms_min": {n: round(t[0], 4) for n, t in per_step.items()},
        "wall_s": round(wall, 3),
        **({"wg_trace": args.wg_trace} if args.wg_trace else {}),
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": None if reshaped else measured_traffic(w.name, dominant)},
    }
    # The peak scaled to the shader clock the profiler saw under this kernel
    # (busy cycles over duration); the nominal peak assumes 2.4 GHz.
    ghz = None if reshaped else measured_profile(w.name, dominant).get("clock_ghz")
    rec["clock"] = None if ghz is None else {
        "kernel": dominant, "ghz": round(ghz, 3), "peak_at_clock": round(peak * ghz / 2.4, 1),
        "frac_at_clock": round(achieved / (peak * ghz / 2.4), 4)}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_heads)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
