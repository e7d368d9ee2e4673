"""Host logic of the rocprofv3 summary tool, on hand-made CSV files."""
import csv
import json
import os

import pytest

from tiled_attention_fa_amd import profiling

FWD = "void miattn::fwd_pp_kernel<128, 1, 0>(miattn::FwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _counters(path, rows, dur_ns=None):
    """rows: (dispatch, kernel, counter, value); dur_ns: dispatch -> duration."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                               "End_Timestamp"])
        w.writeheader()
        for d, k, c, v in rows:
            t0 = 1000 * d
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v,
                        "Start_Timestamp": t0, "End_Timestamp": t0 + (dur_ns or {}).get(d, 1)})


def _trace(path, rows):
    """rows: (kernel, [durations in ns, in dispatch order])."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        d = 0
        for name, durs in rows:
            for t in durs:
                d += 1
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Start_Timestamp": 10**9 * d,
                            "End_Timestamp": 10**9 * d + t})


@pytest.fixture
def fake_run(tmp_path, monkeypatch):
    out = tmp_path / "out"
    mib = profiling.COPY_MIB << 20
    # The copy reads half its bytes in FETCH_SIZE's KiB and all in WRITE_SIZE's.
    _counters(out / "copy_FETCH_SIZE", [(1, COPY, "FETCH_SIZE", mib / 2048)])
    _counters(out / "copy_WRITE_SIZE", [(1, COPY, "WRITE_SIZE", mib / 1024)])
    w = out / "gqa_causal_B1_S2048"
    n = profiling.BENCH_WARMUP + profiling.BENCH_STEPS
    # Every dispatch's counter is split over two rows (summed); the warm-up
    # dispatches read differently and must be left out.
    fetch, write = [], []
    for d in range(1, n + 1):
        warm = d <= profiling.BENCH_WARMUP
        fetch += [(d, FWD, "FETCH_SIZE", 9000 if warm else 3000), (d, FWD, "FETCH_SIZE", 1000)]
        write += [(d, FWD, "WRITE_SIZE", 9000 if warm else 600)]
    _counters(w / "FETCH_SIZE", fetch)
    _counters(w / "WRITE_SIZE", write)
    sq = {"SQ_BUSY_CYCLES": 32 * 1.5e5, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1.5e5 * 1024, "SQ_INSTS_VALU": 730,
          "SQ_INSTS_MFMA": 100, "SQ_INSTS_LDS": 150, "SQ_LDS_BANK_CONFLICT": 0}
    # 1.5e5 cycles in 100 us (1.5 GHz) per timed dispatch; warm-up dispatches take 300 us.
    _counters(w / "sq", [(d, FWD, c, v) for d in range(1, n + 1) for c, v in sq.items()],
              {d: 300e3 if d <= profiling.BENCH_WARMUP else 100e3 for d in range(1, n + 1)})
    _trace(w / "trace", [(FWD, [400e3] * profiling.BENCH_WARMUP + [100e3, 110e3, 90e3] + [100e3] *
                          (profiling.BENCH_STEPS - 3)), ("some_torch_kernel", [1e3] * 5)])
    monkeypatch.setattr(profiling, "PROFILES", str(tmp_path / "profiles"))
    return out


def test_summary_scales_and_derives(fake_run, tmp_path):
    rec = profiling.summarize("gqa_causal", str(fake_run), (1, 2048))
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    k = rec["kernels"]["fwd"]
    assert set(rec["kernels"]) == {"fwd"}  # kernels of other libraries are left out
    assert k["fetch_kib"] == pytest.approx(4000) and k["write_kib"] == pytest.approx(600)
    assert k["bytes_per_launch"] == round(4000 * 1024 * 2 + 600 * 1024)
    assert k["clock_ghz"] == pytest.approx(1.5)  # 1.5e5 cycles in 100 us
    assert k["timed_calls"] == profiling.BENCH_STEPS and k["calls"] == profiling.BENCH_STEPS + profiling.BENCH_WARMUP
    assert k["avg_us"] == pytest.approx(100.0) and k["min_us"] == pytest.approx(90.0)
    assert k["max_us"] == pytest.approx(110.0) and k["avg_all_us"] > 150.0
    assert k["mfma_busy"] == pytest.approx(0.5)
    assert k["valu_per_mfma"] == pytest.approx(7.3) and k["lds_per_mfma"] == pytest.approx(1.5)
    # Compulsory forward bytes of B1 Hq32 Hkv8 S2048 D128 bf16.
    assert rec["compulsory"] == {"read": (32 + 2 * 8) * 2048 * 128 * 2, "written": 32 * 2048 * (128 * 2 + 4)}
    jpath, mpath = profiling.write_summary(rec)
    assert jpath is None  # an overridden shape writes no traffic file for bench.py
    assert os.path.basename(mpath) == "gqa_causal_B1_S2048_counters.md"
    text = open(mpath).read()
    assert "--batch 1 --seq-len 2048" in text and "Compulsory bytes" in text


def test_default_shape_writes_traffic_file(fake_run):
    os.rename(fake_run / "gqa_causal_B1_S2048", fake_run / "gqa_causal")
    rec = profiling.summarize("gqa_causal", str(fake_run))
    jpath, _ = profiling.write_summary(rec)
    data = json.load(open(jpath))
    assert data["source_sha"] == profiling.source_sha()
    assert data["kernels"]["fwd"]["bytes_per_launch"] == round(4000 * 1024 * 2 + 600 * 1024)
    assert "compulsory" not in rec


def test_kernel_keys():
    assert profiling.kernel_key(FWD) == "fwd"
    assert profiling.kernel_key("void miattn::bwd_dq_ds_kernel<128, 1>(miattn::BwdArgs)") == "bwd_dq"
    assert profiling.kernel_key("void miattn::bwd_dkdv_kernel<128, 1, 0, false, false>(miattn::BwdArgs)") == "bwd_dkdv"
    assert profiling.kernel_key(COPY) is None


def _fake_bench(label, args):
    w = args[args.index("--workload") + 1]
    bwd = w == "causal_fwd_bwd"
    rec = {"value": 800.0, "ms_per_step": 2.25, "dtype": "bf16", "fwd_tflops": 1000.0, "bwd_tflops": 700.0,
           "config": {"workload": w, "B": 2, "Hq": 16, "Hkv": 16, "S": 8192, "D": 128, "mask": "causal",
                      "mod": "none", "window": 0, "pass": "fwd+bwd" if bwd else "fwd", "admissible_pairs": 1000,
                      "schedule": "persistent" if "persistent" in label else "static",
                      **({"bwd_dq": "stored" if "stored" in label else "recompute"} if bwd else {})},
           "kernel_ms": {"fwd": 0.5, **({"bwd_delta": 0.03, "bwd_dkdv": 1.0, "bwd_dq": 0.7} if bwd else {})},
           "roofline": {"kernel": "bwd_dkdv" if bwd else "fwd", "frac": 0.43}}
    return "some log line\n" + json.dumps(rec) + "\n"


@pytest.mark.parametrize("which,name,rows", [("workloads", "workloads_all_bench.md", 10),
                                             ("seqlen", "causal_by_seqlen.md", 6),
                                             ("variants", "schedule_and_dq_variants.md", 24)])
def test_bench_tables(tmp_path, monkeypatch, which, name, rows):
    monkeypatch.setattr(profiling, "PROFILES", str(tmp_path / "profiles"))
    d = tmp_path / "out" / "bench"
    d.mkdir(parents=True)
    runs = profiling.bench_runs(which)
    assert len(runs) == rows and len({lab for lab, _ in runs}) == rows
    for lab, args in runs:
        (d / f"{lab}.json").write_text(_fake_bench(lab, args))
    path = profiling.write_bench_table(which, str(tmp_path / "out"))
    assert os.path.basename(path) == name
    table = [ln for ln in open(path).read().splitlines() if ln.startswith("| ") and not ln.startswith("| workload |")
             and not ln.startswith("| S |") and not ln.startswith("| run |")]
    assert len(table) == rows
    assert "python3 bench.py --workload" in open(path).read()


def test_wgtrace_decode_and_stats(tmp_path, monkeypatch):
    """Records of two compute units on XCDs 0 and 1, each running two
    workgroups at once; tile time 2 us + 0.5 us per step."""
    import numpy as np

    from tiled_attention_fa_amd import binding
    rec = np.zeros((8, binding.FA_WG_TRACE_WORDS), dtype=np.int64)
    # P, start (us), steps, xcd, cu field (HW_ID bits 15:8)
    plan = [(0, 0.0, 4, 0, 3), (2, 0.0, 8, 0, 3), (1, 0.0, 4, 1, 5), (3, 0.0, 2, 1, 5),
            (4, 4.5, 2, 0, 3), (5, 3.5, 6, 1, 5)]
    for p, t0, steps, xcd, cu in plan:
        dur = 2.0 + 0.5 * steps
        rec[p] = [int(t0 * 100), int((t0 + dur) * 100), (xcd << 32) | (cu << 8) | 0x3, (128 << 32) | steps]
    recs = binding.decode_wg_trace(rec)
    assert len(recs) == 6 and {r["P"] for r in recs} == {0, 1, 2, 3, 4, 5}  # unwritten records skipped
    assert all(r["rows"] == 128 for r in recs) and {r["cu"] for r in recs} == {(0 << 8) | 3, (1 << 8) | 5}
    st = profiling.wgtrace_stats(recs)
    assert st["compute_units"] == 2 and st["per_cu_concurrency"] == 2
    assert st["fit"]["fixed_us"] == pytest.approx(2.0) and st["fit"]["per_step_us"] == pytest.approx(0.5)
    assert st["fit"]["r2"] == pytest.approx(1.0)
    assert st["span_us"] == pytest.approx(8.5)  # P 5: 3.5 + 5
    assert st["ideal_span_us"] == pytest.approx(sum(2.0 + 0.5 * s for _, _, s, _, _ in plan) / 4)
    assert st["xcd_match"] == pytest.approx(sum(p % 8 == x for p, _, _, x, _ in plan) / len(plan))
    assert st["gap_us"]["median"] == pytest.approx(0.5)  # P 4 starts 0.5 us after P 0 ends; P 5 at 0.5 after P 3
    assert st["xcds"][0]["steps"] == 14 and st["xcds"][1]["steps"] == 12
    d = tmp_path / "out" / "wgtrace"
    d.mkdir(parents=True)
    np.save(d / "gqa_causal.npy", rec)
    monkeypatch.setattr(profiling, "PROFILES", str(tmp_path / "profiles"))
    text = open(profiling.write_wgtrace_summary("gqa_causal", str(tmp_path / "out"))).read()
    assert "--wg-trace" in text and "| 0 | 3 |" in text


def test_stall_stats_and_summary(tmp_path, monkeypatch):
    """The stall passes' counters as fractions: wave-time counters over
    SQ_WAVE_CYCLES, matrix-core counters over cycles x SIMDs, LDS counters
    over cycles x compute units; warm-up dispatches left out."""
    out = tmp_path / "out"
    w = out / "gqa_causal"
    n = profiling.BENCH_WARMUP + profiling.BENCH_STEPS
    cyc = 1.5e5  # per dispatch; SQ_BUSY_CYCLES is summed over the shader engines
    a = {"SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 400.0, "SQ_WAIT_INST_ANY": 250.0, "SQ_WAIT_INST_LDS": 50.0,
         "SQ_ACTIVE_INST_ANY": 600.0, "SQ_ACTIVE_INST_VALU": 300.0, "SQ_ACTIVE_INST_LDS": 100.0,
         "SQ_BUSY_CYCLES": cyc * profiling.SHADER_ENGINES}
    b = {"SQ_VALU_MFMA_BUSY_CYCLES": 0.6 * cyc * profiling.SIMDS, "SQ_VALU_MFMA_COEXEC_CYCLES": 0.15 * cyc * profiling.SIMDS,
         "SQ_LDS_IDX_ACTIVE": 0.5 * cyc * profiling.COMPUTE_UNITS, "SQ_LDS_DATA_FIFO_FULL": 0.0,
         "SQ_LDS_CMD_FIFO_FULL": 0.01 * cyc * profiling.COMPUTE_UNITS,
         "SQ_INSTS_LDS_LOAD_BANDWIDTH": 2.0 * cyc * profiling.COMPUTE_UNITS, "SQ_INSTS_MFMA": 128.0 * cyc,
         "SQ_BUSY_CYCLES": cyc * profiling.SHADER_ENGINES}
    assert set(a) == set(profiling.STALL_PASSES["stallA"]) and set(b) == set(profiling.STALL_PASSES["stallB"])
    for name, ctrs in (("stallA", a), ("stallB", b)):
        rows = []
        for d in range(1, n + 1):
            warm = d <= profiling.BENCH_WARMUP
            # every counter split over two rows; warm-up dispatches read 3x
            rows += [(d, FWD, c, (3.0 if warm else 1.0) * v / 2) for c, v in ctrs.items() for _ in range(2)]
        _counters(w / name, rows)
    st = profiling.stall_stats("gqa_causal", str(out))["fwd"]
    assert st["wait_dependency"] == pytest.approx(0.4) and st["wait_issue"] == pytest.approx(0.25)
    assert st["wait_issue_lds"] == pytest.approx(0.05) and st["active_any"] == pytest.approx(0.6)
    assert st["active_valu"] == pytest.approx(0.3) and st["active_lds"] == pytest.approx(0.1)
    assert st["mfma_busy"] == pytest.approx(0.6) and st["mfma_coexec"] == pytest.approx(0.25)
    assert st["lds_active"] == pytest.approx(0.5) and st["lds_cmd_fifo_full"] == pytest.approx(0.01)
    assert st["lds_bytes_per_cu_cycle"] == pytest.approx(128.0)
    assert st["lds_bytes_per_mfma"] == pytest.approx(64.0 * 2.0 * profiling.COMPUTE_UNITS / 128.0)
    monkeypatch.setattr(profiling, "PROFILES", str(tmp_path / "profiles"))
    text = open(profiling.write_stall_summary("gqa_causal", str(out))).read()
    assert "| fwd | 0.40 | 0.25 | 0.05 |" in text and "--pmc SQ_WAVE_CYCLES" in text
