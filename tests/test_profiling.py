"""Host logic of the rocprofv3 summary tool, on hand-made CSV files."""
import csv
import json
import os

import pytest

from tiled_attention_fa_amd import profiling

FWD = "void miattn::fwd_pp_kernel<128, 1, 0>(miattn::FwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, k, c, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def _stats(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_kernel_stats.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        for name, calls, avg in rows:
            w.writerow({"Name": name, "Calls": calls, "TotalDurationNs": calls * avg, "AverageNs": avg,
                        "MinNs": avg, "MaxNs": avg})


@pytest.fixture
def fake_run(tmp_path, monkeypatch):
    out = tmp_path / "out"
    mib = profiling.COPY_MIB << 20
    # The copy reads half its bytes in FETCH_SIZE's KiB and all in WRITE_SIZE's.
    _counters(out / "copy_FETCH_SIZE", [(1, COPY, "FETCH_SIZE", mib / 2048)])
    _counters(out / "copy_WRITE_SIZE", [(1, COPY, "WRITE_SIZE", mib / 1024)])
    w = out / "gqa_causal_B1_S2048"
    # Two dispatches; each dispatch's counter is split over two rows (summed).
    _counters(w / "FETCH_SIZE", [(1, FWD, "FETCH_SIZE", 3000), (1, FWD, "FETCH_SIZE", 1000),
                                 (2, FWD, "FETCH_SIZE", 2500), (2, FWD, "FETCH_SIZE", 1500)])
    _counters(w / "WRITE_SIZE", [(1, FWD, "WRITE_SIZE", 500), (2, FWD, "WRITE_SIZE", 700)])
    sq = {"SQ_BUSY_CYCLES": 32 * 1.5e5, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1.5e5 * 1024, "SQ_INSTS_VALU": 730,
          "SQ_INSTS_MFMA": 100, "SQ_INSTS_LDS": 150, "SQ_LDS_BANK_CONFLICT": 0}
    _counters(w / "sq", [(1, FWD, c, v) for c, v in sq.items()])
    _stats(w / "trace", [(FWD, 13, 100e3), ("some_torch_kernel", 5, 1e3)])
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
