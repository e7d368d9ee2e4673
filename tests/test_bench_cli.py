"""bench.py's host-side contract, run as the driver runs it (a subprocess):
more than one GPU is refused with a message before any GPU work, and the
oracle-only mode needs no GPU and prints one JSON line."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr


def test_oracle_full_runs_on_the_host():
    """The full-oracle mode on the small fp32 workload (B1 H2 S256 D64):
    every head through the fp64 oracle in two processes, one JSON line."""
    r = _bench("--workload", "tiny_mha_f32", "--oracle", "full", "--oracle-procs", "2")
    assert r.returncode == 0, r.stderr
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])["oracle_full"]
    assert rec["workload"] == "tiny_mha_f32" and rec["kind"] == "oracle" and rec["mode"] == "full"
    assert rec["heads"] == 2 and rec["processes"] == 2 and len(rec["busy_s_per_process"]) == 2
    assert rec["tflops"] > 0 and rec["pairs_per_s_per_core"] > 0 and rec["affinity_cores"] >= 1
