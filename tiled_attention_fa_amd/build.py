"""Compile libmiattn.so for gfx950 in-tree with hipcc.

Every HIP translation unit in csrc/ is compiled in parallel, then linked
into tiled_attention_fa_amd/libmiattn.so.  Run as
``python -m tiled_attention_fa_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmiattn.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for all device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libmiattn needs ROCm to build")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O2", "-std=c++17", "-fPIC", "-x", "hip",
               "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libmiattn.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    _check_no_missing_kernels(tmp)
    os.replace(tmp, LIB)
    return LIB


def _check_no_missing_kernels(path: str) -> None:
    """A kernel whose host-side launch stub was not emitted leaves an undefined
    symbol of the library's own namespace that only fails at load time; fail
    the build instead."""
    nm = shutil.which("nm") or "/usr/bin/nm"
    r = subprocess.run([nm, "-D", "--undefined-only", path], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"nm failed on {path}:\n{r.stderr}")
    missing = [ln.split()[-1] for ln in r.stdout.splitlines() if "_ZN6miattn" in ln]
    if missing:
        raise RuntimeError(f"{len(missing)} undefined library symbols, e.g. {missing[:3]}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
