"""Build the gfx950 HIP library ``libsla.so`` in-tree with hipcc.

Usage: ``python -m sparse_linear_attention_mean_amd.builder`` (or ``build()``).
Every ``csrc/*.hip`` file is compiled to an object (in parallel) and linked
into ``sparse_linear_attention_mean_amd/libsla.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsla.so")
OBJDIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"
    errs = [ln for ln in res.stderr.splitlines() if ln.strip() and noise not in ln]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    sources = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = min(len(sources), int(os.environ.get("MAX_JOBS", "8")))
    objs = [os.path.join(OBJDIR, s[:-4] + ".o") for s in sources]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s), o) for s, o in zip(sources, objs)]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
