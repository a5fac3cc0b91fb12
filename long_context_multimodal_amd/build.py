"""Build ``libmmsp.so`` (all HIP sources of ``csrc/``) for gfx950 with hipcc,
and ``mmsp_ring_step``, a native program that calls only its C-ABI.

Usage: ``python -m long_context_multimodal_amd.build`` (or ``build()``).  The
library lands next to this file; objects go to ``_build/`` at the repo root.
Always recompiles: sources are few and each takes seconds.
"""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmmsp.so")
# a native caller of the C-ABI (no Python): one rank's training step from a file
TOOL_SRC = os.path.join(PKG, "ring_step.cpp")
TOOL = os.path.join(PKG, "mmsp_ring_step")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(args):
    hipcc, src, obj = args
    cmd = [hipcc, *HIPCC_FLAGS, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return err


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
        jobs.append((hipcc, src, obj))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for (_, src, _), warn in zip(jobs, ex.map(_compile, jobs)):
            if verbose and warn.strip():
                print(f"[{os.path.basename(src)}]\n{warn}")
    tmp = OUT + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[j[2] for j in jobs]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    tmp = TOOL + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, TOOL_SRC, "-L", PKG, "-lmmsp", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {os.path.basename(TOOL)} failed:\n{r.stderr}")
    os.replace(tmp, TOOL)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
