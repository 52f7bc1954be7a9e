"""Build libcoospmm.so (HIP, gfx950) in-tree with hipcc.

    python -m coo_spmm_fwd_amd.build        # or __graft_entry__.build()

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection switched off (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcoospmm.so")
SOURCES = ["layer.hip", "build.hip", "sort.hip", "spmm.hip", "restructure.hip", "occupancy.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the coospmm HIP library cannot be built")


def flags() -> list[str]:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fno-gpu-rdc"]


def build(verbose: bool = False, jobs: int = 6) -> str:
    """Compile each source to an object (in parallel), then link the shared library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _wait(procs)
            procs = []
    _wait(procs)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _wait(procs):
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())
        if p.returncode != 0:
            failed.append((src, out))
        elif text:
            sys.stderr.write(text + "\n")
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
