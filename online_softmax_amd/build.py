"""Build libsa_attn.so in-tree for gfx950 with hipcc (and g++ for the host-only unit).

    python -m online_softmax_amd.build [--verbose]

The library lands next to this file; objects go to ``_build/``.  Every call
compiles from scratch so that a stale library is never mistaken for the
current sources.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libsa_attn.so"
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code (the compiler
# would otherwise form them from float2-shaped arithmetic by itself).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
# The backward's unit keeps MFMA results in ordinary vector registers (see
# the header of sa_attn_bwd.hip).
BWD_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libsa_attn")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(str(c) for c in cmd), flush=True)
    res = subprocess.run([str(c) for c in cmd], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(map(str, cmd))}\n"
                           f"{res.stdout}\n{res.stderr}")
    # The host pass does not know the packed-fp32 target feature; drop that note.
    noise = ("packed-fp32-ops", "not a recognized feature")
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> Path:
    hipcc = _hipcc()
    BUILD.mkdir(exist_ok=True)
    for p in BUILD.glob("*.o"):
        p.unlink()
    host_o = BUILD / "host_logic.o"
    steps = [["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", CSRC / "host_logic.cpp", "-o", host_o]]
    objs = []
    # One compilation unit per entry-point file, built in parallel.
    for src in sorted(CSRC.glob("*.hip")):
        obj = BUILD / (src.stem + ".o")
        extra = BWD_FLAGS if src.stem == "sa_attn_bwd" else []
        steps.append([hipcc, *HIP_FLAGS, *extra, "-c", src, "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(len(steps)) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd in steps]:
            f.result()
    tmp = LIB.with_suffix(".so.tmp")
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs, host_o], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
