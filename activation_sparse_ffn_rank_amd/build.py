"""Build the gfx950 shared library libpi.so in-tree with hipcc.

All HIP code is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass warns that it does
not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpi.so")
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "pi_abi.hip"), os.path.join(CSRC, "pi_persist_b.hip"), os.path.join(CSRC, "pi_split.hip")]
HOST_SOURCES = [os.path.join(CSRC, "pi_cold.cpp"),   # host half of the hybrid split (g++, OpenMP)
                os.path.join(CSRC, "pi_place.cpp"),  # offline placement under a memory budget
                os.path.join(CSRC, "pi_ranks.cpp")]  # per-layer predictor rank under a memory budget
DEPENDS = SOURCES + HOST_SOURCES + [os.path.join(CSRC, n) for n in ("pi_kernels.hpp", "pi_sync.hpp", "pi_occupancy.hpp", "pi_tail.hpp", "pi_split.hpp", "pi_wide.hpp")] + [
                     os.path.join(ROOT, "include", "pi_sparse_ffn.h")]
OBJDIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
NOISE = "is not a recognized feature for this target"


CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-mavx2", "-mfma", "-mf16c", "-fopenmp"]
HOST_OBJS = [os.path.join(OBJDIR, os.path.basename(p).replace(".cpp", ".o")) for p in HOST_SOURCES]


def _units():
    """(source, object, extra flags): the ABI unit, one tail-kernel unit per batch width, the split
    sparse-FFN unit."""
    units = [(SOURCES[0], os.path.join(OBJDIR, "pi_abi.o"), [])]
    for b in range(1, 9):
        units.append((SOURCES[1], os.path.join(OBJDIR, f"pi_persist_b{b}.o"), [f"-DPIK_B={b}"]))
    units.append((SOURCES[2], os.path.join(OBJDIR, "pi_split.o"), []))
    return units


def _gomp() -> str:
    """libgomp of the host compiler (the OpenMP runtime torch loads too)."""
    out = subprocess.run([CXX, "-print-file-name=libgomp.so"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) else "-lgomp"


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if NOISE not in l)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every unit (in parallel) and link libpi.so; always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    pending = [[HIPCC, *FLAGS, *inc, *extra, "-c", src, "-o", obj] for src, obj, extra in _units()]
    for src, obj in zip(HOST_SOURCES, HOST_OBJS):
        pending.append([CXX, *HOST_FLAGS, *inc, "-c", src, "-o", obj])
    running = []
    while pending or running:
        while pending and len(running) < jobs:
            cmd = pending.pop(0)
            if verbose:
                print(" ".join(cmd), flush=True)
            running.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        cmd, proc = running.pop(0)
        out, err = proc.communicate()
        if proc.returncode != 0:
            for _, p in running:
                p.wait()
            raise RuntimeError(f"{cmd[0]} failed ({proc.returncode}) on {cmd[-3]}:\n{_clean(err)}")
    tmp = LIB + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp] + [obj for _, obj, _ in _units()] + [
        *HOST_OBJS, _gomp()]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{_clean(res.stderr)}")
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPENDS)


if __name__ == "__main__":
    print(build(verbose=True))
