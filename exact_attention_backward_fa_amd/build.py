"""Builds libfa_mi355x.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m exact_attention_backward_fa_amd.build

Objects go to ``_build/`` at the repository root (not tracked); the shared
library lands next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_api.cpp"]
# fa_bwd_inst.hip is compiled once per backward template instance:
# (dtype 0 fp16 / 1 bf16, head dim, causal).
INSTANCES = [(dt, d, c) for dt in (0, 1) for d in (64, 128) for c in (0, 1)]

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # float atomics compile to global_atomic_add_f32 rather than a CAS loop
    "-munsafe-fp-atomics",
    # no packed fp32 math (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa_mi355x.so)")


def _filter_noise(text: str) -> str:
    # The host compiler pass does not know the packed-fp32 target feature and says
    # so once per file; that warning is expected.
    keep = [ln for ln in text.splitlines()
            if "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
    return "\n".join(keep).strip()


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    t0 = time.time()
    jobs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        jobs.append((src, [cc, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]))
    for dt, d, c in INSTANCES:
        obj = os.path.join(BUILD_DIR, f"fa_bwd_inst_{dt}_{d}_{c}.o")
        objs.append(obj)
        jobs.append((f"fa_bwd_inst.hip [{dt},{d},{c}]",
                     [cc, *HIP_FLAGS, f"-DFA_DT={dt}", f"-DFA_D={d}", f"-DFA_CAUSAL={c}", "-c",
                      os.path.join(CSRC, "fa_bwd_inst.hip"), "-o", obj]))
    # the heaviest compilations first, at most one per CPU
    jobs.sort(key=lambda j: "inst" not in j[0])
    width = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    procs = []
    pending = list(jobs)
    failed = []
    results = []
    while pending or procs:
        while pending and len(procs) < width:
            src, cmd = pending.pop(0)
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                text=True)))
        src, p = procs.pop(0)
        out, _ = p.communicate()
        results.append((src, p, out))
    for src, p, out in results:
        msg = _filter_noise(out or "")
        if p.returncode != 0:
            failed.append(src)
            print(f"[build] {src} failed:\n{msg}", file=sys.stderr, flush=True)
        elif msg and verbose:
            print(f"[build] {src}:\n{msg}", flush=True)
    if failed:
        raise RuntimeError(f"HIP compilation failed for {failed}")
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"[build] {LIB_PATH} in {time.time() - t0:.1f}s", flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
