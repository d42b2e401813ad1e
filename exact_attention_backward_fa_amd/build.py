"""Builds libfa_mi355x.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m exact_attention_backward_fa_amd.build [--incremental]

Every kernel template instance is its own compilation unit, so the units build in
parallel: the forward once per (dtype, head dim, causal, feature set), the backward
once per (dtype, head dim, causal, feature set, kernel).  Objects go to ``_build/`` at the repository
root (not tracked); the shared library lands next to this file, where the binding
loads it.  ``build()`` compiles every unit each time it is called;
``build(incremental=True)`` reuses an object whose source, included headers and
flags are unchanged (the key is a hash over all of them).
"""
from __future__ import annotations

import hashlib
import json
import os
import re
import shutil
import subprocess
import sys
import time
from typing import Dict, List, Optional, Sequence, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

# Host-side sources (entry points, dispatch, conversions).
SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_api.cpp", "fa_noalloc.hip"]
# Template instances: (dtype 0 fp16 / 1 bf16, head dim, causal).
HEAD_DIMS = (32, 64, 96, 128, 160, 192, 224, 256)
INSTANCES = [(dt, d, c) for dt in (0, 1) for d in HEAD_DIMS for c in (0, 1)]
# The fused atomic dK/dV/dQ kernel is built for these head dims only.
ATOMIC_HEAD_DIMS = (64, 128)
# Feature sets (1: additive score bias and its gradient, 2: bias and dropout of P,
# 3: a per-(batch, key) bias without gradient, 4: dropout without bias) are built
# for these head dims, and set 3 for every head dim; every head dim has the plain
# set 0.
FEATURE_HEAD_DIMS = (64, 128)
FEATURES = (1, 2, 3, 4)
ALL_DIM_FEATURES = (3,)
# Backward kernel families compiled per instance (FA_KIND in fa_bwd_inst.hip).
BWD_KINDS = {0: "pre", 1: "dkdv", 2: "dq", 3: "atomic"}

# Units whose kernels the committed counter profiles describe (the bf16, d = 128,
# causal instance).  After linking, build() hashes their device assembly into
# CODE_HASHES, so a profile can tell whether it still describes the kernels built.
PROFILED_UNITS = ("fwd_1_128_1", "pre_1_128_1", "dkdv_1_128_1", "dq_1_128_1", "atomic_1_128_1")
CODE_HASHES = os.path.join(PKG_DIR, "kernel_code.json")

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


class Unit:
    """One compilation: a source file plus -D defines."""

    def __init__(self, name: str, src: str, defines: Sequence[Tuple[str, int]] = ()):
        self.name = name
        self.src = src
        self.defines = list(defines)

    def flags(self) -> List[str]:
        return [f"-D{k}={v}" for k, v in self.defines]


def units() -> List[Unit]:
    out = [Unit(os.path.splitext(s)[0], s) for s in SOURCES]
    for dt, d, c in INSTANCES:
        fts = (0,) + tuple(ft for ft in FEATURES if d in FEATURE_HEAD_DIMS or ft in ALL_DIM_FEATURES)
        for ft in fts:
            sfx = f"{dt}_{d}_{c}" + (f"_f{ft}" if ft else "")
            out.append(Unit(f"fwd_{sfx}", "fa_fwd_inst.hip",
                            [("FA_DT", dt), ("FA_D", d), ("FA_CAUSAL", c), ("FA_FT", ft)]))
            for kind, kname in BWD_KINDS.items():
                if kname == "atomic" and (d not in ATOMIC_HEAD_DIMS or ft):
                    continue
                # the row preprocess kernel serves the atomic path only
                if kname == "pre" and (ft or d not in ATOMIC_HEAD_DIMS):
                    continue
                out.append(Unit(f"{kname}_{sfx}", "fa_bwd_inst.hip",
                                [("FA_DT", dt), ("FA_D", d), ("FA_CAUSAL", c), ("FA_FT", ft),
                                 ("FA_KIND", kind)]))
    return out


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa_mi355x.so)")


_INC = re.compile(r'^\s*#\s*include\s+"([^"]+)"', re.M)


def _deps(path: str, seen: Dict[str, None]) -> None:
    if path in seen:
        return
    seen[path] = None
    with open(path) as f:
        text = f.read()
    for inc in _INC.findall(text):
        for base in (os.path.dirname(path), CSRC, INCLUDE):
            cand = os.path.join(base, inc)
            if os.path.exists(cand):
                _deps(os.path.abspath(cand), seen)
                break


def unit_key(u: Unit, extra: Sequence[str] = ()) -> str:
    """Hash of the unit's source, every header it includes (transitively) and the
    compile flags."""
    seen: Dict[str, None] = {}
    _deps(os.path.join(CSRC, u.src), seen)
    h = hashlib.sha256()
    for path in sorted(seen):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(HIP_FLAGS + u.flags() + list(extra)).encode())
    return h.hexdigest()[:16]


def _filter_noise(text: str) -> str:
    # The host compiler pass does not know the packed-fp32 target feature and says
    # so once per file; that warning is expected.
    keep = [ln for ln in text.splitlines()
            if "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
    return "\n".join(keep).strip()


def _run_jobs(jobs: List[Tuple[str, List[str]]], verbose: bool) -> None:
    """Run compile commands in parallel (at most one per CPU, 16 at most).  Each
    job writes its output to a file of its own, read once the job has ended (a pipe
    read only then would block a job whose output outgrows the pipe's buffer)."""
    width = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    logs = os.path.join(BUILD_DIR, "logs")
    os.makedirs(logs, exist_ok=True)
    pending = list(jobs)
    running = []
    failed = []
    while pending or running:
        while pending and len(running) < width:
            name, cmd = pending.pop(0)
            if verbose:
                print(" ".join(cmd), flush=True)
            log = os.path.join(logs, f"{name}.log")
            with open(log, "w") as f:
                running.append((name, subprocess.Popen(cmd, stdout=f, stderr=subprocess.STDOUT), log))
        # wait for whichever job ends first
        while True:
            done = [r for r in running if r[1].poll() is not None]
            if done:
                break
            time.sleep(0.05)
        for name, p, log in done:
            running.remove((name, p, log))
            with open(log, errors="replace") as f:
                out = f.read()
            msg = _filter_noise(out or "")
            if p.returncode != 0:
                failed.append(name)
                print(f"[build] {name} failed:\n{msg}", file=sys.stderr, flush=True)
            elif msg and verbose:
                print(f"[build] {name}:\n{msg}", flush=True)
    if failed:
        raise RuntimeError(f"HIP compilation failed for {failed}")


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every unit and link the shared library; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    t0 = time.time()
    jobs = []
    objs = []
    done = []  # (unit, object path, scratch directory) of the units compiled now
    for u in units():
        obj = os.path.join(BUILD_DIR, f"{u.name}-{unit_key(u)}.o")
        objs.append(obj)
        if incremental and os.path.exists(obj):
            continue
        # each unit compiles in a scratch directory of its own, keeping the compiler's
        # intermediate files: its device assembly goes to the assembly cache, so the
        # hazard scan of the tests needs no second compilation
        work = os.path.join(BUILD_DIR, "tmp", u.name)
        shutil.rmtree(work, ignore_errors=True)
        os.makedirs(work)
        done.append((u, obj, work))
        jobs.append((u.name, [cc, *HIP_FLAGS, *u.flags(), "-save-temps=obj", "-c",
                              os.path.join(CSRC, u.src), "-o", os.path.join(work, "unit.o")]))
    # the kernel instances are the long compilations: start them first
    jobs.sort(key=lambda j: j[0] in [os.path.splitext(s)[0] for s in SOURCES])
    _run_jobs(jobs, verbose)
    adir = os.path.join(BUILD_DIR, "asm")
    os.makedirs(adir, exist_ok=True)
    for u, obj, work in done:
        os.replace(os.path.join(work, "unit.o"), obj)
        dev = [f for f in os.listdir(work) if f.endswith(f"-hip-amdgcn-amd-amdhsa-{ARCH}.s")]
        if dev:
            os.replace(os.path.join(work, dev[0]), os.path.join(adir, f"{u.name}-{unit_key(u, ['asm'])}.s"))
        shutil.rmtree(work, ignore_errors=True)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB_PATH)
    write_code_hashes(verbose)
    if verbose:
        print(f"[build] {LIB_PATH} ({len(jobs)} of {len(objs)} units compiled) in "
              f"{time.time() - t0:.1f}s", flush=True)
    return LIB_PATH


def device_asm(selected: Sequence[Unit], verbose: bool = False) -> Dict[str, str]:
    """gfx950 assembly of the given units (device code only), cached in
    ``_build/asm`` under the unit key; returns {unit name: path of the .s file}."""
    cc = hipcc()
    adir = os.path.join(BUILD_DIR, "asm")
    os.makedirs(adir, exist_ok=True)
    paths = {}
    jobs = []
    for u in selected:
        path = os.path.join(adir, f"{u.name}-{unit_key(u, ['asm'])}.s")
        paths[u.name] = path
        if not os.path.exists(path):
            flags = [f for f in HIP_FLAGS if f != "-fPIC"]
            jobs.append((u.name, [cc, *flags, *u.flags(), "--cuda-device-only", "-S",
                                  os.path.join(CSRC, u.src), "-o", path + ".part"]))
    _run_jobs(jobs, verbose)
    for path in paths.values():
        if os.path.exists(path + ".part"):
            os.replace(path + ".part", path)
    return paths


def asm_code_hash(path: str) -> str:
    """Hash of a unit's device assembly with comments, file/tool notes and the
    per-compilation unit id removed: equal for two builds that generate the same
    instructions and metadata."""
    h = hashlib.sha256()
    with open(path) as f:
        for line in f:
            line = line.split(";", 1)[0].rstrip()
            if not line or line.lstrip().startswith((".file", ".ident")):
                continue
            line = re.sub(r"__hip_cuid_[0-9a-f]+", "__hip_cuid", line)
            h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def write_code_hashes(verbose: bool = False) -> Dict[str, str]:
    """Hashes the device code of PROFILED_UNITS into CODE_HASHES ({unit: hash})."""
    sel = [u for u in units() if u.name in PROFILED_UNITS]
    paths = device_asm(sel, verbose)
    hashes = {name: asm_code_hash(path) for name, path in sorted(paths.items())}
    tmp = CODE_HASHES + ".tmp"
    with open(tmp, "w") as f:
        json.dump(hashes, f, indent=1, sort_keys=True)
    os.replace(tmp, CODE_HASHES)
    return hashes


_KERNEL_UNIT = {"fwd_kernel": "fwd", "bwd_pre_kernel": "pre", "bwd_dkdv_kernel": "dkdv",
                "bwd_dq_kernel": "dq", "bwd_dkdv_atomic_kernel": "atomic"}


def unit_of_kernel(kernel: str) -> Optional[str]:
    """Compilation unit of a kernel named as a profiler prints it, e.g.
    ``bwd_dkdv_kernel<1, 128, true, 0>`` -> ``dkdv_1_128_1``; None for others."""
    m = re.match(r"(?:fa::)?(\w+)<(\d+), (\d+)(?:, (true|false))?(?:, (\d+))?(?:, (?:true|false|\d+))?>",
                 kernel)
    if not m or m.group(1) not in _KERNEL_UNIT:
        return None
    fam = _KERNEL_UNIT[m.group(1)]
    # the preprocess takes no causal flag: the causal unit holds it as well
    causal = "1" if fam == "pre" or m.group(4) == "true" else "0"
    ft = int(m.group(5) or 0)
    return f"{fam}_{m.group(2)}_{m.group(3)}_{causal}" + (f"_f{ft}" if ft else "")


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv[1:])
