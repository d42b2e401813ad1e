"""Summaries of rocprofv3 output for the committed profiles.

    python -m exact_attention_backward_fa_amd.profiling trace  <dir> <out.md> "<command>"
    python -m exact_attention_backward_fa_amd.profiling traffic <fetch_dir> <write_dir> <out.txt> "<commands>"
    python -m exact_attention_backward_fa_amd.profiling mfma <dir> <out.txt> "<command>"

``trace`` reads the kernel statistics a ``rocprofv3 --kernel-trace --stats
--output-format csv`` run writes and tabulates per-kernel average durations.

``traffic`` reads two ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs
of ``bench.py --copy-calibration`` and converts the counters (KiB per dispatch) to
HBM bytes per launch of each attention kernel, scaling each counter by what it
reads for the calibration copy of known size (512 MiB read, 512 MiB written).

``mfma`` reads a ``rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 MfmaFlopsF16`` run: the
share of SIMD cycles in which the matrix unit was busy while the GPU was active,
and the MFMA flops each launch executed.

The traffic and MFMA summaries record a hash of the kernel sources so the
benchmark can tell when the counters no longer describe the current kernels.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("csrc/fa_bwd.hip", "csrc/fa_bwd_inst.hip", "csrc/fa_bwd_kernels.hpp",
                  "csrc/fa_bwd_atomic.hpp", "csrc/fa_bwd_common.hpp", "csrc/fa_fwd.hip",
                  "csrc/fa_fwd_inst.hip", "csrc/fa_fwd_kernels.hpp", "csrc/fa_pipeline.hpp",
                  "csrc/fa_common.hpp")
COPY_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(PROFILES, "hbm_traffic_llama_gqa_bf16_8192.txt")
MFMA_FILE = os.path.join(PROFILES, "mfma_busy_llama_gqa_bf16_8192.txt")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = re.sub(r"^void ", "", name)
    name = re.sub(r"\(.*$", "", name)
    return name.replace("fa::", "")


def _find(d: str, pattern: str) -> str:
    hits = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not hits:
        raise FileNotFoundError(f"{pattern} under {d}")
    return hits[0]


def trace_summary(d: str, command: str) -> str:
    path = _find(d, "*kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    out = ["# Kernel trace summary", "", f"Command: `{command}`", "",
           f"kernel_source_sha256_16: {kernel_source_hash()}", "",
           "| kernel | calls | avg (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        avg = float(r["AverageNs"]) / 1e3
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {avg:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.1f}% |")
    return "\n".join(out) + "\n"


def _pmc(d: str, counter: str):
    path = _find(d, "*counter_collection.csv")
    per = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in per.items()}


def traffic_summary(fetch_dir: str, write_dir: str, commands: str) -> str:
    fetch = _pmc(fetch_dir, "FETCH_SIZE")
    write = _pmc(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "copyBuffer" in k or "copy" in k.lower() and "elementwise" not in k]
    if not copy:
        raise RuntimeError("calibration copy kernel not found")
    ck = copy[0]
    f_scale = COPY_BYTES / (fetch[ck] * 1024.0)
    w_scale = COPY_BYTES / (write[ck] * 1024.0)
    out = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
           f"Commands: {commands}", "",
           f"kernel_source_sha256_16: {kernel_source_hash()}", "",
           f"Calibration: `{short_name(ck)}` copying 512 MiB reads FETCH_SIZE = "
           f"{fetch[ck]:.0f} KiB and WRITE_SIZE = {write[ck]:.0f} KiB; scale factors "
           f"fetch x{f_scale:.3f}, write x{w_scale:.3f}.", "",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | written bytes | traffic bytes |",
           "|---|---|---|---|---|---|"]
    for k in fetch:
        if not k.startswith("void fa::"):
            continue
        rb = fetch[k] * 1024.0 * f_scale
        wb = write.get(k, 0.0) * 1024.0 * w_scale
        out.append(f"| `{short_name(k)}` | {fetch[k]:.0f} | {write.get(k, 0.0):.0f} | {rb:.4g} | "
                   f"{wb:.4g} | {rb + wb:.4g} |")
    return "\n".join(out) + "\n"


def mfma_summary(d: str, command: str) -> str:
    util = _pmc(d, "MfmaUtil")
    flops = defaultdict(float)
    for counter in ("MfmaFlopsBF16", "MfmaFlopsF16"):
        for k, v in _pmc(d, counter).items():
            flops[k] += v
    out = ["# MFMA busy share and executed MFMA flops per launch (rocprofv3 --pmc)", "",
           f"Command: {command}", "",
           f"kernel_source_sha256_16: {kernel_source_hash()}", "",
           "MfmaUtil = summed SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMD count) x 100; "
           "MfmaFlops = MFMA MOPs (bf16 + fp16) x 512.", "",
           "| kernel | MfmaUtil % | executed MFMA TFLOP per launch |",
           "|---|---|---|"]
    for k in util:
        if not k.startswith("void fa::"):
            continue
        out.append(f"| `{short_name(k)}` | {util[k]:.1f} | {flops.get(k, 0.0) / 1e12:.4g} |")
    return "\n".join(out) + "\n"


def _read_row(path: str, kernel_prefix: str):
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"kernel_source_sha256_16: (\w+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.split("|")]
        if len(cells) > 3 and cells[1].strip("`").startswith(kernel_prefix):
            return cells[2:-1]
    return None


def read_mfma(kernel_prefix: str):
    """(MFMA busy %, executed MFMA TFLOP per launch) recorded for a kernel, or None
    when the summary is missing or was taken from different kernel sources."""
    cells = _read_row(MFMA_FILE, kernel_prefix)
    return None if cells is None else (float(cells[0]), float(cells[1]))


def read_traffic(kernel_prefix: str):
    """Traffic bytes per launch recorded for a kernel, or None when the summary is
    missing or was taken from different kernel sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"kernel_source_sha256_16: (\w+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.split("|")]
        if len(cells) > 6 and cells[1].strip("`").startswith(kernel_prefix):
            return float(cells[6])
    return None


def main(argv) -> int:
    if argv[1] == "trace":
        _, _, d, out, cmd = argv
        text = trace_summary(d, cmd)
    elif argv[1] == "traffic":
        _, _, fd, wd, out, cmd = argv
        text = traffic_summary(fd, wd, cmd)
    elif argv[1] == "mfma":
        _, _, d, out, cmd = argv
        text = mfma_summary(d, cmd)
    else:
        raise SystemExit(__doc__)
    with open(out, "w") as f:
        f.write(text)
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
