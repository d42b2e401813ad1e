"""Summaries of rocprofv3 output for the committed profiles.

    python -m exact_attention_backward_fa_amd.profiling trace  <dir> <out.md> "<command>"
    python -m exact_attention_backward_fa_amd.profiling traffic <fetch_dir> <write_dir> <out.txt> "<commands>"
    python -m exact_attention_backward_fa_amd.profiling mfma <dir> <out.txt> "<command>"
    python -m exact_attention_backward_fa_amd.profiling workloads <lines.jsonl> <out.md> "<command>"

``trace`` reads the kernel statistics a ``rocprofv3 --kernel-trace --stats
--output-format csv`` run writes and tabulates per-kernel average durations.

``traffic`` reads two ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs
of ``bench.py --copy-calibration`` and converts the counters (KiB per dispatch) to
HBM bytes per launch of each attention kernel, scaling each counter by what it
reads for the calibration copy of known size (512 MiB read, 512 MiB written).

``mfma`` reads a ``rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 MfmaFlopsF16`` run: the
share of SIMD cycles in which the matrix unit was busy while the GPU was active,
and the MFMA flops each launch executed.

Every summary records, per kernel, a hash of the kernel's generated device code
(written by the build next to the library), so the benchmark can tell when the
counters no longer describe the kernels built: a change elsewhere in the sources
that leaves a kernel's instructions alone keeps its profile valid.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(PROFILES, "hbm_traffic_llama_gqa_bf16_8192.txt")
# the fused atomic-dQ path's counters, taken in a run of their own
TRAFFIC_FILE_ATOMIC = os.path.join(PROFILES, "hbm_traffic_atomic_dq_llama_gqa_bf16_8192.txt")
MFMA_FILE = os.path.join(PROFILES, "mfma_busy_llama_gqa_bf16_8192.txt")


def kernel_code_hash(kernel: str):
    """Hash of the device code built for a kernel (short name), or None when the
    build recorded none for it."""
    from . import build
    unit = build.unit_of_kernel(kernel)
    try:
        with open(build.CODE_HASHES) as f:
            return json.load(f).get(unit) if unit else None
    except (OSError, ValueError):
        return None


def _code_lines(kernels) -> list:
    out = []
    for k in kernels:
        h = kernel_code_hash(short_name(k))
        if h:
            out.append(f"code_sha256_16 `{short_name(k)}`: {h}")
    return out + [""] if out else []


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
           *_code_lines(r["Name"] for r in rows),
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
           *_code_lines(fetch),
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
           *_code_lines(util),
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
    """Cells of the row of the first kernel whose name starts with kernel_prefix,
    or None when the file or the row is missing, or the code hash it recorded for
    that kernel is not the hash of the kernel built now."""
    try:
        text = open(path).read()
    except OSError:
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.split("|")]
        if len(cells) > 3 and cells[1].strip("`").startswith(kernel_prefix):
            name = cells[1].strip("`")
            m = re.search(r"code_sha256_16 `" + re.escape(name) + r"`: (\w+)", text)
            now = kernel_code_hash(name)
            if not m or now is None or m.group(1) != now:
                return None
            return cells[2:-1]
    return None


def read_mfma(kernel_prefix: str):
    """(MFMA busy %, executed MFMA TFLOP per launch) recorded for a kernel, or None
    when the summary is missing or was taken from different kernel sources."""
    cells = _read_row(MFMA_FILE, kernel_prefix)
    return None if cells is None else (float(cells[0]), float(cells[1]))


def read_traffic(kernel_prefix: str):
    """Traffic bytes per launch recorded for a kernel, or None when the summary is
    missing or was taken from different kernel code."""
    for path in (TRAFFIC_FILE, TRAFFIC_FILE_ATOMIC):
        cells = _read_row(path, kernel_prefix)
        if cells is not None and len(cells) >= 5:
            return float(cells[4])
    return None


def workloads_summary(jsonl: str, command: str) -> str:
    """A table of the benchmark's JSON lines (one per workload)."""
    out = ["# fa_bwd throughput per workload (bench.py JSON lines)", "",
           f"Command: `{command}`", "",
           "TFLOP/s counts 2.5x the forward's 4*N_q*N_kv*d flops per query head, halved "
           "for causal; % is of the 2516.6 TFLOP/s dense bf16/fp16 MFMA peak.", "",
           "| workload | dQ path | fwd ms | bwd ms | bwd TFLOP/s | % of peak | dK/dV kernel ms | "
           "dK/dV TFLOP/s |",
           "|---|---|---|---|---|---|---|---|"]
    for line in open(jsonl):
        line = line.strip()
        if not line.startswith("{"):
            continue
        r = json.loads(line)
        rf = r.get("roofline") or {}
        km = rf.get("kernel_ms")
        ach = rf.get("achieved")
        out.append(f"| {r['config']['workload']} | {r['config'].get('dq_path')} | {r['fwd_ms']:.4g} | "
                   f"{r['bwd_ms']:.4g} | {r['value']:.1f} | {r['pct_of_peak']:.1f} | "
                   f"{'-' if km is None else f'{km:.4g}'} | {'-' if ach is None else f'{ach:.1f}'} |")
    return "\n".join(out) + "\n"


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
    elif argv[1] == "workloads":
        _, _, jsonl, out, cmd = argv
        text = workloads_summary(jsonl, cmd)
    else:
        raise SystemExit(__doc__)
    with open(out, "w") as f:
        f.write(text)
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
