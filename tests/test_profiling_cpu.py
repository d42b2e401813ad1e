"""Host logic of the measurement: the counter summaries the benchmark reads are
trusted only while their recorded source hash matches the kernel sources, and
the benchmark refuses more than one GPU."""
import os
import subprocess
import sys

import pytest

from exact_attention_backward_fa_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = "bwd_dkdv_kernel<1, 128, true>"


def _summary(tmp_path, name, hash_value, row):
    p = tmp_path / name
    p.write_text(f"# summary\n\nkernel_source_sha256_16: {hash_value}\n\n| kernel | a | b |\n"
                 f"|---|---|---|\n{row}\n")
    return str(p)


def test_mfma_summary_read_when_hash_matches(tmp_path, monkeypatch):
    path = _summary(tmp_path, "m.txt", profiling.kernel_source_hash(), f"| `{KERNEL}` | 67.9 | 4.436 |")
    monkeypatch.setattr(profiling, "MFMA_FILE", path)
    assert profiling.read_mfma(KERNEL) == (67.9, 4.436)
    assert profiling.read_mfma("bwd_dq_kernel") is None


def test_stale_or_missing_summaries_read_as_none(tmp_path, monkeypatch):
    path = _summary(tmp_path, "m.txt", "0000000000000000", f"| `{KERNEL}` | 67.9 | 4.436 |")
    monkeypatch.setattr(profiling, "MFMA_FILE", path)
    assert profiling.read_mfma(KERNEL) is None
    monkeypatch.setattr(profiling, "MFMA_FILE", str(tmp_path / "absent.txt"))
    assert profiling.read_mfma(KERNEL) is None
    monkeypatch.setattr(profiling, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert profiling.read_traffic(KERNEL) is None


def test_traffic_summary_read_when_hash_matches(tmp_path, monkeypatch):
    row = f"| `{KERNEL}` | 2142380 | 142889 | 4.387e+09 | 1.463e+08 | 4.533e+09 |"
    p = tmp_path / "t.txt"
    p.write_text(f"kernel_source_sha256_16: {profiling.kernel_source_hash()}\n\n{row}\n")
    monkeypatch.setattr(profiling, "TRAFFIC_FILE", str(p))
    assert profiling.read_traffic(KERNEL) == pytest.approx(4.533e9)


def test_hash_changes_with_kernel_sources(tmp_path, monkeypatch):
    before = profiling.kernel_source_hash()
    pkg = tmp_path / "pkg"
    (pkg / "csrc").mkdir(parents=True)
    for rel in profiling.KERNEL_SOURCES:
        src = os.path.join(profiling.PKG, rel)
        (pkg / rel).write_bytes(open(src, "rb").read())
    monkeypatch.setattr(profiling, "PKG", str(pkg))
    assert profiling.kernel_source_hash() == before
    with open(pkg / profiling.KERNEL_SOURCES[-1], "ab") as f:
        f.write(b"\n")
    assert profiling.kernel_source_hash() != before


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "--gpus 1" in r.stderr
