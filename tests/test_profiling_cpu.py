"""Host logic of the measurement: a counter summary the benchmark reads is trusted
for a kernel only while the device-code hash it recorded for that kernel matches
the hash of the code built now, and the benchmark refuses more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

from exact_attention_backward_fa_amd import build, profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = "bwd_dkdv_kernel<1, 128, true, 0>"


@pytest.fixture
def code_hashes(tmp_path, monkeypatch):
    """A built-code hash file holding hash H for the bf16 d=128 causal dK/dV unit."""
    p = tmp_path / "kernel_code.json"
    p.write_text(json.dumps({"dkdv_1_128_1": "feedfacecafe0123"}))
    monkeypatch.setattr(build, "CODE_HASHES", str(p))
    return "feedfacecafe0123"


def _summary(tmp_path, name, hash_value, row):
    p = tmp_path / name
    code = f"code_sha256_16 `{KERNEL}`: {hash_value}\n\n" if hash_value else ""
    p.write_text(f"# summary\n\n{code}| kernel | a | b |\n|---|---|---|\n{row}\n")
    return str(p)


def test_mfma_summary_read_when_code_hash_matches(tmp_path, monkeypatch, code_hashes):
    path = _summary(tmp_path, "m.txt", code_hashes, f"| `{KERNEL}` | 67.9 | 4.436 |")
    monkeypatch.setattr(profiling, "MFMA_FILE", path)
    assert profiling.read_mfma("bwd_dkdv_kernel<1, 128, true") == (67.9, 4.436)
    assert profiling.read_mfma("bwd_dq_kernel") is None


def test_stale_or_missing_summaries_read_as_none(tmp_path, monkeypatch, code_hashes):
    path = _summary(tmp_path, "m.txt", "0000000000000000", f"| `{KERNEL}` | 67.9 | 4.436 |")
    monkeypatch.setattr(profiling, "MFMA_FILE", path)
    assert profiling.read_mfma(KERNEL) is None
    path = _summary(tmp_path, "n.txt", None, f"| `{KERNEL}` | 67.9 | 4.436 |")
    monkeypatch.setattr(profiling, "MFMA_FILE", path)
    assert profiling.read_mfma(KERNEL) is None
    monkeypatch.setattr(profiling, "MFMA_FILE", str(tmp_path / "absent.txt"))
    assert profiling.read_mfma(KERNEL) is None
    monkeypatch.setattr(profiling, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    monkeypatch.setattr(profiling, "TRAFFIC_FILE_ATOMIC", str(tmp_path / "absent.txt"))
    assert profiling.read_traffic(KERNEL) is None
    # no hash recorded by the build for the kernel: nothing is trusted
    monkeypatch.setattr(build, "CODE_HASHES", str(tmp_path / "absent.json"))
    path = _summary(tmp_path, "o.txt", code_hashes, f"| `{KERNEL}` | 67.9 | 4.436 |")
    monkeypatch.setattr(profiling, "MFMA_FILE", path)
    assert profiling.read_mfma(KERNEL) is None


def test_traffic_summary_read_when_code_hash_matches(tmp_path, monkeypatch, code_hashes):
    row = f"| `{KERNEL}` | 2142380 | 142889 | 4.387e+09 | 1.463e+08 | 4.533e+09 |"
    p = tmp_path / "t.txt"
    p.write_text(f"code_sha256_16 `{KERNEL}`: {code_hashes}\n\n{row}\n")
    monkeypatch.setattr(profiling, "TRAFFIC_FILE", str(p))
    assert profiling.read_traffic(KERNEL) == pytest.approx(4.533e9)


ASM = """\t.text
\t.file\t"fa_bwd_inst.hip"
kernel:                                 ; @kernel
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3] ; comment
\ts_endpgm
\t.globl\t__hip_cuid_0123456789abcdef
__hip_cuid_0123456789abcdef:
\t.ident\t"AMD clang version X"
"""


def test_code_hash_ignores_comments_tool_notes_and_unit_id(tmp_path):
    a = tmp_path / "a.s"
    a.write_text(ASM)
    b = tmp_path / "b.s"
    b.write_text(ASM.replace("; comment", "; other").replace("0123456789abcdef", "fedcba9876543210")
                 .replace("version X", "version Y").replace("fa_bwd_inst.hip", "elsewhere.hip"))
    c = tmp_path / "c.s"
    c.write_text(ASM.replace("a[0:3], v[0:3]", "a[0:3], v[8:11]"))
    assert build.asm_code_hash(str(a)) == build.asm_code_hash(str(b))
    assert build.asm_code_hash(str(a)) != build.asm_code_hash(str(c))


def test_unit_of_kernel():
    assert build.unit_of_kernel("bwd_dkdv_kernel<1, 128, true, 0>") == "dkdv_1_128_1"
    assert build.unit_of_kernel("fa::bwd_dq_kernel<0, 64, false, 2>") == "dq_0_64_0_f2"
    assert build.unit_of_kernel("fwd_kernel<1, 128, true, 1>") == "fwd_1_128_1_f1"
    assert build.unit_of_kernel("fwd_kernel<1, 128, true, 0, 1>") == "fwd_1_128_1"
    assert build.unit_of_kernel("bwd_dkdv_atomic_kernel<1, 128, true>") == "atomic_1_128_1"
    assert build.unit_of_kernel("bwd_pre_kernel<1, 128>") == "pre_1_128_1"
    assert build.unit_of_kernel("bwd_dq_kernel<1, 128, true, 1, true>") == "dq_1_128_1_f1"
    assert build.unit_of_kernel("dq_convert_kernel<1>") is None
    names = {u.name for u in build.units()}
    assert set(build.PROFILED_UNITS) <= names


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "--gpus 1" in r.stderr
