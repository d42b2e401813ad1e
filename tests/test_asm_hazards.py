"""CPU check of the kernels' assembly for the inline-MFMA hazards the compiler
does not track (see tests/asm_check.py).  Compiles two template instances of the
backward and the forward kernels to gfx950 assembly (no GPU needed)."""
import os
import shutil
import subprocess
import tempfile

import pytest

from exact_attention_backward_fa_amd import build as fabuild
from tests import asm_check

# (dtype 0 fp16 / 1 bf16, head dim, causal): the headline instance and the other
# extreme of the template parameters
INSTANCES = [(1, 128, 1), (0, 64, 0)]
KERNELS = ("bwd_dkdv_kernel", "bwd_dq_kernel")
FWD_INSTANCES = [(1, 128, 1), (0, 64, 0)]


def _have_hipcc():
    try:
        fabuild.hipcc()
        return True
    except RuntimeError:
        return False


@pytest.fixture(scope="module")
def assembly():
    if not _have_hipcc():
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="fa_asm_")
    try:
        procs = []
        for dt, d, c in INSTANCES:
            out = os.path.join(tmp, f"inst_{dt}_{d}_{c}.s")
            cmd = [fabuild.hipcc(), *[f for f in fabuild.HIP_FLAGS if f != "-fPIC"],
                   f"-DFA_DT={dt}", f"-DFA_D={d}", f"-DFA_CAUSAL={c}", "--cuda-device-only", "-S",
                   os.path.join(fabuild.CSRC, "fa_bwd_inst.hip"), "-o", out]
            procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                text=True)))
        for dt, d, c in FWD_INSTANCES:
            src = os.path.join(tmp, f"fwd_{dt}_{d}_{c}.hip")
            with open(src, "w") as f:
                f.write('#include "fa_fwd_kernels.hpp"\n'
                        f"template __global__ void fa::fwd_kernel<{dt}, {d}, {'true' if c else 'false'}>"
                        "(fa::FwdParams);\n")
            out = src[:-4] + ".s"
            cmd = [fabuild.hipcc(), *[f for f in fabuild.HIP_FLAGS if f != "-fPIC"], "-I", fabuild.CSRC,
                   "--cuda-device-only", "-S", src, "-o", out]
            procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                text=True)))
        texts = {}
        for out, p in procs:
            log, _ = p.communicate(timeout=900)
            assert p.returncode == 0, log[-2000:]
            with open(out) as f:
                texts[os.path.basename(out)] = f.read()
        return texts
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _kernels(texts):
    for name, text in texts.items():
        for sym, ins in asm_check.kernel_bodies(text).items():
            if any(k in sym for k in KERNELS) or "fwd_kernel" in sym:
                yield f"{name}:{sym}", ins


def test_kernels_found(assembly):
    found = [s for s, _ in _kernels(assembly)]
    assert len(found) == len(INSTANCES) * len(KERNELS) + len(FWD_INSTANCES), found


def test_no_valu_write_right_before_inline_mfma(assembly):
    for sym, ins in _kernels(assembly):
        bad = asm_check.valu_to_mfma_hazards(ins)
        assert not bad, f"{sym}: {len(bad)} MFMA sources written just before, e.g. {bad[:3]}"


def test_no_early_read_of_inline_mfma_results(assembly):
    for sym, ins in _kernels(assembly):
        bad = asm_check.early_result_reads(ins)
        assert not bad, f"{sym}: {len(bad)} reads of an MFMA result too soon, e.g. {bad[:3]}"


def test_checker_catches_planted_hazards():
    """The scans flag the two patterns they exist for (planted in text)."""
    text = """
_Zplanted:
\tv_mov_b32_e32 v3, 0
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
\t;;#ASMEND
\tv_accvgpr_read_b32 v8, a2
\tv_add_f32_e32 v9, v8, v8
\t;;#ASMSTART
\tv_mfma_f32_16x16x32_bf16 v[20:23], v[0:3], v[4:7], 0
\t;;#ASMEND
\tv_add_f32_e32 v30, v21, v21
.Lfunc_end0:
"""
    ins = asm_check.kernel_bodies(text)["_Zplanted"]
    assert len(asm_check.valu_to_mfma_hazards(ins)) == 1  # v3 written, then read as A
    reads = asm_check.early_result_reads(ins)
    assert any("v_accvgpr_read_b32 v8, a2" in r for r in reads)
    assert any("v30" in r for r in reads)
    # with the wait states in place neither pattern is reported
    safe = text.replace("\tv_mov_b32_e32 v3, 0\n", "\tv_mov_b32_e32 v3, 0\n\ts_nop 1\n").replace(
        "\t;;#ASMEND\n\tv_accvgpr_read", "\t;;#ASMEND\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\tv_accvgpr_read").replace(
        "\t;;#ASMEND\n\tv_add_f32_e32 v30", "\t;;#ASMEND\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\tv_add_f32_e32 v30")
    ins = asm_check.kernel_bodies(safe)["_Zplanted"]
    assert asm_check.valu_to_mfma_hazards(ins) == []
    assert asm_check.early_result_reads(ins) == []
