"""CPU check of the kernels' assembly for the inline-MFMA hazards the compiler
does not track (see tests/asm_check.py).  Every shipped template instance of the
forward, dK/dV, dQ-pass and fused atomic kernels is compiled to gfx950 assembly
(no GPU needed; the build caches the assembly under the units' source hash)."""
import pytest

from exact_attention_backward_fa_amd import build as fabuild
from tests import asm_check

# kernel units whose assembly is scanned: every instance of every kernel family
# that issues inline-assembly MFMAs
KINDS = ("fwd", "dkdv", "dq", "atomic")
KERNELS = ("fwd_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel", "bwd_dkdv_atomic_kernel")


def _have_hipcc():
    try:
        fabuild.hipcc()
        return True
    except RuntimeError:
        return False


def _scanned_units():
    return [u for u in fabuild.units() if u.name.split("_")[0] in KINDS]


@pytest.fixture(scope="module")
def assembly():
    if not _have_hipcc():
        pytest.skip("hipcc not available")
    paths = fabuild.device_asm(_scanned_units())
    texts = {}
    for name, path in paths.items():
        with open(path) as f:
            texts[name] = f.read()
    return texts


def _kernels(texts):
    for name, text in texts.items():
        for sym, ins in asm_check.kernel_bodies(text).items():
            if any(k in sym for k in KERNELS):
                yield f"{name}:{sym}", ins


def _expected_kernels(unit):
    """Kernels a unit instantiates: one, or two for a dQ pass with a dBias (feature
    sets 1 and 2: 2-byte and 8-byte dBias stores) and for a forward without bias
    (plain or feature set 4, dropout alone: its fast pass and the rerun of the
    items that pass marks)."""
    if unit.name.startswith("dq_") and unit.name.endswith(("_f1", "_f2")):
        return 2
    if unit.name.startswith("fwd_") and ("_f" not in unit.name or unit.name.endswith("_f4")):
        return 2
    return 1


def test_kernels_found(assembly):
    found = [s for s, _ in _kernels(assembly)]
    assert len(found) == sum(_expected_kernels(u) for u in _scanned_units()), found


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
