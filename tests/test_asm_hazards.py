"""The kernels' gfx950 assembly holds no load that overwrites an operand of an
MFMA still in flight, and no MFMA that accumulates onto the result of an MFMA
of another shape (see tests/asm_hazards.py).  Compiles every csrc/*.hip to
assembly with the library's own flags (hipcc cross-compiles without a GPU)."""
import glob
import os
import subprocess

import pytest

from gated_deltanet_linear_pre_amd import build as B
from tests.asm_hazards import load_over_mfma_operands, mfma_cross_shape_chains

SOURCES = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))


_ASM = {}


def _asm(src, tmp_path):
    if src in _ASM:
        return _ASM[src]
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in B.CFLAGS if f not in ("-fPIC",)]
    cmd = [B.HIPCC, *flags, "--offload-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(f"assembly of {src} failed:\n{r.stderr[-2000:]}")
    _ASM[src] = out.read_text()
    return _ASM[src]


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", SOURCES, ids=[os.path.basename(s) for s in SOURCES])
def test_no_load_overwrites_an_mfma_operand_in_flight(src, tmp_path):
    found = load_over_mfma_operands(_asm(src, tmp_path))
    assert not found, "\n".join(f"{f[:60]} line {n}: {ins} (MFMA at line {m})" for f, n, ins, m in found)


def test_checker_flags_a_planted_overwrite():
    # a load into v[4:7] right after an MFMA that reads v[4:7] as its A operand
    asm = "\n".join([
        "_Zplanted:",
        "\tv_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
        "\tds_read_b128 v[4:7], v20",
        "\tv_add_f32_e32 v30, v0, v1",
        "\tds_read_b128 v[8:11], v21",
    ])
    found = load_over_mfma_operands(asm)
    assert [f[2] for f in found] == ["ds_read_b128 v[4:7], v20"]


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", SOURCES, ids=[os.path.basename(s) for s in SOURCES])
def test_no_mfma_accumulates_onto_another_shape(src, tmp_path):
    found = mfma_cross_shape_chains(_asm(src, tmp_path))
    assert not found, "\n".join(f"{f[:60]} line {n}: {ins} (C written by {w})" for f, n, ins, w in found)


def test_checker_flags_a_planted_cross_shape_chain():
    asm = "\n".join([
        "_Zplanted:",
        # 16x16x32 result read as C by a 16x16x16: flagged
        "\tv_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
        "\tv_mfma_f32_16x16x16_f16 v[12:15], v[16:17], v[18:19], v[0:3]",
        # same-shape chain: allowed
        "\tv_mfma_f32_16x16x32_f16 v[20:23], v[4:7], v[8:11], 0",
        "\tv_mfma_f32_16x16x32_f16 v[20:23], v[4:7], v[8:11], v[20:23]",
        # through a VALU add: allowed
        "\tv_mfma_f32_16x16x16_f16 v[24:27], v[16:17], v[18:19], 0",
        "\tv_add_f32_e32 v24, v24, v1",
        "\tv_add_f32_e32 v25, v25, v1",
        "\tv_add_f32_e32 v26, v26, v1",
        "\tv_add_f32_e32 v27, v27, v1",
        "\tv_mfma_f32_16x16x32_f16 v[24:27], v[4:7], v[8:11], v[24:27]",
    ])
    found = mfma_cross_shape_chains(asm)
    assert [f[2] for f in found] == ["v_mfma_f32_16x16x16_f16 v[12:15], v[16:17], v[18:19], v[0:3]"]
