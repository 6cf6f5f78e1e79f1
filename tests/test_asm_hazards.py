"""The kernels' gfx950 assembly holds no load that overwrites an operand of an
MFMA still in flight (see tests/asm_hazards.py).  Compiles every csrc/*.hip to
assembly with the library's own flags (hipcc cross-compiles without a GPU)."""
import glob
import os
import subprocess

import pytest

from gated_deltanet_linear_pre_amd import build as B
from tests.asm_hazards import load_over_mfma_operands

SOURCES = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))


def _asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in B.CFLAGS if f not in ("-fPIC",)]
    cmd = [B.HIPCC, *flags, "--offload-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(f"assembly of {src} failed:\n{r.stderr[-2000:]}")
    return out.read_text()


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
