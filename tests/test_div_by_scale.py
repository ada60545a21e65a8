"""The E4M3 quantization kernels divide by the block scale with one reciprocal and
Markstein's correction instead of an IEEE division per element; the codes must stay those
of E4M3(RN(x / s)) (Sol-Attn2 draft, "FP8 quantization").  tests/host/div_by_scale.c
compares the two quotients on the host over the bf16 inputs and scales that occur
(every 5th bf16 block maximum here; stride 1 checks all of them, about half a minute)."""
import pathlib
import shutil
import subprocess

import pytest

HERE = pathlib.Path(__file__).parent


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_division_gives_the_ieee_quotient(tmp_path):
    exe = tmp_path / "div_by_scale"
    # -ffp-contract=off: only the two written fmaf calls are fused
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), str(HERE / "host" / "div_by_scale.c"), "-lm"],
                   check=True)
    res = subprocess.run([str(exe), "5"], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout
    assert ", 0 violations" in res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_the_check_rejects_the_uncorrected_product(tmp_path):
    exe = tmp_path / "div_plain"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-DPLAIN_PRODUCT", "-o", str(exe),
                    str(HERE / "host" / "div_by_scale.c"), "-lm"], check=True)
    res = subprocess.run([str(exe), "97"], capture_output=True, text=True, timeout=300)
    assert res.returncode == 1 and ", 0 violations" not in res.stdout
