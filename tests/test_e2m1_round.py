"""The NVFP4 quantiser's direct E2M1 rounding (csrc/nvfp4.h, e2m1_round)
equals the threshold definition of the E2M1 grid (nearest value, ties to the
code with mantissa bit 0, saturating at 6; NVFP4 release card, precision
table: FP4 E2M1 values) for every non-negative float.  The formula is
written out again in plain C (tests/e2m1_round_check.c) and compared with the
definition over all 2^31 - 2^23 + 1 non-NaN non-negative floats; the device
code itself is checked bit for bit against the oracle's quantiser on the GPU
(test_gpu_ops.py, test_nvfp4_quantize_is_bit_exact)."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_e2m1_round_equals_definition_for_every_float():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "e2m1_round_check")
        subprocess.run(["gcc", "-O2", "-o", exe, os.path.join(HERE, "e2m1_round_check.c"), "-lm"], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "0 mismatches" in r.stdout
