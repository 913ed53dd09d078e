"""The decode kernels compute the DQ block scale k = fp32(s / 127) with a
three-operation division (product with fp32(1/127), one fused correction).
It must equal the correctly rounded quotient, which the dequantization
definition uses, for every finite fp32 s. Checked here on a strided sample
of all fp32 bit patterns (stride 5: about 860 million values; stride 1, the
whole set, passes too) with the host's IEEE division and fmaf."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_three_op_division_by_127_is_correctly_rounded(tmp_path):
    exe = str(tmp_path / "div127")
    src = os.path.join(HERE, "cdiv", "div127.c")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", src, "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe, "5"], check=True, capture_output=True, text=True, timeout=300).stdout.split()
    tested, bad = int(out[0]), int(out[1])
    assert tested > 800_000_000
    assert bad == 0
