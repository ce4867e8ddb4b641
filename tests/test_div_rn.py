"""The row quantizers' division identity, on the CPU.

The HIP quantizers compute v / s as RN(q0 + (v - q0 * s) * y) with
y = RN(1 / s) and q0 = RN(v * y), two FMAs instead of an IEEE division per
element. The codes must equal the oracle's, which divides; this checks that
the quotient itself is identical near every code boundary (n + 1/2) * s for
every 4th significand of s in one binade (IEEE single operations, so the
result carries over to the GPU's v_mul_f32 / v_fma_f32)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fma_corrected_quotient_equals_ieee_division(tmp_path):
    exe = tmp_path / "div_rn_check"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "div_rn_check.c"), "-lm"], check=True)
    out = subprocess.run([str(exe), "4"], check=True, capture_output=True, text=True,
                         env=dict(os.environ, OMP_NUM_THREADS=os.environ.get("OMP_NUM_THREADS", "8"))).stdout
    bad, cases = int(out.split()[1]), int(out.split()[3])
    assert cases == (1 << 21) * 256 * 7
    assert bad == 0, out
