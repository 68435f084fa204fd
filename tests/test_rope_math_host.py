"""Host checks of the fp64 RoPE arithmetic the kernels share
(``block_sparse_amd/csrc/rope_math.h``), compiled for the CPU.

The rounding of a rotated fp64 value to bf16 (through fp32, with a fix-up
when the fp32 value lands on a bf16 midpoint) is compared with a one-step
nearest-even rounding done on the fp64 bits, on random values, exact
midpoints and values one fp64 ulp or a fraction of an fp32 ulp from a
midpoint: no mismatch is allowed.

The cos/sin routine (Cody-Waite reduction by pi/2, Taylor series) is
compared with long double sinl/cosl over the angles RoPE produces: integer
positions up to past 2^20 times the base-500000 frequencies, every position
around 2^20 at theta_0 = 1, and arguments next to multiples of pi/2.  A
rotated value is x1 c - x2 s with |c|, |s| <= 1, so its error is bounded by
the absolute error of c and s: at most one fp64 ulp of 1 (2^-52) here, which
leaves the one bf16 rounding of a rotated value equal to that of the exact
rotation except within ~2^-44 (relative) of a rounding midpoint.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_sincos_and_bf16_rounding(tmp_path):
    from block_sparse_amd import build as B
    exe = tmp_path / "rope_math_check"
    src = os.path.join(ROOT, "tests", "host", "rope_math_check.cpp")
    r = subprocess.run([B.hipcc(), "-O2", "-std=c++17", "-x", "hip", "--cuda-host-only", src,
                        "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr[-2000:])
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    max_abs, max_ulp, n = float(out[0]), float(out[1]), int(out[2])
    bad, nb = int(out[3]), int(out[4])
    assert n > 2_000_000
    assert max_abs <= 2.0 ** -52, max_abs
    assert max_ulp <= 3.0, max_ulp
    assert nb > 3_000_000 and bad == 0, (bad, nb)
