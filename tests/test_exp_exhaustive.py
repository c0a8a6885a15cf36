"""The raster kernels' exact exponentials (exp_rn, and the forward's exp_neg_rn of the negated argument), built for the host from the kernels' own header, against the oracle's
definition of the fp32 e^x, float(exp(double(x))), over every float argument the kernels evaluate (x in [-5.55, 0],
about 1.09e9 floats): every decision that depends on exp(-sigma) is then the same on both sides.

float(exp(double(x))) is the correctly rounded value unless e^x lies within about 1e-16 of an fp32 rounding
midpoint; the two arguments where an earlier, less accurate evaluation disagreed with it (3e-15 and 2.7e-16 from a
midpoint) are checked against a 60-digit evaluation.
"""
import os
import shutil
import subprocess
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "differentiable_gaussian_splatting_amd", "csrc")


def correctly_rounded_exp(x: float) -> np.float32:
    getcontext().prec = 60
    f = Fraction(x)
    e = (Decimal(f.numerator) / Decimal(f.denominator)).exp()
    return np.float32(float(Fraction(e)))  # double then float: exact here (checked below by the midpoint margin)


@pytest.mark.parametrize("xhex,want", [("-0x1.03d5bep+0", "0x1.731b82p-2"), ("-0x1.e1dbe2p-8", "0x1.fc3fd2p-1")])
def test_reference_on_near_midpoint_arguments(xhex, want):
    """The two arguments whose e^x lies closest to an fp32 midpoint (3e-15 and 2.7e-16 relative) round up."""
    x = float.fromhex(xhex)
    assert np.float32(np.exp(np.float64(x))) == np.float32(float.fromhex(want))
    assert correctly_rounded_exp(x) == np.float32(float.fromhex(want))


def test_exact_exponential_is_correctly_rounded_on_every_argument(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "exp_exhaustive"
    subprocess.run([hipcc, "-O2", "-std=c++17", "-ffp-contract=off", "-pthread", f"-I{CSRC}",
                    f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "exp_exhaustive.cpp"),
                    "-o", str(exe)], check=True, capture_output=True)
    threads = str(min(16, os.cpu_count() or 1))
    out = subprocess.run([str(exe), threads], check=True, capture_output=True, text=True).stdout.split()
    total, bad, bad_neg = int(out[0]), int(out[1]), int(out[2])
    assert total == 1_085_381_019
    assert bad == 0
    assert bad_neg == 0
