"""Exhaustive host proof of the device quotient method (CPU only).

The quantizers form x / s as a scaled reciprocal plus one FMA correction
instead of a full division per element.  tests/csrc/divcheck.c runs the same
fp32 steps over every (amax, x) pair of positive finite bf16 values with
x <= amax (532,701,119 pairs) and compares with IEEE single division; the
two must agree bit for bit wherever the quotient can change the E4M3 code.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_quotient_method_exhaustive(tmp_path):
    exe = str(tmp_path / "divcheck")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "csrc", "divcheck.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    pairs, diff, bad = (int(v) for v in r.stdout.split())
    assert pairs == 532701119
    assert bad == 0, r.stderr
    assert r.returncode == 0


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_static_scale_quotient_exhaustive(tmp_path):
    """The same method with an arbitrary normal scale (static quantizers,
    KV cache): every fp32 scale mantissa against every bf16 input mantissa,
    at the x' exponents 0, -11 and 9 (3 * 2^30 pairs), bit for bit."""
    exe = str(tmp_path / "divcheck_scale")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "csrc", "divcheck_scale.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    pairs, bad = (int(v) for v in r.stdout.split())
    assert pairs == 3 * 2 ** 30
    assert bad == 0, r.stderr
    assert r.returncode == 0
