"""Exhaustive CPU check of the polynomial exp2 that the forward kernel's
hybrid exponential uses (exact_attention_39_amd/csrc/exp2_poly.h).

Every fp32 in [-126, 0] and in [0, 8] (the argument range the kernel feeds
it with the default rescale threshold) is compared with the C library's
exp2 in double precision.  Bound: max relative error <= 2e-4 for both
degrees (the explainer pages only say the polynomial is accurate enough for
bf16; bf16 itself resolves 2^-9 = 2e-3).  Also: exact powers of two at
integer x, monotone on a dense grid, exactly 0 below -126 and at -inf.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def report(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("exp2") / "exp2chk")
    subprocess.check_call(["g++", "-O2", "-fopenmp", "-std=c++17",
                           "-I", os.path.join(ROOT, "exact_attention_39_amd", "csrc"),
                           os.path.join(ROOT, "tests", "exp2_poly_check.cpp"), "-o", exe])
    out = subprocess.check_output([exe], text=True, timeout=600)
    return out.strip().splitlines()


def test_max_relative_error_over_all_floats(report):
    scans = [l.split() for l in report if not l.split()[1].startswith("exact")]
    assert len(scans) == 4
    for deg, lo, hi, cnt, err, arg in scans:
        assert int(cnt) > 10 ** 9, (deg, lo, hi)
        assert float(err) <= 2e-4, (deg, lo, hi, err, arg)
        if deg == "deg5":
            assert float(err) <= 1e-6


def test_integers_exact_monotone_and_zero_below(report):
    flags = [l.split() for l in report if l.split()[1] == "exact_integers"]
    assert len(flags) == 2
    for f in flags:
        assert f[2] == "1" and f[4] == "1" and f[6] == "1", f
