"""Pins of the oracle's pinned binary32 sigmoid S(x) (routing score).

The pages name a scoring step without fixing the function; the workload uses
sigmoid scores.  S() must be a faithful binary32 sigmoid, so it is pinned
against the binary64 sigmoid 1/(1+exp(-x)) from libm over every binary32
input with 2^-26 <= |x| <= 80 (exhaustive) and a stride through the tiny
inputs, plus exact special values.  Error bound 3 ulp: the Cody-Waite
reduction and degree-7 Taylor polynomial contribute < 2 ulp to exp(-x), the
sum 1 + e and the division one rounding each.
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _bits(f):
    return int(np.float32(f).view(np.uint32))


@pytest.fixture(scope="module")
def sweep_lib(tmp_path_factory):
    out = tmp_path_factory.mktemp("sweep") / "sweep.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                    "-fPIC", "-shared", os.path.join(HERE, "c", "score_sweep.c"),
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", str(out), "-lm"],
                   check=True)
    lib = ctypes.CDLL(str(out))
    lib.sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    lib.sweep.restype = None
    return lib


def _sweep(lib, lo, hi, step=1):
    out = np.zeros(4)
    lib.sweep(lo, hi, step, out.ctypes.data)
    return out


def test_special_values(orc):
    s = orc.score(np.array([0.0, -0.0, 80.0, 1e30, np.inf], np.float32))
    assert s[0] == 0.5 and s[1] == 0.5
    assert s[2] == 1.0 and s[3] == 1.0 and s[4] == 1.0
    lo = orc.score(np.array([-80.0, -1e30, -np.inf, np.nan], np.float32))
    # the clamp at -80 keeps the result normal; NaN is treated as -80
    assert np.all(lo == lo[0])
    assert lo[0] > 0
    assert abs(float(lo[0]) - 1.0 / (1.0 + math.exp(80.0))) <= 3 * 2.0 ** -23 * float(lo[0])


def test_exhaustive_accuracy_positive(sweep_lib):
    max_ulp, where, _, n = _sweep(sweep_lib, _bits(2.0 ** -26), _bits(80.0))
    assert n > 2.7e8
    assert max_ulp <= 3.0, (max_ulp, where)


def test_exhaustive_accuracy_negative(sweep_lib):
    max_ulp, where, _, n = _sweep(sweep_lib, _bits(-(2.0 ** -26)), _bits(-80.0))
    assert n > 2.7e8
    assert max_ulp <= 3.0, (max_ulp, where)


def test_tiny_inputs(sweep_lib):
    # |x| < 2^-26: sigmoid(x) = 0.5 + x/4 rounds to 0.5 within one ulp
    for lo, hi in ((0, _bits(2.0 ** -26)), (0x80000000, _bits(-(2.0 ** -26)))):
        max_ulp, where, nonmono, _ = _sweep(sweep_lib, lo, hi, 97)
        assert max_ulp <= 1.0, (max_ulp, where)
        assert nonmono == 0


def test_symmetry_and_range(orc):
    rng = np.random.default_rng(5)
    x = rng.normal(0, 4, 100000).astype(np.float32)
    s, sn = orc.score(x), orc.score(-x)
    assert np.all(s > 0) and np.all(s <= 1)
    # sigmoid(x) + sigmoid(-x) = 1
    assert np.max(np.abs(s.astype(np.float64) + sn - 1.0)) <= 4 * 2.0 ** -24
