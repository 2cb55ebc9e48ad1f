"""Pins of the oracle's specified binary32 exp / sigmoid / SiLU against
float64 mathematics (math.exp) and closed forms."""

import math

import numpy as np

from oracle import spec_exp, spec_sigmoid, spec_silu
from oracle.specmath import LN2_HI, LN2_LO


def _ulp32(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


def test_cody_waite_constants():
    bits = np.array([LN2_HI], np.float32).view(np.uint32)[0]
    assert bits & 0x1FF == 0                       # 9 trailing zero bits
    assert abs(float(LN2_HI) + float(LN2_LO) - math.log(2.0)) < 1e-12
    n = np.arange(-128, 129, dtype=np.float32)
    assert np.array_equal((n * LN2_HI).astype(np.float64), n.astype(np.float64) * float(LN2_HI))


def test_exp_accuracy_dense_grid():
    rng = np.random.default_rng(0)
    y = np.concatenate([np.linspace(-80, 80, 4_000_001, dtype=np.float32),
                        rng.uniform(-1, 1, 1_000_000).astype(np.float32),
                        np.arange(-115, 116, dtype=np.float32) * np.float32(math.log(2))])
    got = spec_exp(y).astype(np.float64)
    ref = np.exp(y.astype(np.float64))
    err = np.abs(got - ref) / _ulp32(ref)
    assert err.max() <= 2.0, err.max()


def test_exp_special_values():
    assert spec_exp(np.float32(0.0)) == 1.0
    assert spec_exp(np.float32(100.0)) == spec_exp(np.float32(80.0))
    assert spec_exp(np.float32(-100.0)) == spec_exp(np.float32(-80.0))
    assert np.isfinite(spec_exp(np.float32(80.0))) and spec_exp(np.float32(-80.0)) > 0


def test_sigmoid_closed_forms():
    assert spec_sigmoid(np.float32(0.0)) == np.float32(0.5)
    assert spec_sigmoid(np.float32(200.0)) == np.float32(1.0)
    x = np.linspace(-30, 30, 600_001, dtype=np.float32)
    s = spec_sigmoid(x)
    ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    assert (np.abs(s - ref) / _ulp32(ref)).max() <= 3.0
    assert np.all(np.diff(s) >= 0)                         # monotone
    sym = s.astype(np.float64) + spec_sigmoid(-x).astype(np.float64)
    assert np.abs(sym - 1.0).max() <= 2 ** -22


def test_silu_closed_forms():
    assert spec_silu(np.float32(0.0)) == 0.0
    x = np.linspace(-20, 20, 200_001, dtype=np.float32)
    ref = x.astype(np.float64) / (1.0 + np.exp(-x.astype(np.float64)))
    got = spec_silu(x).astype(np.float64)
    assert (np.abs(got - ref) <= 4 * _ulp32(ref) + 1e-45).all()
