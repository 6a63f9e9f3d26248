"""Pins of the oracle's ordered binary32 exponential and tanh (LeanExe GPT-2 README,
numerical functions: an ordered binary32 exponential approximation; muInference
page, IEEE-ops table: range reduction, a Taylor polynomial and 2^k as a bit
pattern, checked over all 2^32 inputs).  Against float64 numpy: the exponential
within 2 ulp on dense and random samples of its finite range, tanh within 2e-7
absolute; exact special values; the defined cut-offs."""
import numpy as np

import oracle


def _ulp_err(y, ref):
    return np.abs(y.astype(np.float64) - ref) / np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)


def test_exp_within_two_ulp():
    x = np.linspace(-87.0, 88.72, 3_000_001).astype(np.float32)
    assert _ulp_err(oracle.exp_spec(x), np.exp(x.astype(np.float64))).max() <= 2.0
    rng = np.random.default_rng(0)
    b = rng.integers(0, 2 ** 32, 8_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    b = b[np.isfinite(b) & (b >= -87.0) & (b < 88.7)]
    assert b.size > 1_000_000
    assert _ulp_err(oracle.exp_spec(b), np.exp(b.astype(np.float64))).max() <= 2.0


def test_exp_special_values_and_cutoffs():
    f = oracle.exp_spec
    assert f(np.array([0.0], np.float32))[0] == 1.0
    assert f(np.array([-0.0], np.float32))[0] == 1.0
    assert np.isnan(f(np.array([np.nan], np.float32))[0])
    big = np.array([88.72283935546875, 89.0, 1e30, np.inf], np.float32)
    assert np.all(np.isposinf(f(big)))
    assert np.isfinite(f(np.array([88.7228], np.float32))[0])
    small = np.array([-87.00001, -100.0, -1e30, -np.inf], np.float32)
    assert np.all(f(small) == 0.0)
    lo = f(np.array([-87.0], np.float32))[0]
    assert lo >= np.finfo(np.float32).tiny  # no subnormal results
    # exp(1) and exp(-1) to the nearest binary32 or its neighbour
    for v in (1.0, -1.0, 0.5, -10.0, 20.0):
        got = f(np.array([v], np.float32))[0]
        assert _ulp_err(np.array([got]), np.exp(np.float64(np.float32(v)))) <= 1.5


def test_tanh_accuracy_symmetry_saturation():
    z = np.linspace(-20.0, 20.0, 2_000_001).astype(np.float32)
    t = oracle.tanh_spec(z)
    assert np.abs(t.astype(np.float64) - np.tanh(z.astype(np.float64))).max() <= 2e-7
    assert np.array_equal(oracle.tanh_spec(-z), -t)
    assert oracle.tanh_spec(np.array([0.0], np.float32))[0] == 0.0
    assert np.all(oracle.tanh_spec(np.array([10.0, 50.0, np.inf], np.float32)) == 1.0)
    assert np.all(oracle.tanh_spec(np.array([-10.0, -50.0, -np.inf], np.float32)) == -1.0)


def test_special_bits_matches_values():
    first = np.float32(-3.5).view(np.uint32).item()
    y = oracle.special_bits(0, first, 1000)
    x = (np.arange(1000, dtype=np.uint64) + first).astype(np.uint32).view(np.float32)
    assert np.array_equal(y, oracle.exp_spec(x))
