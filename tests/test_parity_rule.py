"""The acceptance rule itself (no GPU): tolerance 1e-4 * sum|x*w| per output
and cosine >= 0.9999 over all outputs."""
import numpy as np

import oracle


def test_rule_accepts_and_rejects():
    rng = np.random.default_rng(1)
    y = rng.normal(size=1000)
    s = np.abs(y) * 10 + 1.0
    assert oracle.check_parity(y, y, s)["ok"]
    assert oracle.check_parity(y + 0.9e-4 * s, y, s)["ok"]
    assert not oracle.check_parity(y + 1.1e-4 * s, y, s)["ok"]
    bad = y.copy()
    bad[7] = np.nan
    assert not oracle.check_parity(bad, y, s)["ok"]


def test_rule_zero_bound_requires_exact():
    y = np.zeros(4)
    s = np.zeros(4)
    assert oracle.check_parity(y, y, s)["ok"]
    assert not oracle.check_parity(np.array([0, 0, 1e-30, 0]), y, s)["ok"]


def test_rule_accumulate_adds_half_ulp():
    y = np.array([1.0, -2.0])
    s = np.array([0.0, 0.0])
    base = np.array([3.0, 5.0])
    got = np.float32(base + y).astype(np.float64)
    assert oracle.check_parity(got, y, s, base=base)["ok"]


def test_cosine_floor():
    rng = np.random.default_rng(2)
    a = rng.normal(size=500)
    assert oracle.cosine(a, a) > 0.999999
    assert oracle.cosine(a, np.zeros(500)) == 0.0
    s = np.full(500, 1e9)  # huge bound: only the cosine can fail
    assert not oracle.check_parity(rng.normal(size=500), a, s)["ok"]
