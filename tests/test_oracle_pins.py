"""The CPU oracle against the definition, closed forms, invariants and
library routines (no GPU)."""
import numpy as np
import pytest

import oracle
from oracle import brute
import _pins


@pytest.mark.parametrize("check", _pins.ALL, ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle)


def test_brute_matches_sdpa_independently():
    """The two brute-force evaluations (numpy softmax per prefix, torch SDPA)
    agree with each other, so neither is pinned only by the C oracle."""
    rng = np.random.default_rng(30)
    for n, d in ((1, 1), (17, 3), (300, 64)):
        q = rng.standard_normal(d)
        K = 4 * rng.standard_normal((n, d))
        V = rng.standard_normal((n, d))
        a = brute.brute_scan(q, K, V, 0.5)
        b = brute.sdpa_scan(q, K, V, 0.5)
        assert np.max(np.abs(a - b) / (1 + np.abs(b))) <= 1e-12


def test_oracle_rejects_bad_arguments():
    q = np.zeros((1, 4), np.float32)
    k = np.zeros((1, 1, 0, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.reduce(q, k, k, 1.0)                     # 0/0: no value
    with pytest.raises(ValueError):
        oracle.scan_segmented(q, np.zeros((3, 1, 4), np.float32), np.zeros((3, 1, 4), np.float32),
                              np.array([0, 2, 1, 3]), 1.0)   # offsets decrease
    with pytest.raises(TypeError):
        oracle.scan(q.astype(np.float64), k, k, 1.0)


def test_empty_scan_is_empty():
    q = np.zeros((2, 4), np.float32)
    k = np.zeros((3, 2, 0, 4), np.float32)
    assert oracle.scan(q, k, k, 1.0).shape == (3, 2, 0, 4)


def test_max_scaled_err():
    assert oracle.max_scaled_err([1.0, 2.0], [1.0, 2.0]) == 0.0
    assert abs(oracle.max_scaled_err([2.0], [1.0]) - 0.5) < 1e-15
    assert oracle.max_scaled_err([np.nan], [1.0]) == float("inf")
    assert oracle.max_scaled_err([np.nan], [np.nan]) == 0.0
