"""Oracle pins for the per-layer budget rule and the shared list of a layer.

GateSight Sec. 4.2 and Appendix G (layer_power_budget: budgets proportional to the layer
gate weight, largest-remainder integerised to the flat total L*round(p*(n-prot)), prompt in
addition) and Appendix H (one kept list per layer ranked by the larger per-head score, kept
count a multiple of four).
"""

import math

import numpy as np
import pytest

import oracle


def test_layer_budget_worked_examples():
    # exact proportional shares: 120 = 10 * 12 over weights 1:2:3:4
    assert oracle.layer_power_budget([1, 2, 3, 4], 100, 0.3) == [12, 24, 36, 48]
    # equal weights, T = 3 * round(0.5 * 7) = 3 * 4 = 12 (3.5 rounds to even 4): flat
    assert oracle.layer_power_budget([0.3, 0.3, 0.3], 7, 0.5) == [4, 4, 4]
    # T = 3 * round(12 / 3) = 12: q = 12/7 * (1, 2, 4) = 1.71, 3.43, 6.86 -> floors 1, 3, 6
    # and the two largest remainders (.86 of layer 2, .71 of layer 0) get +1
    assert oracle.layer_power_budget([1, 2, 4], 12, 1 / 3) == [2, 3, 7]
    # T = 3 * round(10 / 3) = 9: q = 9/7 * (1, 2, 4) = 1.29, 2.57, 5.14 -> one extra, to layer 1
    assert oracle.layer_power_budget([1, 2, 4], 10, 1 / 3) == [1, 3, 5]
    # equal remainders go to the lower layer: T = 3 * 2 = 6, q = 1.5, 1.5, 3 -> 2, 1, 3
    assert oracle.layer_power_budget([1, 1, 2], 4, 0.5) == [2, 1, 3]


@pytest.mark.parametrize("seed", range(8))
def test_layer_budget_sum_quota_and_order(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 40))
    gate = np.exp(rng.uniform(np.log(0.022), np.log(0.459), L)).astype(np.float32)
    n_body = int(rng.integers(1, 40000))
    p = float(rng.uniform(0, 0.045))  # gates span < 21x, so no layer reaches the cap n_body
    K = oracle.layer_power_budget(gate, n_body, p)
    flat = oracle.budget(1, n_body, 0, p)
    assert sum(K) == L * flat
    share = L * flat * gate.astype(np.float64) / gate.astype(np.float64).sum()
    assert np.all(np.abs(np.array(K) - share) < 1 + 1e-9)  # largest-remainder quota
    order = np.argsort(gate, kind="stable")
    assert np.all(np.diff(np.array(K)[order]) >= 0)        # a larger gate never keeps less


def test_layer_budget_flat_zero_full():
    assert oracle.layer_power_budget([0.1] * 16, 32512, 0.25) == [8128] * 16  # the page's flat budget
    assert oracle.layer_power_budget([0.05, 0.4, 0.2], 500, 0.0) == [0, 0, 0]
    assert oracle.layer_power_budget([0.05, 0.4, 0.2], 500, 1.0) == [500, 500, 500]  # capped
    K = oracle.layer_power_budget([0.02, 0.02, 0.9], 100, 0.6)  # 180 with the third capped at 100
    assert K[2] == 100 and sum(K) == 180 and K[0] == K[1] == 40
    with pytest.raises(ValueError):
        oracle.layer_power_budget([0.1, 0.0], 10, 0.5)


def test_layer_budget_page_shape():
    """16 attention layers with gates over the page's 0.022..0.459 range, n = 32768, prot = 256."""
    gate = np.geomspace(0.022, 0.459, 16).astype(np.float32)
    K = oracle.layer_power_budget(gate, 32768 - 256, 0.25)
    assert sum(K) == 16 * 8128 and max(K) < 32512 and min(K) > 0
    assert K == sorted(K)


def test_shared_max_scores():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((6 * 4, 50)).astype(np.float32)
    got = oracle.shared_max_scores(s, 4)
    assert np.array_equal(got, s.reshape(6, 4, 50).max(axis=1))  # distinct finite values
    assert np.array_equal(oracle.shared_max_scores(s, 1), s)      # one head: identity
    t = np.array([[np.nan, -0.0, 1.0, np.nan, -np.inf],
                  [0.5, 0.0, 1.0, np.nan, np.nan]], dtype=np.float32)
    got = oracle.shared_max_scores(t, 2)[0]
    assert got[0] == 0.5                                    # NaN ranks below everything
    assert got[1] == 0.0 and math.copysign(1, got[1]) < 0   # -0 ties +0: the lower head's bits
    assert got[2] == 1.0
    assert np.isnan(got[3])                                 # all NaN stays NaN
    assert got[4] == -np.inf                                # -inf beats NaN


def test_shared_kept_count():
    assert oracle.shared_kept_count(2048, 1024) == 2048
    assert oracle.shared_kept_count(2047, 1024) == 2044
    assert oracle.shared_kept_count(103, 100) == 100
    with pytest.raises(ValueError):
        oracle.shared_kept_count(102, 101)


@pytest.mark.parametrize("seed", range(6))
def test_layer_budget_capped(seed):
    """Past the cap: capped layers keep n_body, the rest share the remainder by quota."""
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(2, 30))
    gate = np.exp(rng.uniform(np.log(0.022), np.log(0.459), L)).astype(np.float32)
    n_body = int(rng.integers(10, 5000))
    p = float(rng.uniform(0.3, 1.0))
    K = np.array(oracle.layer_power_budget(gate, n_body, p))
    T = L * oracle.budget(1, n_body, 0, p)
    assert K.sum() == T and np.all(K <= n_body) and np.all(K >= 0)
    order = np.argsort(gate, kind="stable")
    assert np.all(np.diff(K[order]) >= 0)
    capped = K == n_body
    free = ~capped
    if free.any() and capped.any():
        g = gate.astype(np.float64)
        share = (T - n_body * capped.sum()) * g[free] / g[free].sum()
        assert np.all(np.abs(K[free] - share) < 1 + 1e-9)
        assert np.all(share < n_body + 1)
