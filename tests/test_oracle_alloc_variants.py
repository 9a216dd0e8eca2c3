"""Pins of the oracle's allocation variants (KVSculpt, gist.science page,
section 2 "Adaptive Budget Allocation": allocation at the layer and the
KV-head level; section 4 "Budget Allocation": static signals such as value
norms).

The two-level split is checked by hand arithmetic and by its reductions to
the flat split (one head per layer, or one layer).  Both reductions are
checked against the flat allocator, which is pinned by hand cases of its
own.  The value-norm signal is checked by hand and by invariances.
"""
import numpy as np
import pytest

from oracle import kvsculpt as O


def test_two_level_hand_case():
    # layers (1, 4), (9, 16), (0, 0): layer means 2.5, 12.5, 0; weights
    # sqrt: 1.5811, 3.5355, 0.  Layer 2 sits at its lower bound 2 (two heads
    # x k_min 1); 58 left: 17.92 and 40.08 -> 18 and 40 (largest remainder).
    # Layer 0 splits 18 by 1 : 2 -> 6, 12; layer 1 splits 40 by 3 : 4 ->
    # 17.14, 22.86 -> 17, 23; layer 2 splits 2 uniformly.
    assert O.allocate_budget_two_level([1, 4, 9, 16, 0, 0], 3, 2, 60) == [6, 12, 17, 23, 1, 1]
    # alpha = 1: layer weights 2.5, 12.5, 0 -> 2 fixed, 58 by 1 : 5 -> 9.67, 48.33 -> 10, 48
    # heads: 10 by 1 : 4 -> 2, 8; 48 by 9 : 16 -> 17.28, 30.72 -> 17, 31
    assert O.allocate_budget_two_level([1, 4, 9, 16, 0, 0], 3, 2, 60, alpha=1.0) == \
        [2, 8, 17, 31, 1, 1]


def test_two_level_reduces_to_the_flat_split():
    rng = np.random.default_rng(0)
    for _ in range(50):
        L = int(rng.integers(1, 9))
        mse = list(rng.exponential(1.0, L) ** 3)
        K = int(rng.integers(L, 40 * L))
        # one head per layer: the flat split over layers
        assert O.allocate_budget_two_level(mse, L, 1, K) == O.allocate_budget(mse, K)
        # one layer: the flat split over its heads
        assert O.allocate_budget_two_level(mse, 1, L, K) == O.allocate_budget(mse, K)


def test_two_level_invariants():
    rng = np.random.default_rng(1)
    for _ in range(100):
        L, H = int(rng.integers(1, 6)), int(rng.integers(1, 5))
        mse = list(rng.exponential(1.0, L * H) ** 2)
        kmin, kmax = int(rng.integers(1, 4)), int(rng.integers(8, 64))
        K = int(rng.integers(L * H * kmin, L * H * kmax + 1))
        k = O.allocate_budget_two_level(mse, L, H, K, 0.5, kmin, kmax)
        assert sum(k) == K and min(k) >= kmin and max(k) <= kmax
    # layers with equal means and equal head patterns get equal budgets
    same = [1.0, 3.0] * 4
    k = O.allocate_budget_two_level(same, 4, 2, 80)
    assert k[0::2] == [k[0]] * 4 and k[1::2] == [k[1]] * 4 and sum(k[:2]) == 20
    with pytest.raises(ValueError):
        O.allocate_budget_two_level([1.0, 2.0, 3.0], 2, 2, 10)


def test_value_norm_signal():
    assert O.value_norm_signal([[3.0, 4.0], [0.0, 0.0], [1.0, 0.0]]) == pytest.approx(2.0, abs=0)
    rng = np.random.default_rng(2)
    V = rng.standard_normal((50, 16))
    s = O.value_norm_signal(V)
    assert O.value_norm_signal(2.5 * V) == pytest.approx(2.5 * s, rel=1e-14)
    assert O.value_norm_signal(V[rng.permutation(50)]) == pytest.approx(s, rel=1e-14)
    assert O.value_norm_signal(V * np.where(rng.random(16) < 0.5, -1, 1)) == pytest.approx(s, rel=1e-14)
