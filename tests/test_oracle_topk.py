"""Pins of the oracle's Top-k selection ([PN] 整体框架 Phase 1: the k = N rho least similar tokens).

Brute force on tiny inputs: Python's own float ordering with the documented rules (NaN lowest,
-0 == +0, equal scores to the lower index), every k, and an exhaustive subset check for N <= 10.
"""
import itertools
import math

import numpy as np
import pytest

import oracle


def brute(s, k):
    def key(i):
        v = float(s[i])
        return (-math.inf if math.isnan(v) else v, 0 if math.isnan(v) else 1, i)
    return sorted(sorted(range(len(s)), key=key)[:k])


def tricky_scores(rng, n):
    pool = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, 1.0, -1.0, 0.5, 1e-38, -1e-45,
                     np.float32(0.99999994), 1.0 - 2 ** -24], dtype=np.float32)
    s = rng.uniform(-1, 1, n).astype(np.float32)
    mask = rng.random(n) < 0.5
    s[mask] = rng.choice(pool, mask.sum())
    return s


@pytest.mark.parametrize("seed", range(12))
def test_matches_brute_force_every_k(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 65))
    s = tricky_scores(rng, n)
    for k in range(0, n + 1):
        got = oracle.select_topk(s, k)
        assert got.dtype == np.int32
        assert got.tolist() == brute(s, k), (n, k)


def precedes(s, i, j):
    """Strict total order used by the selection: (NaN first, value, index)."""
    a, b = float(s[i]), float(s[j])
    ka = (-math.inf if math.isnan(a) else a, 0 if math.isnan(a) else 1, i)
    kb = (-math.inf if math.isnan(b) else b, 0 if math.isnan(b) else 1, j)
    return ka < kb


@pytest.mark.parametrize("seed", range(6))
def test_unique_subset_exhaustive(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 11))
    s = tricky_scores(rng, n)
    for k in range(n + 1):
        good = [set(c) for c in itertools.combinations(range(n), k)
                if all(precedes(s, i, j) for i in c for j in range(n) if j not in c)]
        assert len(good) == 1
        assert set(oracle.select_topk(s, k).tolist()) == good[0]


def test_order_key_is_monotone():
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.standard_normal(500).astype(np.float32),
                        np.array([-np.inf, np.inf, 0.0, -0.0, 1e-45, -1e-45, 3.4e38, -3.4e38], np.float32)])
    key = oracle.order_key(v)
    for _ in range(2000):
        i, j = rng.integers(0, len(v), 2)
        if v[i] < v[j]:
            assert key[i] < key[j]
        elif v[i] == v[j]:
            assert key[i] == key[j]
    assert oracle.order_key(np.array([np.nan, -np.inf], np.float32)).tolist()[0] == 0


def test_drifted_tokens_selected():
    # the least similar k of well separated scores are exactly the planted low ones
    rng = np.random.default_rng(10)
    s = (1 - rng.uniform(0, 1e-6, 256)).astype(np.float32)
    low = rng.choice(256, 40, replace=False)
    s[low] = rng.uniform(0.2, 0.9, 40)
    assert oracle.select_topk(s, 40).tolist() == sorted(low.tolist())
