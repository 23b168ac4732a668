"""Pins of the oracle's per-layer budget rho(l), k_l ([PN] 关键设计 3, the rho(l) equation).

What the pages fix: rho(1) = rho_1, rho(l_p) = rho_p, rho(L) = rho_L; a bell that rises to the
peak and falls after it; with (rho_p, rho_1, rho_L) = (25%, 5%, 8%) the mean budget is about 16%
([PN] 实验关键数据, ablation table: peak 25%, mean 16%).
"""
import math

import numpy as np
import pytest

import oracle

LLADA = dict(n_layers=32, l_peak=12, rho_peak=0.25, rho_first=0.05, rho_last=0.08)
DREAM = dict(n_layers=28, l_peak=10, rho_peak=0.25, rho_first=0.05, rho_last=0.08)


@pytest.mark.parametrize("p,n", [(LLADA, 1024), (DREAM, 2048)])
def test_endpoints_and_peak_exact(p, n):
    rho, k = oracle.budget(n_tokens=n, **p)
    assert rho[0] == p["rho_first"]
    assert rho[p["l_peak"] - 1] == p["rho_peak"]
    assert rho[-1] == p["rho_last"]
    assert k[p["l_peak"] - 1] == int(n * p["rho_peak"])


@pytest.mark.parametrize("p", [LLADA, DREAM])
def test_bell_shape(p):
    rho, _ = oracle.budget(n_tokens=1024, **p)
    lp = p["l_peak"]
    assert np.all(np.diff(rho[:lp]) > 0), "must rise strictly up to the peak"
    assert np.all(np.diff(rho[lp - 1:]) < 0), "must fall strictly after the peak"
    assert rho.max() == p["rho_peak"] and int(np.argmax(rho)) == lp - 1


def test_half_way_value_closed_form():
    # l_p = 3, l = 2 sits half way on the left branch (t = -1/2): rho = rho_p^(3/4) rho_1^(1/4).
    # 0.25^0.75 = 0.353553390593..., 0.05^0.25 = 0.472870804501...; product 0.167185076244...
    rho, _ = oracle.budget(3, 3, 0.25, 0.05, 0.05, 100)
    assert abs(rho[1] - 0.16718507624410553) < 1e-15
    # right branch, L = 5, l_p = 1, l = 3 (t = 1/2): rho_p^(3/4) rho_L^(1/4) with rho_L = 0.05
    rho, _ = oracle.budget(5, 1, 0.25, 0.25, 0.05, 100)
    assert abs(rho[2] - 0.16718507624410553) < 1e-15


def test_gaussian_in_layer_index():
    # log(rho(l)/rho_p) must be a quadratic in (l - l_p) on each branch: second differences equal.
    rho, _ = oracle.budget(n_tokens=1024, **LLADA)
    lg = np.log(rho / 0.25)
    left = lg[:12]
    d2 = np.diff(left, 2)
    assert np.allclose(d2, d2[0], rtol=0, atol=1e-12)
    right = lg[11:]
    d2r = np.diff(right, 2)
    assert np.allclose(d2r, d2r[0], rtol=0, atol=1e-12)
    # curvature: log(rho_1/rho_p) / (l_p - 1)^2 per unit step squared, times 2
    assert abs(d2[0] - 2 * math.log(0.05 / 0.25) / 11 ** 2) < 1e-12
    assert abs(d2r[0] - 2 * math.log(0.08 / 0.25) / 20 ** 2) < 1e-12


def test_mean_budget_near_sixteen_percent():
    # the pages quote a 16% mean for a 25% peak; the excerpts do not print the exact l_p / rho_1 /
    # rho_L behind it, so this is a loose check (it fails for a wrong branch or a missing square).
    rho, k = oracle.budget(n_tokens=1024, **LLADA)
    assert 0.15 < rho.mean() < 0.18
    assert 0.15 < k.mean() / 1024 < 0.18
    rho_d, _ = oracle.budget(n_tokens=2048, **DREAM)
    assert 0.15 < rho_d.mean() < 0.18


def test_k_rounding():
    _, k = oracle.budget(1, 1, 0.05, 0.05, 0.05, 1024)
    assert k[0] == 51                    # 1024 * 0.05 = 51.2 -> floor
    _, k = oracle.budget(1, 1, 0.29, 0.29, 0.29, 100)
    assert k[0] == 29                    # 100 * 0.29 = 28.999999999999996 -> guard gives 29
    _, k = oracle.budget(1, 1, 1e-6, 1e-6, 1e-6, 64)
    assert k[0] == 1                     # clamped to at least one row
    _, k = oracle.budget(1, 1, 1.0, 1.0, 1.0, 64)
    assert k[0] == 64


def test_degenerate_layouts():
    rho, _ = oracle.budget(1, 1, 0.3, 0.1, 0.2, 10)
    assert rho.tolist() == [0.3]                       # a single layer is the peak
    rho, _ = oracle.budget(4, 1, 0.3, 0.1, 0.2, 10)    # peak first: only the right branch
    assert rho[0] == 0.3 and rho[-1] == 0.2 and np.all(np.diff(rho) < 0)
    rho, _ = oracle.budget(4, 4, 0.3, 0.1, 0.2, 10)    # peak last: only the left branch
    assert rho[0] == 0.1 and rho[-1] == 0.3 and np.all(np.diff(rho) > 0)
    rho, _ = oracle.budget(6, 3, 0.2, 0.2, 0.2, 10)    # uniform budget
    assert np.all(rho == 0.2)


@pytest.mark.parametrize("args", [(0, 1, .2, .1, .1, 8), (4, 5, .2, .1, .1, 8), (4, 0, .2, .1, .1, 8),
                                  (4, 2, 0.0, .1, .1, 8), (4, 2, .2, 1.5, .1, 8), (4, 2, .2, .1, .1, 0)])
def test_rejects_bad_arguments(args):
    with pytest.raises(ValueError):
        oracle.budget(*args)
