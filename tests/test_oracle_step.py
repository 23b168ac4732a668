"""Pins of the oracle's whole cached layer step ([PN] 整体框架 phases 1-3; [GS] part 3).

What the pages fix: with every token selected (rho = 1) the cached step is the full recompute;
rows outside I keep their cached K/V/H; K/V of I are written to the cache before the sparse
queries attend to it; tokens that drift most are the ones recomputed.
"""
import numpy as np
import pytest

import oracle
import synth

EPS = 1e-6


def setup(shape, seed, std=0.1, gains="random"):
    w = synth.random_weights(shape, seed=seed, std=std, gains=gains)
    w_r = oracle.singular_proxy(w["w_v"], w["g_attn"], shape.rank)
    x0 = synth.random_hidden(shape, seed=seed + 1)
    return w, w_r, x0


SHAPES = [synth.LayerShape(2, 40, 64, 4, 4, 16, 96, 8, "f32"),
          synth.LayerShape(1, 48, 96, 6, 2, 16, 80, 12, "f32")]


@pytest.mark.parametrize("shape", SHAPES)
def test_rho_one_equals_full_recompute(shape):
    w, w_r, x0 = setup(shape, 11)
    cache = oracle.warmup(x0, w, w_r, shape.head_dim, EPS, "f64")
    x1 = x0 + 0.3 * synth.random_hidden(shape, seed=99)
    new, idx, s = oracle.cached_layer_step(x1, w, w_r, cache, shape.n_tokens, shape.head_dim, EPS, "f64")
    assert np.array_equal(idx, np.tile(np.arange(shape.n_tokens), (shape.batch, 1)))
    kc, vc, h = oracle.full_layer(x1, w, shape.head_dim, EPS, "f64")
    assert np.max(np.abs(new.k - kc)) < 1e-12
    assert np.max(np.abs(new.v - vc)) < 1e-12
    assert np.max(np.abs(new.h - h)) < 1e-12
    assert np.array_equal(new.p, oracle.proxy(x1, w_r).astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("dtype", ["f64", "bf16"])
def test_unselected_rows_untouched(dtype):
    shape = SHAPES[1]
    w, w_r, x0 = setup(shape, 21)
    cache = oracle.warmup(x0, w, w_r, shape.head_dim, EPS, dtype)
    x1 = x0 + 0.3 * synth.random_hidden(shape, seed=98)
    k = 11
    new, idx, _ = oracle.cached_layer_step(x1, w, w_r, cache, k, shape.head_dim, EPS, dtype)
    rest = np.setdiff1d(np.arange(shape.n_tokens), idx[0])
    assert np.array_equal(new.h[0][rest], cache.h[0][rest])
    assert np.array_equal(new.k[0][:, rest], cache.k[0][:, rest])
    assert np.array_equal(new.v[0][:, rest], cache.v[0][:, rest])
    assert not np.array_equal(new.h[0][idx[0]], cache.h[0][idx[0]])


def test_fixed_point_for_unchanged_input():
    shape = SHAPES[0]
    w, w_r, x0 = setup(shape, 31)
    cache = oracle.warmup(x0, w, w_r, shape.head_dim, EPS, "f64")
    for k in (1, 7, 40):
        new, _, s = oracle.cached_layer_step(x0, w, w_r, cache, k, shape.head_dim, EPS, "f64")
        assert np.max(np.abs(new.h - cache.h)) < 1e-12
        assert np.max(np.abs(new.k - cache.k)) < 1e-12
        assert np.allclose(s, 1.0, atol=1e-6)


def test_permutation_equivariance():
    shape = SHAPES[1]
    w, w_r, x0 = setup(shape, 41)
    cache = oracle.warmup(x0, w, w_r, shape.head_dim, EPS, "f64")
    x1 = x0 + 0.2 * synth.random_hidden(shape, seed=97)
    perm = np.random.default_rng(5).permutation(shape.n_tokens)
    pc = oracle.LayerCache(cache.k[:, :, perm], cache.v[:, :, perm], cache.h[:, perm], cache.p[:, perm])
    a, ia, sa = oracle.cached_layer_step(x1, w, w_r, cache, 9, shape.head_dim, EPS, "f64")
    b, ib, sb = oracle.cached_layer_step(x1[:, perm], w, w_r, pc, 9, shape.head_dim, EPS, "f64")
    assert np.array_equal(sb, sa[:, perm])
    assert sorted(perm[ib[0]].tolist()) == ia[0].tolist()
    assert np.max(np.abs(b.h - a.h[:, perm])) < 1e-12


def test_attention_reads_cache_after_scatter():
    # Attending to the stale cache (before the K/V scatter) gives a different H^c[I]; the oracle
    # must match an explicit "scatter, then attend" computation written out here row by row.
    shape = SHAPES[0].replace(batch=1)
    w, w_r, x0 = setup(shape, 51)
    cache = oracle.warmup(x0, w, w_r, shape.head_dim, EPS, "f64")
    x1 = x0 + 0.5 * synth.random_hidden(shape, seed=96)
    idx = np.array([[3, 8, 20, 33]])
    new = oracle.sparse_update(x1, w, cache, idx, shape.head_dim, EPS, "f64")
    hd, n = shape.head_dim, shape.n_tokens
    xf = x1[0]
    a_all = oracle.rmsnorm(xf, w["g_attn"], EPS)
    kfull = cache.k[0].copy()
    vfull = cache.v[0].copy()
    for i in idx[0]:
        kfull[:, i] = (a_all[i] @ w["w_k"].T).reshape(-1, hd)
        vfull[:, i] = (a_all[i] @ w["w_v"].T).reshape(-1, hd)
    q = (a_all[idx[0]] @ w["w_q"].T).reshape(len(idx[0]), -1, hd)
    o_new = oracle.attention(q, kfull, vfull)
    o_old = oracle.attention(q, cache.k[0], cache.v[0])
    def finish(o):
        y = xf[idx[0]] + o @ w["w_o"].T
        bb = oracle.rmsnorm(y, w["g_ffn"], EPS)
        return y + (oracle.silu(bb @ w["w_gate"].T) * (bb @ w["w_up"].T)) @ w["w_down"].T
    assert np.max(np.abs(new.h[0][idx[0]] - finish(o_new))) < 1e-12
    assert np.max(np.abs(finish(o_old) - finish(o_new))) > 1e-6


def test_policies():
    shape = SHAPES[0]
    w, w_r, x0 = setup(shape, 61)
    cache = oracle.warmup(x0, w, w_r, shape.head_dim, EPS, "f64")
    x1 = x0 + 0.3 * synth.random_hidden(shape, seed=95)
    p_new = oracle.proxy(x1, w_r).astype(np.float32).astype(np.float64)
    a, ia, _ = oracle.cached_layer_step(x1, w, w_r, cache, 5, shape.head_dim, EPS, "f64", oracle.POLICY_ALL)
    b, ib, _ = oracle.cached_layer_step(x1, w, w_r, cache, 5, shape.head_dim, EPS, "f64", oracle.POLICY_SELECTED)
    assert np.array_equal(a.p, p_new)
    for bi in range(shape.batch):
        rest = np.setdiff1d(np.arange(shape.n_tokens), ib[bi])
        assert np.array_equal(b.p[bi][ib[bi]], p_new[bi][ib[bi]])
        assert np.array_equal(b.p[bi][rest], cache.p[bi][rest])
    assert np.array_equal(a.h, b.h)


@pytest.mark.parametrize("seed", range(4))
def test_tiny_config_recalls_planted_drift(seed):
    # tiny fp32 config: 13 of 64 tokens drift by N(0, 0.5^2), the rest by N(0, (1e-3)^2); with k = 16
    # every drifted token must be among the selected ones.
    wl = synth.WORKLOADS["tiny-f32"]
    shape = wl.shape
    w = synth.layer_weights(wl)
    w_r = oracle.singular_proxy(w["w_v"], w["g_attn"], shape.rank)
    x0 = synth.first_hidden(wl)
    rng = np.random.default_rng([1, 0, 3, seed])
    x1, rows = synth.drift_step(x0, 13, rng, shape.dtype)
    cache = oracle.warmup(x0, w, w_r, shape.head_dim, EPS, "f32")
    _, k = oracle.budget(1, 1, wl.rho, wl.rho, wl.rho, shape.n_tokens)
    assert k[0] == 16
    _, idx, s = oracle.cached_layer_step(x1, w, w_r, cache, int(k[0]), shape.head_dim, EPS, "f32")
    assert set(rows[0].tolist()) <= set(idx[0].tolist())
