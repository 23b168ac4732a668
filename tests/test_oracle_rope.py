"""Pins of the oracle's optional architecture terms: rotary position embedding on q and k, and
biases on q, k, v (fidelity to the LLaDA / Dream layers; the pages name neither).

RoPE is checked against its definition as a complex rotation (each adjacent pair of dims is a
complex number multiplied by exp(i pos theta^(-2j/hd))), against the 2 x 2 rotation matrix for a
single pair, and against the properties that make it a position code: identity at position 0, norm
preservation, and q . k depending only on the position difference. The whole block with both terms
is checked against a torch.nn.functional composition that applies the rotation as complex products.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def t64(a):
    return torch.as_tensor(np.asarray(a, np.float64))


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((1, 3, 16))
    assert np.array_equal(oracle.rope(x, [0], 10000.0), x)


def test_rope_single_pair_is_a_rotation_by_the_position():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 1, 2))
    pos = np.array([0, 1, 7, 100, 12345])
    got = oracle.rope(x, pos, 500000.0)        # head_dim 2: the only frequency is theta^0 = 1
    for i, p in enumerate(pos):
        rot = np.array([[math.cos(p), -math.sin(p)], [math.sin(p), math.cos(p)]])
        assert np.allclose(got[i, 0], rot @ x[i, 0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("hd,theta", [(16, 10000.0), (64, 500000.0), (128, 1e6)])
def test_rope_matches_complex_rotation(hd, theta):
    rng = np.random.default_rng(hd)
    x = rng.standard_normal((9, 3, hd))
    pos = rng.integers(0, 4096, 9)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    freq = np.array([theta ** (-(2.0 * j) / hd) for j in range(hd // 2)])
    zr = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    got = oracle.rope(x, pos, theta)
    assert np.allclose(got[..., 0::2], zr.real, rtol=1e-12, atol=1e-12)
    assert np.allclose(got[..., 1::2], zr.imag, rtol=1e-12, atol=1e-12)


def test_rope_preserves_pair_norms_and_depends_on_relative_position():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 32))
    k = rng.standard_normal((1, 1, 32))
    theta = 10000.0
    for m, n in [(0, 5), (3, 3), (100, 17), (2048, 1)]:
        rq, rk = oracle.rope(q, [m], theta), oracle.rope(k, [n], theta)
        assert np.allclose(rq[..., 0::2] ** 2 + rq[..., 1::2] ** 2, q[..., 0::2] ** 2 + q[..., 1::2] ** 2, rtol=1e-12)
        for t in (1, 50, 999):
            sq, sk = oracle.rope(q, [m + t], theta), oracle.rope(k, [n + t], theta)
            assert abs(np.sum(rq * rk) - np.sum(sq * sk)) < 1e-10


def torch_block_rope_bias(x, w, hd, eps, theta):
    """The pre-norm SwiGLU block from torch.nn.functional with linear biases on q, k, v and the
    rotary embedding applied as complex multiplication (float64)."""
    x = t64(x)
    hq = w["w_q"].shape[0] // hd
    hkv = w["w_k"].shape[0] // hd
    b, n, d = x.shape
    a = F.rms_norm(x, (d,), weight=t64(w["g_attn"]), eps=eps)
    q = F.linear(a, t64(w["w_q"]), t64(w["b_q"])).view(b, n, hq, hd)
    k = F.linear(a, t64(w["w_k"]), t64(w["b_k"])).view(b, n, hkv, hd)
    v = F.linear(a, t64(w["w_v"]), t64(w["b_v"])).view(b, n, hkv, hd).transpose(1, 2)
    freq = theta ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = torch.arange(n, dtype=torch.float64)[:, None] * freq[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]

    def rotate(t):
        c = torch.view_as_complex(t.reshape(*t.shape[:-1], hd // 2, 2).contiguous()) * rot
        return torch.view_as_real(c).reshape(t.shape)

    q = rotate(q).transpose(1, 2)
    k = rotate(k).transpose(1, 2)
    o = F.scaled_dot_product_attention(q, k.repeat_interleave(hq // hkv, 1), v.repeat_interleave(hq // hkv, 1))
    y = x + F.linear(o.transpose(1, 2).reshape(b, n, hq * hd), t64(w["w_o"]))
    bb = F.rms_norm(y, (d,), weight=t64(w["g_ffn"]), eps=eps)
    h = y + F.linear(F.silu(F.linear(bb, t64(w["w_gate"]))) * F.linear(bb, t64(w["w_up"])), t64(w["w_down"]))
    return k.numpy(), v.numpy(), h.numpy()


def _with_rope_bias(w, shape, seed, theta):
    rng = np.random.default_rng([97, seed])
    w = dict(w)
    w["b_q"] = rng.standard_normal(shape.d_q) * 0.1
    w["b_k"] = rng.standard_normal(shape.d_kv) * 0.1
    w["b_v"] = rng.standard_normal(shape.d_kv) * 0.1
    w["rope_theta"] = theta
    return w


@pytest.mark.parametrize("shape,theta", [
    (synth.LayerShape(2, 24, 64, 4, 4, 16, 96, 8, "f32"), 10000.0),
    (synth.LayerShape(1, 33, 96, 6, 2, 16, 80, 8, "f32"), 1e6),
])
def test_full_layer_with_rope_and_biases_matches_torch(shape, theta):
    w = _with_rope_bias(synth.random_weights(shape, seed=15, std=0.1, gains="random"), shape, 15, theta)
    x = synth.random_hidden(shape, seed=16)
    kc, vc, h = oracle.full_layer(x, w, shape.head_dim, 1e-6, "f64")
    rk, rv, rh = torch_block_rope_bias(x, w, shape.head_dim, 1e-6, theta)
    assert np.allclose(kc, rk, rtol=1e-12, atol=1e-12)
    assert np.allclose(vc, rv, rtol=1e-12, atol=1e-12)
    assert np.allclose(h, rh, rtol=1e-12, atol=1e-12)


def test_cached_step_at_rho_one_equals_full_layer_with_rope_and_biases():
    shape = synth.LayerShape(2, 40, 64, 4, 2, 16, 96, 16, "f32")
    w = _with_rope_bias(synth.random_weights(shape, seed=17, std=0.1), shape, 17, 10000.0)
    w_r = oracle.singular_proxy(w["w_v"], w["g_attn"], shape.rank)
    x0, x1 = synth.random_hidden(shape, seed=18), synth.random_hidden(shape, seed=19)
    cache = oracle.warmup(x0, w, w_r, shape.head_dim, 1e-6, "f64")
    new, idx, _ = oracle.cached_layer_step(x1, w, w_r, cache, shape.n_tokens, shape.head_dim, 1e-6, "f64")
    kc, vc, h = oracle.full_layer(x1, w, shape.head_dim, 1e-6, "f64")
    assert np.array_equal(idx, np.tile(np.arange(shape.n_tokens), (shape.batch, 1)))
    assert np.allclose(new.k, kc, rtol=1e-12, atol=1e-12)
    assert np.allclose(new.v, vc, rtol=1e-12, atol=1e-12)
    assert np.allclose(new.h, h, rtol=1e-12, atol=1e-12)


def test_rope_moves_keys_by_position_in_the_cache():
    """The rotation uses each token's own index: a token's cached key differs from the unrotated key by
    exactly its position's rotation, whether it was written by the warm-up or by a sparse update."""
    shape = synth.LayerShape(1, 12, 64, 4, 4, 16, 48, 8, "f32")
    w = synth.random_weights(shape, seed=20, std=0.1)
    wr = dict(w, rope_theta=10000.0)
    x = synth.random_hidden(shape, seed=21)
    k_plain, _ = oracle.kv_project(x, w, shape.head_dim, 1e-6, "f64")
    k_rot, _ = oracle.kv_project(x, wr, shape.head_dim, 1e-6, "f64")
    want = oracle.rope(k_plain[0].transpose(1, 0, 2), np.arange(shape.n_tokens), 10000.0).transpose(1, 0, 2)
    assert np.allclose(k_rot[0], want, rtol=1e-12, atol=1e-12)
    cache = oracle.LayerCache(k_plain * 0, k_plain * 0, x, np.zeros((1, 12, 8)))
    upd = oracle.sparse_update(x, wr, cache, np.array([[3, 7]]), shape.head_dim, 1e-6, "f64")
    assert np.allclose(upd.k[0][:, [3, 7]], k_rot[0][:, [3, 7]], rtol=1e-12, atol=1e-12)
