"""Pins of the oracle's transformer block pieces against independent library routines.

torch.nn.functional (CPU, float64) supplies RMSNorm, SiLU, scaled-dot-product attention and linear
layers; the oracle is written with NumPy only. Also pins the bf16 rounding against torch's cast.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9, 3.0e38, -1e-40]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x)
    assert np.array_equal(got, ref)
    assert np.isnan(oracle.round_bf16(np.array([np.nan]))[0])


def test_rmsnorm_and_silu_match_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 40)) * 3
    g = rng.uniform(0.5, 1.5, 40)
    ref = F.rms_norm(t64(x), (40,), weight=t64(g), eps=1e-6).numpy()
    assert np.allclose(oracle.rmsnorm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-13)
    u = rng.standard_normal(1000) * 20
    assert np.allclose(oracle.silu(u), F.silu(t64(u)).numpy(), rtol=1e-13, atol=1e-13)
    c = np.full((1, 16), -2.5)     # constant row: rmsnorm is sign(c) * g
    assert np.allclose(oracle.rmsnorm(c, np.ones(16), 0.0), -1.0, atol=1e-15)


@pytest.mark.parametrize("hq,hkv,hd,n,m", [(4, 4, 16, 37, 5), (8, 2, 32, 64, 64), (7, 1, 8, 10, 3)])
def test_attention_matches_sdpa(hq, hkv, hd, n, m):
    rng = np.random.default_rng(hq * 100 + n)
    q = rng.standard_normal((m, hq, hd))
    kc = rng.standard_normal((hkv, n, hd))
    vc = rng.standard_normal((hkv, n, hd))
    got = oracle.attention(q, kc, vc)
    kk = t64(kc).repeat_interleave(hq // hkv, dim=0)       # (hq, n, hd): head h reads h // (hq/hkv)
    vv = t64(vc).repeat_interleave(hq // hkv, dim=0)
    ref = F.scaled_dot_product_attention(t64(q).transpose(0, 1), kk, vv).transpose(0, 1).reshape(m, hq * hd)
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_brute_force_loops():
    rng = np.random.default_rng(3)
    hq, hkv, hd, n, m = 4, 2, 3, 5, 2
    q = rng.standard_normal((m, hq, hd))
    kc = rng.standard_normal((hkv, n, hd))
    vc = rng.standard_normal((hkv, n, hd))
    got = oracle.attention(q, kc, vc).reshape(m, hq, hd)
    for i in range(m):
        for h in range(hq):
            g = h // (hq // hkv)
            w = [math.exp(sum(q[i, h, c] * kc[g, j, c] for c in range(hd)) / math.sqrt(hd)) for j in range(n)]
            tot = sum(w)
            for c in range(hd):
                assert abs(got[i, h, c] - sum(w[j] * vc[g, j, c] for j in range(n)) / tot) < 1e-12


def torch_block(x, w, hd, eps):
    """The same pre-norm SwiGLU block composed from torch.nn.functional (float64)."""
    x = t64(x)
    hq = w["w_q"].shape[0] // hd
    hkv = w["w_k"].shape[0] // hd
    b, n, d = x.shape
    a = F.rms_norm(x, (d,), weight=t64(w["g_attn"]), eps=eps)
    q = F.linear(a, t64(w["w_q"])).view(b, n, hq, hd).transpose(1, 2)
    k = F.linear(a, t64(w["w_k"])).view(b, n, hkv, hd).transpose(1, 2)
    v = F.linear(a, t64(w["w_v"])).view(b, n, hkv, hd).transpose(1, 2)
    o = F.scaled_dot_product_attention(q, k.repeat_interleave(hq // hkv, 1), v.repeat_interleave(hq // hkv, 1))
    y = x + F.linear(o.transpose(1, 2).reshape(b, n, hq * hd), t64(w["w_o"]))
    bb = F.rms_norm(y, (d,), weight=t64(w["g_ffn"]), eps=eps)
    h = y + F.linear(F.silu(F.linear(bb, t64(w["w_gate"]))) * F.linear(bb, t64(w["w_up"])), t64(w["w_down"]))
    return k.numpy(), v.numpy(), h.numpy()


@pytest.mark.parametrize("shape", [
    synth.LayerShape(2, 24, 64, 4, 4, 16, 96, 8, "f32"),
    synth.LayerShape(1, 33, 96, 6, 2, 16, 80, 8, "f32"),
])
def test_full_layer_matches_torch_composition(shape):
    w = synth.random_weights(shape, seed=5, std=0.1, gains="random")
    x = synth.random_hidden(shape, seed=6)
    kc, vc, h = oracle.full_layer(x, w, shape.head_dim, 1e-6, "f64")
    rk, rv, rh = torch_block(x, w, shape.head_dim, 1e-6)
    assert np.allclose(kc, rk, rtol=1e-12, atol=1e-12)
    assert np.allclose(vc, rv, rtol=1e-12, atol=1e-12)
    assert np.allclose(h, rh, rtol=1e-12, atol=1e-12)


def test_kv_project_matches_full_layer():
    shape = synth.LayerShape(2, 19, 64, 4, 2, 16, 48, 8, "f32")
    w = synth.random_weights(shape, seed=8, std=0.1, gains="random")
    x = synth.random_hidden(shape, seed=9)
    for dtype in ("f64", "bf16"):
        kc, vc, _ = oracle.full_layer(x, w, shape.head_dim, 1e-6, dtype)
        k2, v2 = oracle.kv_project(x, w, shape.head_dim, 1e-6, dtype)
        assert np.array_equal(kc, k2) and np.array_equal(vc, v2)
