"""Plain CPU oracle of the SPA-Cache per-layer decoding step (NumPy, float64).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU-baseline leg use this
module. The HIP library never imports, links or calls it, and this module imports nothing from the
HIP path: the two share no kernels, headers, helpers or constants. It is deliberately slow and
literal: every function follows one passage of the pages, in their order and notation, with no
blocking, fusion or reordering beyond what that passage states.

Sources (pages on "SPA-Cache: Singular Proxies for Adaptive Caching in Diffusion Language Models",
arXiv 2602.02544):
  [PN]  papernotes.org notes (ICML 2026). Sections used: "方法详解 / 整体框架" (Algorithm 1's three
        phases), "关键设计 2: 奇异代理" (W_r = Lambda_r V_r^T and the Theorem 3.4 bound),
        "关键设计 3: 分段高斯自适应预算" (the rho(l) equation).
  [GS]  gist.science technical summary, "Methodology: SPA-Cache", parts 1 (singular proxy),
        2 (adaptive budget) and 3 (sparse execution).

Readings where the pages are silent (each listed in the design notes of the repository):
  * The block is a pre-norm LLaMA-style layer: RMSNorm -> QKV -> bidirectional SDPA -> W_o ->
    residual -> RMSNorm -> SwiGLU FFN -> residual. By default no RoPE and no biases (the pages name
    neither). Optionally, for fidelity to the real architectures (the weights dict carries
    "rope_theta" and/or "b_q", "b_k", "b_v"): biases are added to q, k, v, then q and k of every
    head get the rotary position embedding at the token's index in its sequence, in the
    adjacent-pair form (dims 2j and 2j + 1 rotate by pos * theta^(-2j / head_dim)); K^c caches
    the rotated keys. A checkpoint written in the half-split pairing converts to this one by a fixed
    permutation of each head's rows of W_q and W_k (and b_q, b_k), which leaves every q . k unchanged.
  * The proxy reads the raw layer input h ([PN] Phase 1 feeds the input hidden state to the
    projection); the attention RMSNorm gain is folded into W_r, and the row scale of RMSNorm drops
    out of the cosine.
  * Cosine uses max(||p||, 1e-8) in each denominator, so a zero proxy scores 0.
  * Top-k picks the k smallest under the total order (key(s), index): NaN sorts below -inf
    (always recomputed), -0 equals +0, equal scores go to the lower index. Output is ascending.
  * rho(l): the right branch mirrors the printed left one with rho_L and (L - l_p) in place of
    rho_1 and (l_p - 1); layers are 1-based; k_l = clamp(floor(N rho(l) + 1e-9), 1, N).
  * Scatter K/V into the cache first, then attend (the [PN] Phase 2 order).
  * Storage rounding (bf16 round-to-nearest-even, or fp32) applies where a value is written to a
    cache (K^c, V^c, H^c; P^c is fp32); every other intermediate stays float64.

Parity status: every function below is pinned by a CPU test (tests/test_oracle_*.py) against a
closed form, a library routine, brute force, or an invariant the pages fix. None is unpinned.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "round_bf16", "store", "budget", "singular_proxy", "proxy", "cosine", "order_key",
    "select_topk", "rmsnorm", "silu", "rope", "attention", "full_layer", "kv_project", "warmup", "sparse_update",
    "cached_layer_step", "LayerCache", "POLICY_ALL", "POLICY_SELECTED",
]

POLICY_ALL = 0
POLICY_SELECTED = 1
COS_EPS = 1e-8


# ----------------------------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------------------------
def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each element, returned as float64.

    bfloat16 is the upper half of an IEEE binary32: round to binary32 first, then drop 16 bits
    with round-to-nearest-even on the dropped half. NaN stays NaN.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(np.float32).copy()
    out[np.isnan(x32)] = np.float32("nan")
    return out.astype(np.float64)


def store(x, dtype: str) -> np.ndarray:
    """Round to the storage dtype ("bf16", "f32", or "f64" = exact) and return float64."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return np.array(x, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------------
# [PN] 关键设计 3 / [GS] part 2: piecewise-Gaussian per-layer budget
# ----------------------------------------------------------------------------------------------
def budget(n_layers: int, l_peak: int, rho_peak: float, rho_first: float, rho_last: float,
           n_tokens: int) -> Tuple[np.ndarray, np.ndarray]:
    """rho(l) for l = 1..L and the per-layer row budget k_l = clamp(floor(N rho(l) + 1e-9), 1, N).

    Left branch (l <= l_p), as printed:  rho_p * exp(ln(rho_1/rho_p) * ((l - l_p)/(l_p - 1))^2).
    Right branch (l > l_p), the mirror:  rho_p * exp(ln(rho_L/rho_p) * ((l - l_p)/(L - l_p))^2).
    The peak and the two endpoints are returned exactly.
    """
    if not (n_layers >= 1 and 1 <= l_peak <= n_layers and n_tokens >= 1):
        raise ValueError("bad layer/token counts")
    for v in (rho_peak, rho_first, rho_last):
        if not (0.0 < v <= 1.0):
            raise ValueError("budgets must lie in (0, 1]")
    rho = np.empty(n_layers, dtype=np.float64)
    for l in range(1, n_layers + 1):
        if l == l_peak:
            val = rho_peak
        elif l < l_peak:
            t = (l - l_peak) / (l_peak - 1)
            val = rho_peak * math.exp(math.log(rho_first / rho_peak) * t * t)
            if l == 1:
                val = rho_first
        else:
            t = (l - l_peak) / (n_layers - l_peak)
            val = rho_peak * math.exp(math.log(rho_last / rho_peak) * t * t)
            if l == n_layers:
                val = rho_last
        rho[l - 1] = val
    k = np.array([min(max(int(math.floor(n_tokens * r + 1e-9)), 1), n_tokens) for r in rho],
                 dtype=np.int32)
    return rho, k


# ----------------------------------------------------------------------------------------------
# [PN] 关键设计 2 / [GS] part 1: the singular proxy
# ----------------------------------------------------------------------------------------------
def singular_proxy(w_v: np.ndarray, g_attn: Optional[np.ndarray], r: int) -> np.ndarray:
    """W_r = Lambda_r V_r^T from the SVD W = U Lambda V^T of the Value projection (r x d).

    The Value projection sees rmsnorm(h) * g, so the gain is folded in first: W = W_v diag(g).
    """
    w = np.asarray(w_v, dtype=np.float64)
    if g_attn is not None:
        w = w * np.asarray(g_attn, dtype=np.float64)[None, :]
    _, lam, vt = np.linalg.svd(w, full_matrices=False)
    if not (1 <= r <= lam.shape[0]):
        raise ValueError("rank out of range")
    return lam[:r, None] * vt[:r, :]


def proxy(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """f_proxy(h_i) = W_r h_i for every row of x (..., d) -> (..., r)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64).T


def cosine(p: np.ndarray, pc: np.ndarray, eps: float = COS_EPS) -> np.ndarray:
    """Cosine similarity of each row of p with the same row of the cached proxy pc, as float32."""
    p = np.asarray(p, dtype=np.float64)
    pc = np.asarray(pc, dtype=np.float64)
    dot = np.sum(p * pc, axis=-1)
    n1 = np.maximum(np.sqrt(np.sum(p * p, axis=-1)), eps)
    n2 = np.maximum(np.sqrt(np.sum(pc * pc, axis=-1)), eps)
    return (dot / (n1 * n2)).astype(np.float32)


def order_key(s: np.ndarray) -> np.ndarray:
    """Unsigned 32-bit key whose integer order is the float order of s, with NaN lowest and -0 = +0."""
    s32 = np.array(s, dtype=np.float32, copy=True)
    s32[s32 == 0] = np.float32(0.0)
    u = s32.view(np.uint32).astype(np.uint64)
    neg = (u & np.uint64(0x80000000)) != 0
    key = np.where(neg, (~u) & np.uint64(0xFFFFFFFF), u | np.uint64(0x80000000))
    key[np.isnan(s32)] = 0
    return key.astype(np.uint32)


def select_topk(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k least similar tokens of one sequence, ascending (int32)."""
    s = np.asarray(s, dtype=np.float32)
    n = s.shape[0]
    if not (0 <= k <= n):
        raise ValueError("k out of range")
    order = np.lexsort((np.arange(n), order_key(s)))
    return np.sort(order[:k]).astype(np.int32)


# ----------------------------------------------------------------------------------------------
# the transformer block (pre-norm, SwiGLU, bidirectional attention)
# ----------------------------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray) -> np.ndarray:
    """Exact softmax attention of queries q (M, H_q, hd) over every cached key of one sequence.

    k_cache, v_cache: (H_kv, N, hd). Query head h reads KV head floor(h H_kv / H_q). No mask: the
    model is non-causal. Returns (M, H_q * hd).
    """
    m, hq, hd = q.shape
    hkv = k_cache.shape[0]
    out = np.empty((m, hq, hd), dtype=np.float64)
    for h in range(hq):
        g = (h * hkv) // hq
        s = (q[:, h, :] @ k_cache[g].T) / math.sqrt(hd)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        out[:, h, :] = (e / e.sum(axis=1, keepdims=True)) @ v_cache[g]
    return out.reshape(m, hq * hd)


class LayerCache:
    """Per-layer cache of one batch: K^c, V^c (B, H_kv, N, hd), H^c (B, N, d), P^c (B, N, r) fp32."""

    def __init__(self, k, v, h, p):
        self.k = np.array(k, dtype=np.float64)
        self.v = np.array(v, dtype=np.float64)
        self.h = np.array(h, dtype=np.float64)
        self.p = np.array(p, dtype=np.float64)

    def copy(self) -> "LayerCache":
        return LayerCache(self.k, self.v, self.h, self.p)


def _heads(w: Dict[str, np.ndarray], hd: int):
    hq = w["w_q"].shape[0] // hd
    hkv = w["w_k"].shape[0] // hd
    return hq, hkv


def rope(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """Rotary position embedding of x (n, heads, head_dim) at integer positions (n,): the pair of
    dims (2j, 2j + 1) of every head rotates by the angle pos * theta^(-2j / head_dim)."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    inv = float(theta) ** (-2.0 * np.arange(hd // 2, dtype=np.float64) / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None, None] * inv[None, None, :]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def _qkv(a: np.ndarray, w: Dict[str, np.ndarray], positions, head_dim: int):
    """q, k, v of normalised rows a (n, d) at the given sequence positions: projections, the
    optional biases, then the optional RoPE on q and k. Returns (n, heads, head_dim) arrays."""
    n = a.shape[0]
    hq, hkv = _heads(w, head_dim)
    q = a @ np.asarray(w["w_q"], np.float64).T
    k = a @ np.asarray(w["w_k"], np.float64).T
    v = a @ np.asarray(w["w_v"], np.float64).T
    if "b_q" in w:
        q = q + np.asarray(w["b_q"], np.float64)
        k = k + np.asarray(w["b_k"], np.float64)
        v = v + np.asarray(w["b_v"], np.float64)
    q = q.reshape(n, hq, head_dim)
    k = k.reshape(n, hkv, head_dim)
    v = v.reshape(n, hkv, head_dim)
    theta = float(w.get("rope_theta", 0.0))
    if theta > 0.0:
        q = rope(q, positions, theta)
        k = rope(k, positions, theta)
    return q, k, v


def full_layer(x: np.ndarray, w: Dict[str, np.ndarray], head_dim: int, eps: float,
               dtype: str = "f64"):
    """Full forward of the block over every token of every sequence (vanilla decoding).

    This is the plain definition, written over whole sequences: K/V of all N tokens, N x N
    attention, FFN on all rows. Returns (K^c, V^c, H) with caches rounded to `dtype`.
    """
    x = np.asarray(x, dtype=np.float64)
    b, n, d = x.shape
    hq, hkv = _heads(w, head_dim)
    kc = np.empty((b, hkv, n, head_dim))
    vc = np.empty((b, hkv, n, head_dim))
    hc = np.empty((b, n, d))
    for bi in range(b):
        a = rmsnorm(x[bi], w["g_attn"], eps)
        q, k, v = _qkv(a, w, np.arange(n), head_dim)
        kc[bi] = store(k.transpose(1, 0, 2), dtype)
        vc[bi] = store(v.transpose(1, 0, 2), dtype)
        o = attention(q, kc[bi], vc[bi])
        y = x[bi] + o @ np.asarray(w["w_o"], np.float64).T
        bb = rmsnorm(y, w["g_ffn"], eps)
        z = silu(bb @ np.asarray(w["w_gate"], np.float64).T) * (bb @ np.asarray(w["w_up"], np.float64).T)
        hc[bi] = store(y + z @ np.asarray(w["w_down"], np.float64).T, dtype)
    return kc, vc, hc


def kv_project(x: np.ndarray, w: Dict[str, np.ndarray], head_dim: int, eps: float, dtype: str = "f64"):
    """K and V of every token (the cache contents a full forward leaves), rounded to `dtype`.

    The same arithmetic as the K/V part of full_layer, without the queries, attention and FFN.
    """
    x = np.asarray(x, dtype=np.float64)
    b, n, _ = x.shape
    hkv = w["w_k"].shape[0] // head_dim
    kc = np.empty((b, hkv, n, head_dim))
    vc = np.empty((b, hkv, n, head_dim))
    for bi in range(b):
        a = rmsnorm(x[bi], w["g_attn"], eps)
        _, k, v = _qkv(a, w, np.arange(n), head_dim)
        kc[bi] = store(k.transpose(1, 0, 2), dtype)
        vc[bi] = store(v.transpose(1, 0, 2), dtype)
    return kc, vc


def warmup(x: np.ndarray, w: Dict[str, np.ndarray], w_r: np.ndarray, head_dim: int, eps: float,
           dtype: str = "f64") -> LayerCache:
    """Step t = 0: full recompute fills K^c, V^c, H^c, and the proxy cache P^c = X W_r^T (fp32)."""
    kc, vc, hc = full_layer(x, w, head_dim, eps, dtype)
    pc = proxy(x, w_r).astype(np.float32).astype(np.float64)
    return LayerCache(kc, vc, hc, pc)


def sparse_update(x: np.ndarray, w: Dict[str, np.ndarray], cache: LayerCache, idx: np.ndarray,
                  head_dim: int, eps: float, dtype: str = "f64") -> LayerCache:
    """Phases 2 and 3 of [PN] 整体框架 for given index sets idx (B, k); returns the updated cache.

    Phase 2: Q_I, K_I, V_I for the rows in I only; K_I, V_I scattered into K^c, V^c; then the k
    sparse queries attend to the whole (just updated) cache. Phase 3: the FFN runs on those k rows
    and the block output is scattered into H^c[I]; rows outside I keep their cached values.
    """
    x = np.asarray(x, dtype=np.float64)
    out = cache.copy()
    b = x.shape[0]
    hq, hkv = _heads(w, head_dim)
    for bi in range(b):
        I = np.asarray(idx[bi], dtype=np.int64)
        if I.size == 0:
            continue
        xi = x[bi, I]
        a = rmsnorm(xi, w["g_attn"], eps)
        q, k, v = _qkv(a, w, I, head_dim)
        out.k[bi][:, I, :] = store(k.transpose(1, 0, 2), dtype)
        out.v[bi][:, I, :] = store(v.transpose(1, 0, 2), dtype)
        o = attention(q, out.k[bi], out.v[bi])
        y = xi + o @ np.asarray(w["w_o"], np.float64).T
        bb = rmsnorm(y, w["g_ffn"], eps)
        z = silu(bb @ np.asarray(w["w_gate"], np.float64).T) * (bb @ np.asarray(w["w_up"], np.float64).T)
        out.h[bi][I] = store(y + z @ np.asarray(w["w_down"], np.float64).T, dtype)
    return out


def identify(x: np.ndarray, w_r: np.ndarray, p_cache: np.ndarray):
    """Phase 1 scores: the proxy of every token and its cosine against the cached proxy.
    Returns (P as fp32 values in float64, s float32 (B, N))."""
    p = proxy(x, w_r)
    s = cosine(p, p_cache)
    return p.astype(np.float32).astype(np.float64), s


def cached_layer_step(x: np.ndarray, w: Dict[str, np.ndarray], w_r: np.ndarray, cache: LayerCache,
                      k: int, head_dim: int, eps: float, dtype: str = "f64",
                      policy: int = POLICY_ALL):
    """One SPA-Cache layer step at t >= 1 ([PN] 整体框架, phases 1-3).

    Phase 1: proxies of all tokens, cosine against the cached proxies, the k least similar tokens.
    The proxy cache then takes the new proxies (policy ALL: every row; SELECTED: rows in I).
    Phases 2-3: sparse_update on I. Returns (new cache, I (B, k) int32, s (B, N) float32).
    """
    b = x.shape[0]
    p, s = identify(x, w_r, cache.p)
    idx = np.stack([select_topk(s[bi], k) for bi in range(b)]) if k > 0 else np.zeros((b, 0), np.int32)
    new = sparse_update(x, w, cache, idx, head_dim, eps, dtype)
    if policy == POLICY_ALL:
        new.p = p.copy()
    elif policy == POLICY_SELECTED:
        for bi in range(b):
            new.p[bi][idx[bi]] = p[bi][idx[bi]]
    else:
        raise ValueError("policy")
    return new, idx, s
