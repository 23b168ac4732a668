"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bars: Top-k index sets bit-exact given identical scores; proxy similarities within 1e-3 absolute;
block outputs (rows of the update set of H^c, K^c, V^c) within 2e-2 relative L2 in bf16 and 1e-5 in
fp32; rows outside the update set bit-identical to the cache before the step. In end-to-end steps
the GPU's own index set may differ from the oracle's only by near-ties (scores within 2e-3 of the
k-th boundary); the block outputs are then checked against the oracle's update on the GPU's set.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import check_near_ties, dev, has_gpu, host, rel_l2, tol_for
from parity_cases import (ATTEND_CASES, ATTEND_MANY_CASES, BATCHED_EXACT_RHO, BATCHED_ID_RANKS, DREAM_STACK_K,
                          FUSED_TOPK_SHAPES, LLADA_EXACT_K, LLADA_ID_RANKS, RANK_STEP_CASES, ROPE_STEP_CASES,
                          SMALL_BF16, SMALL_STEP_K, fused_topk_ks)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs an MI355X")]

EPS = 1e-6


def _lib():
    import adaptive_hidden_state_amd as spa
    spa.load_library()
    return spa


class Case:
    """Weights, W_r, X^0 -> X^1 and the oracle's warm-up cache for one shape (host side)."""

    def __init__(self, shape, seed, n_drift, std=0.1, gains="random", warm="full"):
        self.shape = shape
        self.w = synth.random_weights(shape, seed=seed, std=std, gains=gains)
        self.w_r = synth.to_storage(oracle.singular_proxy(self.w["w_v"], self.w["g_attn"], shape.rank), shape.dtype)
        self.x0 = synth.random_hidden(shape, seed=seed + 1)
        rng = np.random.default_rng([77, seed])
        self.x1, self.drifted = synth.drift_step(self.x0, n_drift, rng, shape.dtype)
        st = shape.dtype
        if warm == "full":
            self.cache0 = oracle.warmup(self.x0, self.w, self.w_r, shape.head_dim, EPS, st)
        else:   # K/V of every token, H^c = X^0 (any cache state is a valid step input)
            kc, vc = oracle.kv_project(self.x0, self.w, shape.head_dim, EPS, st)
            pc = oracle.proxy(self.x0, self.w_r).astype(np.float32).astype(np.float64)
            self.cache0 = oracle.LayerCache(kc, vc, np.asarray(self.x0, np.float64), pc)

    def device(self):
        spa = _lib()
        s = self.shape
        w = spa.upload_weights(self.w, self.w_r, s.dtype)
        import torch
        c = spa.DeviceCache(dev(self.cache0.k, s.dtype), dev(self.cache0.v, s.dtype), dev(self.cache0.h, s.dtype),
                            torch.from_numpy(self.cache0.p.astype(np.float32)).cuda())
        return w, c


def _slice(cache, sel):
    return oracle.LayerCache(cache.k[sel], cache.v[sel], cache.h[sel], cache.p[sel])


def _check_step(case, k, policy=oracle.POLICY_ALL, seqs=None, exact=False):
    """One cached step on the GPU against the oracle. Scores, the proxy cache and the untouched rows
    are checked for every sequence; block outputs for the sequences in `seqs` (default: all). The
    oracle only ever sees host inputs: when the GPU's set differs from the oracle's by near-ties,
    the GPU's phases 2-3 are re-run on the oracle's set (spa_sparse_update) and compared with that.
    exact=True: the inputs leave no near-tie at the k-th boundary, so the GPU's set must equal the
    oracle's in every sequence and the step's own block outputs are the ones compared."""
    import torch
    spa = _lib()
    s = case.shape
    sel = list(range(s.batch)) if seqs is None else list(seqs)
    w, c = case.device()
    x1 = dev(case.x1, s.dtype)
    idx = torch.empty(s.batch, k, dtype=torch.int32, device="cuda")
    scores = torch.empty(s.batch, s.n_tokens, dtype=torch.float32, device="cuda")
    ws = spa.alloc_workspace(s, max(k, 1))
    spa.spa_layer_step(s, w, c, x1, k, policy, idx, scores, ws)
    torch.cuda.synchronize()

    p_new, s_o = oracle.identify(case.x1, case.w_r, case.cache0.p)
    idx_o = np.stack([oracle.select_topk(s_o[b], k) for b in range(s.batch)]) if k else np.zeros((s.batch, 0), int)
    s_g = host(scores)
    assert np.max(np.abs(s_g - s_o)) <= 1e-3
    i_g = host(idx).astype(np.int64)
    same = True
    for b in range(s.batch):
        if exact and k:
            assert np.array_equal(i_g[b], idx_o[b]), f"sequence {b}: the update set differs from the oracle's"
        if k and check_near_ties(i_g[b], idx_o[b], s_o[b], k):
            same = same and b not in sel
    hk, hv, hh, hp = host(c.k), host(c.v), host(c.h), host(c.p)
    # proxy cache: every row (ALL) or the rows of the step's set (SELECTED) take the new proxy
    for b in range(s.batch):
        take = np.ones(s.n_tokens, bool) if policy == oracle.POLICY_ALL else np.isin(np.arange(s.n_tokens), i_g[b])
        exp_p = np.where(take[:, None], p_new[b], case.cache0.p[b])
        assert rel_l2(hp[b], exp_p) <= 1e-5, b
        rest = np.setdiff1d(np.arange(s.n_tokens), i_g[b])
        assert np.array_equal(hh[b][rest], case.cache0.h[b][rest])
        assert np.array_equal(hk[b][:, rest], case.cache0.k[b][:, rest])
        assert np.array_equal(hv[b][:, rest], case.cache0.v[b][:, rest])
    if not k:
        return i_g, s_g
    if not same:   # near-tie swaps in a checked sequence: the GPU's phases 2-3 on the oracle's set
        w, c = case.device()
        spa.spa_sparse_update(s, w, c, x1, torch.from_numpy(idx_o.astype(np.int32)).cuda(), ws)
        torch.cuda.synchronize()
        hk, hv, hh = host(c.k), host(c.v), host(c.h)
    ref = oracle.sparse_update(case.x1[sel], case.w, _slice(case.cache0, sel), idx_o[sel], s.head_dim, EPS, s.dtype)
    tol = tol_for(s.dtype)
    for j, b in enumerate(sel):
        I = idx_o[b]
        errs = {"H": rel_l2(hh[b][I], ref.h[j][I]), "K": rel_l2(hk[b][:, I], ref.k[j][:, I]),
                "V": rel_l2(hv[b][:, I], ref.v[j][:, I])}
        assert max(errs.values()) <= tol, (b, errs)
    return i_g, s_g


@pytest.mark.parametrize("shape_i", [0, 1])
@pytest.mark.parametrize("k", SMALL_STEP_K)
def test_layer_step_small_bf16(shape_i, k):
    shape = SMALL_BF16[shape_i]
    case = Case(shape, seed=10 + shape_i, n_drift=min(60, shape.n_tokens // 3))
    _check_step(case, k)


def test_layer_step_tiny_f32_config():
    wl = synth.WORKLOADS["tiny-f32"]
    s = wl.shape
    case = Case(s, seed=3, n_drift=13, std=0.02, gains="ones")
    i_g, _ = _check_step(case, 16)
    assert set(case.drifted[0].tolist()) <= set(i_g[0].tolist())


def test_layer_step_policy_selected():
    case = Case(SMALL_BF16[0], seed=21, n_drift=50)
    _check_step(case, 40, oracle.POLICY_SELECTED)


def test_layer_step_k_zero_and_all():
    import torch
    spa = _lib()
    case = Case(SMALL_BF16[0], seed=31, n_drift=30)
    s = case.shape
    # k = 0: scores and the proxy cache change, nothing else does
    w, c = case.device()
    scores = torch.empty(s.batch, s.n_tokens, dtype=torch.float32, device="cuda")
    ws = spa.alloc_workspace(s, 0)
    spa.spa_layer_step(s, w, c, dev(case.x1, s.dtype), 0, 0, None, scores, ws)
    torch.cuda.synchronize()
    _, s_o = oracle.identify(case.x1, case.w_r, case.cache0.p)
    assert np.max(np.abs(host(scores) - s_o)) <= 1e-3
    assert np.array_equal(host(c.h), case.cache0.h) and np.array_equal(host(c.k), case.cache0.k)
    # k = N: every row recomputed
    _check_step(case, s.n_tokens)


@pytest.mark.parametrize("shape_i", [0, 1])
def test_layer_full_matches_oracle_warmup(shape_i):
    import torch
    spa = _lib()
    s = SMALL_BF16[shape_i]
    case = Case(s, seed=40 + shape_i, n_drift=10)
    w, _ = case.device()
    c = spa.alloc_cache(s)
    ws = spa.alloc_workspace(s, s.n_tokens)
    spa.spa_layer_full(s, w, c, dev(case.x1, s.dtype), ws)
    torch.cuda.synchronize()
    ref = oracle.warmup(case.x1, case.w, case.w_r, s.head_dim, EPS, s.dtype)
    assert rel_l2(host(c.k), ref.k) <= 2e-2
    assert rel_l2(host(c.v), ref.v) <= 2e-2
    assert rel_l2(host(c.h), ref.h) <= 2e-2
    assert rel_l2(host(c.p), ref.p) <= 1e-5


def test_rho_one_step_equals_full_on_gpu():
    """k = N through the cached path equals the full recompute through spa_layer_full (both GPU)."""
    import torch
    spa = _lib()
    s = SMALL_BF16[1]
    case = Case(s, seed=50, n_drift=30)
    w, c = case.device()
    x1 = dev(case.x1, s.dtype)
    idx = torch.empty(s.batch, s.n_tokens, dtype=torch.int32, device="cuda")
    spa.spa_layer_step(s, w, c, x1, s.n_tokens, 0, idx, None, spa.alloc_workspace(s, s.n_tokens))
    c2 = spa.alloc_cache(s)
    spa.spa_layer_full(s, w, c2, x1, spa.alloc_workspace(s, s.n_tokens))
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), torch.arange(s.n_tokens, dtype=torch.int32).expand(s.batch, -1))
    for a, b in ((c.k, c2.k), (c.v, c2.v), (c.h, c2.h), (c.p, c2.p)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("b,n", [(1, 1), (3, 64), (2, 1000), (1, 1024), (2, 1025), (1, 2048), (2, 3000), (1, 4096),
                                 (1, 4097), (2, 16384)])
def test_topk_bit_exact(b, n):
    import torch
    spa = _lib()
    rng = np.random.default_rng(n)
    s = rng.uniform(0.9, 1.0, (b, n)).astype(np.float32)
    s[rng.random((b, n)) < 0.3] = np.float32(0.99)                       # heavy ties
    specials = np.array([np.nan, -0.0, 0.0, -np.inf, np.inf, -1.0], np.float32)
    mask = rng.random((b, n)) < 0.02
    s[mask] = rng.choice(specials, mask.sum())
    st = torch.from_numpy(s).cuda()
    for k in sorted({0, 1, n // 7, n // 2, n - 1, n} - {-1}):
        if k < 0:
            continue
        out = torch.full((b, max(k, 1)), -1, dtype=torch.int32, device="cuda")
        spa.spa_topk(st, k, out[:, :k] if k else None)
        torch.cuda.synchronize()
        got = out.cpu().numpy()[:, :k]
        for bi in range(b):
            assert got[bi].tolist() == oracle.select_topk(s[bi], k).tolist(), (bi, k)


@pytest.mark.parametrize("shape", FUSED_TOPK_SHAPES)
def test_layer_step_fused_topk_equals_spa_topk(shape):
    """The Top-k taken inside the cosine kernel of spa_layer_step (by the workgroup that completes each
    sequence) equals spa_topk on the scores that step returns, and the oracle's selection on them:
    sequences whose tokens share workgroups (N % 8 != 0, N < 8), and the four key-per-thread sizes of
    the fused path (2, 4, 8, 16 keys per thread: N up to 1024, 2048, 4096, 8192)."""
    import torch
    spa = _lib()
    s = shape
    case = Case(s, seed=80 + s.n_tokens, n_drift=max(1, s.n_tokens // 5), warm="kv")
    w, c = case.device()
    x1 = dev(case.x1, s.dtype)
    for k in fused_topk_ks(s.n_tokens):
        idx = torch.full((s.batch, k), -1, dtype=torch.int32, device="cuda")
        scores = torch.empty(s.batch, s.n_tokens, dtype=torch.float32, device="cuda")
        spa.spa_layer_step(s, w, c, x1, k, 0, idx, scores, spa.alloc_workspace(s, k))
        ref = torch.full((s.batch, k), -2, dtype=torch.int32, device="cuda")
        spa.spa_topk(scores, k, ref)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref), k
        sc = host(scores)
        for b in range(s.batch):
            assert host(idx)[b].tolist() == oracle.select_topk(sc[b], k).tolist(), (b, k)


@pytest.mark.parametrize("shape", [synth.WORKLOADS["tiny-f32"].shape, SMALL_BF16[0], SMALL_BF16[1]])
def test_identify_scores_and_proxy(shape):
    import torch
    spa = _lib()
    case = Case(shape, seed=60, n_drift=shape.n_tokens // 4)
    s = shape
    p_out = torch.empty(s.batch, s.n_tokens, s.rank, dtype=torch.float32, device="cuda")
    scores = torch.empty(s.batch, s.n_tokens, dtype=torch.float32, device="cuda")
    pc = torch.from_numpy(case.cache0.p.astype(np.float32)).cuda()
    w_r = spa.spa_pack_weight(dev(case.w_r, s.dtype))
    spa.spa_identify(s, dev(case.x1, s.dtype), w_r, pc, p_out, scores, spa.alloc_workspace(s, 0))
    torch.cuda.synchronize()
    p_o, s_o = oracle.identify(case.x1, case.w_r, case.cache0.p)
    assert np.max(np.abs(host(scores) - s_o)) <= 1e-3
    assert rel_l2(host(p_out), p_o) <= 1e-5
    assert np.array_equal(host(pc), case.cache0.p)        # identify never writes the cache


def _rope_bias_case(shape, seed, n_drift, bias=True):
    """A Case whose layer has q/k/v biases (N(0, 0.1^2)) and the rotary embedding of the shape."""
    case = Case(shape, seed=seed, n_drift=n_drift, warm="kv")
    rng = np.random.default_rng([96, seed])
    if bias:
        for key, n in (("b_q", shape.d_q), ("b_k", shape.d_kv), ("b_v", shape.d_kv)):
            case.w[key] = synth.to_storage(rng.standard_normal(n) * 0.1, shape.dtype)
    case.w["rope_theta"] = shape.rope_theta
    kc, vc = oracle.kv_project(case.x0, case.w, shape.head_dim, EPS, shape.dtype)
    case.cache0 = oracle.LayerCache(kc, vc, np.asarray(case.x0, np.float64), case.cache0.p)
    return case


@pytest.mark.parametrize("shape,k", ROPE_STEP_CASES)
def test_layer_step_rope_and_biases(shape, k):
    """Cached steps of layers with q/k/v biases and the rotary embedding (GQA, ragged N, fp32)."""
    _check_step(_rope_bias_case(shape, 70, shape.n_tokens // 5), k)


@pytest.mark.timeout(600)
def test_layer_step_rope_large_positions():
    """Positions up to 8191 (the fp32 angle pos * theta^(-2j/hd) at its largest), no biases."""
    s = synth.LayerShape(1, 8192, 256, 4, 4, 64, 688, 32, "bf16", rope_theta=1e4)
    _check_step(_rope_bias_case(s, 71, 400, bias=False), 64)


def test_layer_full_rope_and_biases():
    import torch
    spa = _lib()
    s = synth.LayerShape(2, 150, 512, 8, 2, 64, 1024, 32, "bf16", rope_theta=5e5)
    case = _rope_bias_case(s, 72, 30)
    w, _ = case.device()
    c = spa.alloc_cache(s)
    spa.spa_layer_full(s, w, c, dev(case.x1, s.dtype), spa.alloc_workspace(s, s.n_tokens))
    torch.cuda.synchronize()
    ref = oracle.warmup(case.x1, case.w, case.w_r, s.head_dim, EPS, s.dtype)
    errs = {"K": rel_l2(host(c.k), ref.k), "V": rel_l2(host(c.v), ref.v), "H": rel_l2(host(c.h), ref.h)}
    assert max(errs.values()) <= 2e-2, errs


@pytest.mark.timeout(600)
def test_dream_layer_step_rope_and_biases_full_size():
    """A full Dream layer (GQA 28/4, N=2048, k=512) with its q/k/v biases and rope_theta = 1e6."""
    wl = synth.WORKLOADS["dream-stack"]
    s = wl.shape.replace(rope_theta=1e6)
    case = Case.__new__(Case)
    case.shape = s
    case.w = synth.layer_weights(wl, layer=9)
    case.w_r = synth.to_storage(oracle.singular_proxy(case.w["w_v"], case.w["g_attn"], s.rank), s.dtype)
    rng = np.random.default_rng([95, 9])
    for key, n in (("b_q", s.d_q), ("b_k", s.d_kv), ("b_v", s.d_kv)):
        case.w[key] = synth.to_storage(rng.standard_normal(n) * 0.1, s.dtype)
    case.w["rope_theta"] = s.rope_theta
    case.x0 = synth.first_hidden(wl, layer=9)
    case.x1, case.drifted = synth.drift_step(case.x0, 600, np.random.default_rng([4, 9, 4]), s.dtype)
    kc, vc = oracle.kv_project(case.x0, case.w, s.head_dim, EPS, s.dtype)
    pc = oracle.proxy(case.x0, case.w_r).astype(np.float32).astype(np.float64)
    case.cache0 = oracle.LayerCache(kc, vc, np.asarray(case.x0, np.float64), pc)
    _check_step(case, 512)

def test_identify_full_value_identifier():
    """The full-dimension Value identifier: W_r = W_v diag(g_attn), r = d_kv = 2048 (past the 1024
    columns a wave covers in one pass), two sequences of a ragged length."""
    import torch
    spa = _lib()
    s = synth.LayerShape(2, 200, 2048, 16, 16, 128, 1024, 2048, "bf16")
    case = Case(s, seed=61, n_drift=50, warm="kv")
    w_r = synth.to_storage(np.asarray(case.w["w_v"], np.float64) * np.asarray(case.w["g_attn"], np.float64)[None, :],
                           s.dtype)
    pc = oracle.proxy(case.x0, w_r).astype(np.float32).astype(np.float64)
    p_out = torch.empty(s.batch, s.n_tokens, s.rank, dtype=torch.float32, device="cuda")
    scores = torch.empty(s.batch, s.n_tokens, dtype=torch.float32, device="cuda")
    pc_d = torch.from_numpy(pc.astype(np.float32)).cuda()
    spa.spa_identify(s, dev(case.x1, s.dtype), spa.spa_pack_weight(dev(w_r, s.dtype)), pc_d, p_out, scores,
                     spa.alloc_workspace(s, 0))
    torch.cuda.synchronize()
    p_o, s_o = oracle.identify(case.x1, w_r, pc)
    assert np.max(np.abs(host(scores) - s_o)) <= 1e-3
    assert rel_l2(host(p_out), p_o) <= 1e-5


@pytest.mark.timeout(600)
def test_layer_step_full_rank_identifier():
    """A cached step whose identifier has the full Value rank (r = d_kv = 2048)."""
    s = synth.LayerShape(1, 256, 2048, 16, 16, 128, 1024, 2048, "bf16")
    _check_step(Case(s, seed=62, n_drift=40, warm="kv"), 64)

def _attend(spa, shape, q, m, kc, vc, dtype):
    """spa_attend of q against the caches; the output on the host."""
    import torch
    o = torch.empty(shape.batch, m, shape.n_q_heads * shape.head_dim,
                    dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    spa.spa_attend(shape, dev(q, dtype), m, dev(kc, dtype), dev(vc, dtype), o)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("dtype,hd,hq,hkv,n,m", ATTEND_CASES)
def test_attend_matches_oracle(dtype, hd, hq, hkv, n, m):
    """spa_attend against the oracle's attention (ragged key tiles and query blocks, GQA, hd 64, fp32)."""
    spa = _lib()
    b = 2
    rng = np.random.default_rng(n + m)
    q = synth.to_storage(rng.standard_normal((b, m, hq, hd)) * 1.5, dtype)
    kc = synth.to_storage(rng.standard_normal((b, hkv, n, hd)), dtype)
    vc = synth.to_storage(rng.standard_normal((b, hkv, n, hd)), dtype)
    shape = synth.LayerShape(b, n, 256, hq, hkv, hd, 256, 16, dtype)
    got = _attend(spa, shape, q, m, kc, vc, dtype)
    for bi in range(b):
        ref = oracle.attention(q[bi].astype(np.float64), kc[bi].astype(np.float64), vc[bi].astype(np.float64))
        assert rel_l2(got[bi], ref) <= tol_for(dtype), rel_l2(got[bi], ref)


@pytest.mark.parametrize("b,hd,hq,hkv,n,m", ATTEND_MANY_CASES)
def test_attend_many_queries_matches_oracle(b, hd, hq, hkv, n, m):
    """Enough packed rows per KV head for the 256-row blocks of the packed kernel (at least 3/4 of a
    round of workgroups): ragged key tiles (333, 100, 2047 keys), ragged last row blocks, GQA groups of 8,
    4 and 7, hd 64."""
    spa = _lib()
    rng = np.random.default_rng([n, m, hq])
    q = synth.to_storage(rng.standard_normal((b, m, hq, hd)) * 1.5, "bf16")
    kc = synth.to_storage(rng.standard_normal((b, hkv, n, hd)), "bf16")
    vc = synth.to_storage(rng.standard_normal((b, hkv, n, hd)), "bf16")
    shape = synth.LayerShape(b, n, 256, hq, hkv, hd, 256, 16, "bf16")
    got = _attend(spa, shape, q, m, kc, vc, "bf16")
    for bi in (0, b - 1):
        ref = oracle.attention(q[bi].astype(np.float64), kc[bi].astype(np.float64), vc[bi].astype(np.float64))
        assert rel_l2(got[bi], ref) <= tol_for("bf16"), rel_l2(got[bi], ref)


def test_three_layer_chain_matches_oracle():
    """Three layers chained as the stack workloads run them (layer l reads layer l-1's H^c; one
    workspace and one index / score buffer shared by the layers): the warm-up chain (spa_layer_full)
    and one cached-step chain (spa_layer_step) against the oracle's chain, layer by layer. k is the
    number of drifted tokens, whose cosines lie far below the rest at every layer (the later layers'
    other input rows are exactly their cached rows), so both sides select the same sets."""
    import torch
    spa = _lib()
    s = synth.LayerShape(2, 200, 256, 4, 4, 64, 688, 32, "bf16")
    L, n_drift = 3, 30
    ws = [synth.random_weights(s, seed=500 + l, std=0.1, gains="random") for l in range(L)]
    wrs = [synth.to_storage(oracle.singular_proxy(w["w_v"], w["g_attn"], s.rank), s.dtype) for w in ws]
    x0 = synth.random_hidden(s, seed=599)
    x1, drifted = synth.drift_step(x0, n_drift, np.random.default_rng([5, 99]), s.dtype)

    caches_o, x = [], x0
    for l in range(L):
        caches_o.append(oracle.warmup(x, ws[l], wrs[l], s.head_dim, EPS, s.dtype))
        x = caches_o[l].h
    dws = [spa.upload_weights(ws[l], wrs[l], s.dtype) for l in range(L)]
    dcs = [spa.alloc_cache(s) for _ in range(L)]
    wsp = spa.alloc_workspace(s, s.n_tokens)
    xd = dev(x0, s.dtype)
    for l in range(L):
        spa.spa_layer_full(s, dws[l], dcs[l], xd, wsp)
        xd = dcs[l].h
    torch.cuda.synchronize()
    warm_h = [host(dcs[l].h) for l in range(L)]
    for l in range(L):
        assert rel_l2(warm_h[l], caches_o[l].h) <= 2e-2, l

    idx = torch.empty(s.batch, n_drift, dtype=torch.int32, device="cuda")
    scores = torch.empty(s.batch, s.n_tokens, dtype=torch.float32, device="cuda")
    got_idx, xd = [], dev(x1, s.dtype)
    for l in range(L):
        spa.spa_layer_step(s, dws[l], dcs[l], xd, n_drift, spa.SPA_PROXY_WRITE_ALL, idx, scores, wsp)
        got_idx.append(host(idx).astype(np.int64))
        xd = dcs[l].h
    torch.cuda.synchronize()

    x = x1
    for l in range(L):
        new, idx_o, _ = oracle.cached_layer_step(x, ws[l], wrs[l], caches_o[l], n_drift, s.head_dim, EPS, s.dtype)
        hh = host(dcs[l].h)
        for b in range(s.batch):
            I = np.sort(np.asarray(idx_o[b], np.int64))
            assert np.array_equal(I, drifted[b]), (l, b)
            assert np.array_equal(np.sort(got_idx[l][b]), I), (l, b)
            assert rel_l2(hh[b][I], new.h[b][I]) <= tol_for(s.dtype), (l, b)
            rest = np.setdiff1d(np.arange(s.n_tokens), I)
            assert np.array_equal(hh[b][rest], warm_h[l][b][rest]), (l, b)
        x = new.h


def test_sparse_update_unsorted_and_out_of_range_indices():
    import torch
    spa = _lib()
    case = Case(SMALL_BF16[0], seed=70, n_drift=20)
    s = case.shape
    w, c = case.device()
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(s.n_tokens)[:23] for _ in range(s.batch)]).astype(np.int32)
    bad = idx.copy()
    bad[:, 5] = s.n_tokens + 7       # skipped by every write
    spa.spa_sparse_update(s, w, c, dev(case.x1, s.dtype), torch.from_numpy(bad).cuda(), spa.alloc_workspace(s, 23))
    torch.cuda.synchronize()
    good = np.delete(idx, 5, axis=1)
    ref = oracle.sparse_update(case.x1, case.w, case.cache0, good, s.head_dim, EPS, s.dtype)
    # the skipped row was never written: the update used 22 rows and keeps row idx[:,5] cached
    hh = host(c.h)
    for b in range(s.batch):
        assert rel_l2(hh[b][good[b]], ref.h[b][good[b]]) <= 2e-2
        assert np.array_equal(hh[b][idx[b, 5]], case.cache0.h[b][idx[b, 5]])


# ---------------------------------------------------------------------------------------------
# full-size layers: the llada-layer workload (N=1024, d=4096, r=128, k=256), Dream layers at the
# stack's row counts, and the batched stress layer (B=8, N=4096)
# ---------------------------------------------------------------------------------------------
def _redrift(case, n_drift, seed):
    """A copy of `case` whose step input drifts on exactly n_drift rows per sequence (N(0, 0.5^2)
    added; N(0, (1e-3)^2) on every other row). With k = n_drift the update set is the drifted rows,
    whose cosines lie far below the others', so the step's own index sets and outputs are compared
    with the oracle's (no near-tie fallback)."""
    c = Case.__new__(Case)
    c.shape, c.w, c.w_r, c.x0, c.cache0 = case.shape, case.w, case.w_r, case.x0, case.cache0
    rng = np.random.default_rng([78, seed, n_drift])
    c.x1, c.drifted = synth.drift_step(case.x0, n_drift, rng, case.shape.dtype)
    return c


def _kv_cache_case(s, w, x0, w_r):
    """Host case whose cache holds the K/V of every token of x0, H^c = x0 and P^c = proxy(x0)."""
    case = Case.__new__(Case)
    case.shape, case.w, case.w_r, case.x0 = s, w, w_r, x0
    kc, vc = oracle.kv_project(x0, w, s.head_dim, EPS, s.dtype)
    pc = oracle.proxy(x0, w_r).astype(np.float32).astype(np.float64)
    case.cache0 = oracle.LayerCache(kc, vc, np.asarray(x0, np.float64), pc)
    return case


@pytest.fixture(scope="module")
def llada_case():
    """The llada-layer workload; one SVD of W_v gives the proxies of every rank the stack offers (the
    rank-r proxy is the first r rows of the rank-512 one)."""
    wl = synth.WORKLOADS["llada-layer"]
    s = wl.shape
    w = synth.layer_weights(wl)
    w512 = oracle.singular_proxy(w["w_v"], w["g_attn"], 512)
    w_rs = {r: synth.to_storage(w512[:r], s.dtype) for r in sorted(set(LLADA_ID_RANKS) | {s.rank})}
    xs, drifted = synth.drift_sequence(wl, n_steps=1)
    case = _kv_cache_case(s, w, xs[0], w_rs[s.rank])
    case.w_rs = w_rs
    case.x1, case.drifted = xs[1], drifted[0]
    return case


def _identify_check(case, s, w_r):
    """spa_identify of case.x1 against the cached proxies of case.x0 under W_r (rank s.rank): P and the
    scores against the oracle."""
    import torch
    spa = _lib()
    pc = oracle.proxy(case.x0, w_r).astype(np.float32).astype(np.float64)
    p_out = torch.empty(s.batch, s.n_tokens, s.rank, dtype=torch.float32, device="cuda")
    scores = torch.empty(s.batch, s.n_tokens, dtype=torch.float32, device="cuda")
    spa.spa_identify(s, dev(case.x1, s.dtype), spa.spa_pack_weight(dev(w_r, s.dtype)),
                     torch.from_numpy(pc.astype(np.float32)).cuda(), p_out, scores, spa.alloc_workspace(s, 0))
    torch.cuda.synchronize()
    p_o, s_o = oracle.identify(case.x1, w_r, pc)
    assert np.max(np.abs(host(scores) - s_o)) <= 1e-3
    assert rel_l2(host(p_out), p_o) <= 1e-5


@pytest.mark.timeout(600)
def test_llada_layer_step_full_size(llada_case):
    """The workload's own first step (f ~ U(0.1, 0.4): 165 drifted rows) at k = 256: the k-th
    boundary falls among the undrifted rows, so near-ties are allowed there."""
    _check_step(llada_case, 256)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("k", LLADA_EXACT_K)
def test_llada_layer_step_full_size_exact_sets(llada_case, k):
    """Exactly k drifted rows at the LLaDA stack's row counts (51 and 87 of its first layers, 123, and
    k = 130, 200 whose last 128-row GEMM tile holds 2 and 72 rows) and at the workload's k = 256: the
    step's own sets equal the oracle's and its own block outputs are compared."""
    _check_step(_redrift(llada_case, k, 2), k, exact=True)


def _full_value_proxy(case):
    """The full-dimension Value identifier: W_r = W_v diag(g_attn), rounded to storage."""
    return synth.to_storage(np.asarray(case.w["w_v"], np.float64) * np.asarray(case.w["g_attn"], np.float64)[None, :],
                            case.shape.dtype)


@pytest.mark.timeout(600)
def test_llada_identify_full_value_rank(llada_case):
    """The full-dimension Value identifier at the llada shape: r = d_kv = 4096 (spa_identify: P of
    1024 x 4096 and the scores)."""
    c = llada_case
    _identify_check(c, c.shape.replace(rank=c.shape.d_kv), _full_value_proxy(c))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("r", LLADA_ID_RANKS)
def test_llada_identify_ranks(llada_case, r):
    """Identification at the llada shape for the other proxy ranks the stack offers."""
    _identify_check(llada_case, llada_case.shape.replace(rank=r), llada_case.w_rs[r])


@pytest.mark.timeout(600)
def test_llada_layer_full_recompute_full_size(llada_case):
    """The vanilla full recompute of the llada layer (M = 1024 rows in every product, 1024 queries per
    head in attention) against the oracle's warm-up."""
    import torch
    spa = _lib()
    c = llada_case
    s = c.shape
    dw = spa.upload_weights(c.w, c.w_r, s.dtype)
    dc = spa.alloc_cache(s)
    spa.spa_layer_full(s, dw, dc, dev(c.x1, s.dtype), spa.alloc_workspace(s, s.n_tokens))
    torch.cuda.synchronize()
    ref = oracle.warmup(c.x1, c.w, c.w_r, s.head_dim, EPS, s.dtype)
    errs = {"K": rel_l2(host(dc.k), ref.k), "V": rel_l2(host(dc.v), ref.v), "H": rel_l2(host(dc.h), ref.h)}
    assert max(errs.values()) <= 2e-2, errs
    assert rel_l2(host(dc.p), ref.p) <= 1e-5


@pytest.fixture(scope="module")
def dream_case():
    wl = synth.WORKLOADS["dream-stack"]
    s = wl.shape
    w = synth.layer_weights(wl, layer=9)
    w_r = synth.to_storage(oracle.singular_proxy(w["w_v"], w["g_attn"], s.rank), s.dtype)
    case = _kv_cache_case(s, w, synth.first_hidden(wl, layer=9), w_r)
    case.x1, case.drifted = synth.drift_step(case.x0, 600, np.random.default_rng([4, 9, 3]), s.dtype)
    return case


@pytest.mark.timeout(600)
def test_dream_layer_step_full_size(dream_case):
    """The peak layer of the Dream stack (layer 10, k = 512) with 600 drifted rows: near-ties allowed
    at the boundary among the drifted rows."""
    _, ks = oracle.budget(28, 10, 0.25, 0.05, 0.08, dream_case.shape.n_tokens)
    assert int(ks[9]) == 512
    _check_step(dream_case, 512)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("k", DREAM_STACK_K)
def test_dream_layer_step_full_size_stack_rows(dream_case, k):
    """Exactly k drifted rows at row counts of the Dream stack's layers (k_1 = 102 up to the peak
    k_10 = 512): the register-path tiles with two to four workgroups per CU, split-K W_down, and
    the gate/up product split into whole rounds of 256 x 256 tiles plus a remainder of columns on a
    smaller tile."""
    _check_step(_redrift(dream_case, k, 4), k, exact=True)


@pytest.mark.timeout(600)
def test_dream_layer_step_full_value_identifier(dream_case):
    """A Dream step whose identifier is the full Value projection (r = d_kv = 512, past one wave's
    256-column pass in the cosine kernel), exactly k = 102 drifted rows."""
    c = _redrift(dream_case, 102, 6)
    c.w_r = _full_value_proxy(c)
    c.shape = c.shape.replace(rank=c.shape.d_kv)
    c.cache0 = oracle.LayerCache(c.cache0.k, c.cache0.v, c.cache0.h,
                                 oracle.proxy(c.x0, c.w_r).astype(np.float32).astype(np.float64))
    _check_step(c, 102, exact=True)


def _with_proxy(case, w_r):
    """The same case with another singular proxy W_r (its rank from W_r's rows): the cached proxies of
    the warm-up input recomputed under it."""
    case.w_r = w_r
    case.shape = case.shape.replace(rank=w_r.shape[0])
    case.cache0 = oracle.LayerCache(case.cache0.k, case.cache0.v, case.cache0.h,
                                    oracle.proxy(case.x0, w_r).astype(np.float32).astype(np.float64))
    return case


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wl,r,k", RANK_STEP_CASES)
def test_layer_step_other_rank_full_size(llada_case, dream_case, wl, r, k):
    """Cached steps of the llada and Dream layers at proxy rank r (the stacks' rank sweep: the cosine
    pass then serves a row per wave, against two rows per wave at rank 128), exactly k drifted rows."""
    base = llada_case if wl == "llada" else dream_case
    c = _redrift(base, k, 7)
    if wl == "llada":
        w_r = base.w_rs[r]
    else:
        w_r = synth.to_storage(oracle.singular_proxy(c.w["w_v"], c.w["g_attn"], r), c.shape.dtype)
    _check_step(_with_proxy(c, w_r), k, exact=True)


@pytest.mark.timeout(900)
def test_dream_layer_full_recompute_full_size():
    """The full recompute (warm-up) of a Dream layer at full size (N=2048, GQA 28/4, F=18944): the
    gate/up product then runs on 2048 rows, where the 256 x 256 GEMM tiles are used."""
    import torch
    spa = _lib()
    wl = synth.WORKLOADS["dream-stack"]
    s = wl.shape
    w = synth.layer_weights(wl, layer=3)
    w_r = synth.to_storage(oracle.singular_proxy(w["w_v"], w["g_attn"], s.rank), s.dtype)
    x = synth.first_hidden(wl, layer=3)
    dw = spa.upload_weights(w, w_r, s.dtype)
    c = spa.alloc_cache(s)
    ws = spa.alloc_workspace(s, s.n_tokens)
    spa.spa_layer_full(s, dw, c, dev(x, s.dtype), ws)
    torch.cuda.synchronize()
    ref = oracle.warmup(x, w, w_r, s.head_dim, EPS, s.dtype)
    errs = {"K": rel_l2(host(c.k), ref.k), "V": rel_l2(host(c.v), ref.v), "H": rel_l2(host(c.h), ref.h)}
    assert max(errs.values()) <= 2e-2, errs
    assert rel_l2(host(c.p), ref.p) <= 1e-5


@pytest.fixture(scope="module")
def batched_case():
    """The batched stress layer (B=8, N=4096, d=4096): one SVD of W_v gives the proxies of every swept
    rank (the rank-r proxy is the first r rows of the rank-512 one)."""
    wl = synth.WORKLOADS["batched-stress"]
    s = wl.shape
    w = synth.layer_weights(wl)
    w512 = oracle.singular_proxy(w["w_v"], w["g_attn"], 512)
    w_rs = {r: synth.to_storage(w512[:r], s.dtype) for r in (64, 128, 512)}
    xs, drifted = synth.drift_sequence(wl, n_steps=1)
    case = _kv_cache_case(s, w, xs[0], w_rs[s.rank])
    case.w_rs = w_rs
    case.x1, case.drifted = xs[1], drifted[0]
    return case


@pytest.mark.timeout(900)
def test_batched_stress_full_size_sampled(batched_case):
    """The workload's own step (614 drifted rows per sequence) at rho = 0.25 -> k = 1024: every
    sequence's scores, proxy cache, index set (near-ties) and untouched rows; the block outputs of
    the first and the last sequence against the oracle."""
    wl = synth.WORKLOADS["batched-stress"]
    s = batched_case.shape
    k = int(oracle.budget(1, 1, wl.rho, wl.rho, wl.rho, s.n_tokens)[1][0])
    assert k == 1024
    i_g, _ = _check_step(batched_case, k, seqs=[0, s.batch - 1])
    for b in range(s.batch):   # the 614 drifted tokens of every sequence are all selected
        assert set(batched_case.drifted[b].tolist()) <= set(i_g[b].tolist())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("rho", BATCHED_EXACT_RHO)
def test_batched_stress_full_size_exact_sets(batched_case, rho):
    """The sweep's rho = 0.08 and 0.16 points (k = 327, 655; M = 2616 and 5240 rows in the GEMMs) with
    exactly k drifted rows per sequence: every sequence's set equals the oracle's; block outputs of the
    first and the last sequence."""
    s = batched_case.shape
    k = int(oracle.budget(1, 1, rho, rho, rho, s.n_tokens)[1][0])
    assert k == {0.08: 327, 0.16: 655}[rho]
    _check_step(_redrift(batched_case, k, 5), k, seqs=[0, s.batch - 1], exact=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("r", BATCHED_ID_RANKS)
def test_batched_identify_ranks(batched_case, r):
    """Identification of the batched layer (B N = 32768 rows) at the sweep's other proxy ranks:
    spa_identify's P and scores against the oracle."""
    _identify_check(batched_case, batched_case.shape.replace(rank=r), batched_case.w_rs[r])


def test_budget_through_the_c_abi():
    """rho(l) and k_l of spa_budget equal the oracle's for the workloads' budgets (host entry point;
    the CPU suite runs the same comparison on more parameters)."""
    spa = _lib()
    for args in [(32, 12, 0.25, 0.05, 0.08, 1024), (28, 10, 0.25, 0.05, 0.08, 2048), (1, 1, 0.25, 0.25, 0.25, 1024),
                 (1, 1, 0.08, 0.08, 0.08, 4096), (1, 1, 0.16, 0.16, 0.16, 4096), (1, 1, 1.0, 1.0, 1.0, 4096)]:
        rho, k = spa.spa_budget(*args)
        rho_o, k_o = oracle.budget(*args)
        assert k == k_o.tolist(), args
        assert np.max(np.abs(np.array(rho) - rho_o)) <= 1e-15, args


def _pack_reference(w, kind, e):
    """The fragment-packed layout written out on the host: one 1 KB block per (32-row block rb, K
    block kb of 16 bf16 / 8 fp32 elements), rb-major; lane l of a block holds row 32 rb + l % 32 at
    k = 16 kb + 8 (l // 32) + j, j < 8 (bf16) or k = 8 kb + 2 j + l // 32, j < 4 (fp32). Zero padding
    to 32 rows and 64 columns; gate/up: block rb holds the gate rows of units 16 rb .. 16 rb + 15,
    then the up rows of the same units."""
    rows, cols = w.shape
    cols_pad = -(-cols // 64) * 64
    if kind == 1:
        f = rows // 2
        fp = -(-f // 64) * 64
        logical = np.zeros((2 * fp, cols), w.dtype)
        for r in range(2 * fp):
            rb, ww = divmod(r, 32)
            u = rb * 16 + ww % 16
            if u < f:
                logical[r] = w[u] if ww < 16 else w[f + u]
        rows_pad = 2 * fp
    else:
        rows_pad = -(-rows // 32) * 32
        logical = np.zeros((rows_pad, cols), w.dtype)
        logical[:rows] = w
    full = np.zeros((rows_pad, cols_pad), w.dtype)
    full[:, :cols] = logical
    bkf = 16 if e == 2 else 8
    out = []
    for rb in range(rows_pad // 32):
        for kb in range(cols_pad // bkf):
            for lane in range(64):
                r = rb * 32 + lane % 32
                if e == 2:
                    ks = [16 * kb + 8 * (lane // 32) + j for j in range(8)]
                else:
                    ks = [8 * kb + 2 * j + lane // 32 for j in range(4)]
                out.append(full[r, ks])
    return np.concatenate(out)


@pytest.mark.parametrize("scaled", [False, True])
@pytest.mark.parametrize("dtype,rows,cols,kind", [("bf16", 200, 96, 0), ("bf16", 2 * 688, 256, 1),
                                                  ("f32", 16, 256, 0), ("f32", 2 * 48, 80, 1)])
def test_pack_weight_layout_bit_exact(dtype, rows, cols, kind, scaled):
    import torch
    spa = _lib()
    rng = np.random.default_rng(rows + cols)
    w = synth.to_storage(rng.standard_normal((rows, cols)), dtype)
    g = synth.to_storage(rng.uniform(0.5, 1.5, cols), dtype) if scaled else None
    packed = spa.spa_pack_weight(dev(w, dtype), kind, col_scale=None if g is None else dev(g, dtype))
    torch.cuda.synchronize()
    src = w.astype(np.float32)
    if scaled:  # W diag(g): the product in fp32, rounded once to the storage type
        src = synth.to_storage(src * g.astype(np.float32), dtype).astype(np.float32)
    ref = _pack_reference(src, kind, 2 if dtype == "bf16" else 4)
    assert np.array_equal(packed.float().cpu().numpy(), ref)
