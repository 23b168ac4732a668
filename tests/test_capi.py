"""CPU tests of libspacache's C ABI: the library loads, exports what include/spacache.h declares,
the host-only entry points agree with the oracle, and argument validation rejects bad calls
before any launch (so these run without a GPU; no call here reaches a kernel)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spacache.h")


@pytest.fixture(scope="module")
def lib():
    from adaptive_hidden_state_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libspacache.so is not built (python -m adaptive_hidden_state_amd.build)")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    from adaptive_hidden_state_amd import binding
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (spa_[a-z_]+)\b", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    from adaptive_hidden_state_amd import binding
    for code in range(0, -7, -1):
        assert binding.spa_status_string(code).startswith("SPA_")
    assert "unknown" in binding.spa_status_string(42)


@pytest.mark.parametrize("args", [(32, 12, 0.25, 0.05, 0.08, 1024), (28, 10, 0.25, 0.05, 0.08, 2048),
                                  (1, 1, 0.3, 0.1, 0.2, 10), (5, 1, 0.25, 0.25, 0.05, 100),
                                  (7, 7, 0.4, 0.01, 0.3, 333), (3, 2, 1.0, 1e-6, 1e-6, 64)])
def test_budget_matches_oracle(lib, args):
    from adaptive_hidden_state_amd import binding
    rho, k = binding.spa_budget(*args)
    rho_o, k_o = oracle.budget(*args)
    assert k == k_o.tolist()
    assert np.max(np.abs(np.array(rho) - rho_o)) <= 1e-15


@pytest.mark.parametrize("args", [(0, 1, .2, .1, .1, 8), (4, 5, .2, .1, .1, 8), (4, 0, .2, .1, .1, 8),
                                  (4, 2, 0.0, .1, .1, 8), (4, 2, .2, 1.5, .1, 8), (4, 2, .2, .1, .1, 0),
                                  (4, 2, float("nan"), .1, .1, 8)])
def test_budget_rejects(lib, args):
    assert lib.spa_budget(*args, None, None) == -1


def _shape(**kw):
    from adaptive_hidden_state_amd import binding
    base = dict(batch=1, n_tokens=1024, d_model=4096, n_q_heads=32, n_kv_heads=32, head_dim=128, d_ffn=12288,
                rank=128, dtype="bf16", norm_eps=1e-6)
    base.update(kw)
    return binding.make_shape(synth.LayerShape(**{k: v for k, v in base.items()}))


def _ws_bytes(lib, s, k):
    out = ctypes.c_size_t(0)
    st = lib.spa_workspace_bytes(ctypes.byref(s), k, ctypes.byref(out))
    return st, out.value


def test_workspace_sizes(lib):
    s = _shape()
    st, b256 = _ws_bytes(lib, s, 256)
    assert st == 0 and b256 > 0
    st, b1024 = _ws_bytes(lib, s, 1024)
    assert st == 0 and b1024 > b256
    st, b0 = _ws_bytes(lib, s, 0)
    assert st == 0 and 0 < b0 < b256
    # the k-row activations alone (A1, Q, O, Y, B1, Z in bf16) must fit
    assert b256 >= 256 * (4096 * 3 + 4096 * 2 + 12288) * 2
    assert _ws_bytes(lib, s, 1025)[0] == -1 and _ws_bytes(lib, s, -1)[0] == -1


@pytest.mark.parametrize("kw,code", [
    (dict(d_model=4000), -2), (dict(head_dim=96, n_q_heads=32, n_kv_heads=32), -2), (dict(n_kv_heads=5), -2),
    (dict(rank=100), -2), (dict(rank=8192), -2), (dict(rank=4096), 0), (dict(rank=2048, n_kv_heads=8), -2), (dict(n_tokens=20000), -2), (dict(d_ffn=1000), -2),
    (dict(batch=0), -1), (dict(n_tokens=0), -1), (dict(norm_eps=-1.0), -1),
    (dict(rope_theta=-1.0), -1), (dict(rope_theta=0.5), -1), (dict(rope_theta=float("inf")), -1),
    (dict(rope_theta=1e6), 0),
    (dict(dtype="f32"), 0), (dict(n_q_heads=28, n_kv_heads=4, d_model=3584), 0)])
def test_shape_validation(lib, kw, code):
    s = _shape(**kw)
    assert _ws_bytes(lib, s, 1)[0] == code


def _fake(addr):
    return ctypes.c_void_p(addr)


def _weights(base=0x100000, misalign=None):
    from adaptive_hidden_state_amd import binding
    vals = [base + 0x1000000 * i for i in range(5)]
    if misalign is not None:
        vals[misalign] += 2
    return binding.spa_layer_weights(*[_fake(v) for v in vals])


def _cache(base=0x40000000, h=None):
    from adaptive_hidden_state_amd import binding
    step = 0x10000000
    return binding.spa_layer_cache(_fake(base), _fake(base + step), _fake(h if h is not None else base + 2 * step),
                                   _fake(base + 3 * step))


X = 0x80000000


def _step(lib, s, w, c, x, k=256, policy=0, idx=0x90000000, scores=None, ws=0xA0000000, ws_bytes=1 << 40):
    return lib.spa_layer_step(ctypes.byref(s), ctypes.byref(w) if w is not None else None, ctypes.byref(c),
                              _fake(x) if x else None, k, policy, _fake(idx) if idx else None,
                              _fake(scores) if scores else None, _fake(ws) if ws else None, ws_bytes, None)


def test_layer_step_validation(lib):
    s = _shape()
    assert _step(lib, s, None, _cache(), X) == -1                         # null weights
    assert _step(lib, s, _weights(misalign=2), _cache(), X) == -4         # misaligned weight
    assert _step(lib, s, _weights(), _cache(), X + 8) == -4               # misaligned input
    assert _step(lib, s, _weights(), _cache(h=X + 4096), X) == -3         # h_in overlaps H^c
    assert _step(lib, s, _weights(), _cache(), X, k=1025) == -1           # k > N
    assert _step(lib, s, _weights(), _cache(), X, k=-1) == -1
    assert _step(lib, s, _weights(), _cache(), X, policy=7) == -1
    assert _step(lib, s, _weights(), _cache(), X, idx=0) == -1            # k > 0 needs idx_out
    assert _step(lib, s, _weights(), _cache(), X, ws_bytes=1024) == -5    # workspace too small
    assert _step(lib, s, _weights(), _cache(), X, ws=0) == -5
    assert _step(lib, _shape(head_dim=80), _weights(), _cache(), X) == -2


def test_full_and_sparse_validation(lib):
    s = _shape()
    w, c = _weights(), _cache()
    assert lib.spa_layer_full(ctypes.byref(s), ctypes.byref(w), ctypes.byref(c), _fake(X), _fake(0xA0000000),
                              1024, None) == -5
    assert lib.spa_layer_full(ctypes.byref(s), ctypes.byref(w), ctypes.byref(_cache(h=X)), _fake(X),
                              _fake(0xA0000000), 1 << 40, None) == -3
    assert lib.spa_sparse_update(ctypes.byref(s), ctypes.byref(w), ctypes.byref(c), _fake(X), None, 5,
                                 _fake(0xA0000000), 1 << 40, None) == -1
    assert lib.spa_sparse_update(ctypes.byref(s), ctypes.byref(w), ctypes.byref(c), _fake(X), _fake(0x90000004), 5,
                                 _fake(0xA0000000), 1 << 40, None) == -4


def test_identify_topk_attend_validation(lib):
    s = _shape()
    P = 0xB0000000
    assert lib.spa_identify(ctypes.byref(s), _fake(X), _fake(P), None, None, None, _fake(0xA0000000), 1 << 40,
                            None) == -1                                  # nothing to produce
    assert lib.spa_identify(ctypes.byref(s), _fake(X), _fake(P), None, None, _fake(0xC0000000), _fake(0xA0000000),
                            1 << 40, None) == -1                         # scores need a cache
    assert lib.spa_identify(ctypes.byref(s), _fake(X), _fake(P + 2), None, _fake(0xC0000000), None,
                            _fake(0xA0000000), 1 << 40, None) == -4
    assert lib.spa_identify(ctypes.byref(s), _fake(X), _fake(P), _fake(0xC0000000), _fake(0xC0000000), _fake(0xD0000000),
                            _fake(0xA0000000), 1 << 40, None) == -3      # p_out overlaps p_cache
    assert lib.spa_topk(1, 100, _fake(P), 101, _fake(0xC0000000), None) == -1
    assert lib.spa_topk(0, 100, _fake(P), 1, _fake(0xC0000000), None) == -1
    assert lib.spa_topk(1, 20000, _fake(P), 1, _fake(0xC0000000), None) == -2
    assert lib.spa_topk(1, 100, _fake(P + 4), 1, _fake(0xC0000000), None) == -4
    assert lib.spa_topk(1, 100, None, 1, _fake(0xC0000000), None) == -1
    assert lib.spa_attend(ctypes.byref(s), _fake(X), 10, _fake(P), _fake(P), _fake(X), None) == -3
    assert lib.spa_attend(ctypes.byref(s), _fake(X), -1, _fake(P), _fake(P), _fake(0xC0000000), None) == -1


def test_binding_refuses_host_tensors(lib):
    import torch
    import adaptive_hidden_state_amd as spa
    with pytest.raises(ValueError):
        spa.spa_topk(torch.zeros(1, 8), 2, torch.zeros(1, 2, dtype=torch.int32))


def test_offline_proxy_matches_oracle():
    from adaptive_hidden_state_amd import offline
    rng = np.random.default_rng(0)
    w = rng.standard_normal((48, 64))
    g = rng.uniform(0.5, 1.5, 64)
    a = offline.singular_proxy_weights(w, g, 12)
    b = oracle.singular_proxy(w, g, 12)
    assert np.allclose(a.T @ a, b.T @ b, atol=1e-10)     # equal up to row signs
    shape = synth.LayerShape(1, 8, 64, 2, 2, 16, 32, 16, "f32")
    wl = synth.Workload(7, "t", shape, spectrum="power1.2")
    ww = synth.layer_weights(wl, 0, shape, std=0.02)
    c = offline.singular_proxy_from_factors(ww["v_lambda"], ww["v_right"], 16)
    svd = oracle.singular_proxy(ww["w_v"], None, 16)     # w_v is the planted matrix rounded to fp32
    assert np.allclose(c.T @ c, svd.T @ svd, rtol=0, atol=1e-5 * np.abs(svd.T @ svd).max())
    with pytest.raises(ValueError):
        offline.singular_proxy_from_factors(ww["v_lambda"], ww["v_right"], 4, g_attn=np.full(64, 2.0))


def test_packed_weight_bytes(lib):
    from adaptive_hidden_state_amd import binding
    assert binding.spa_packed_weight_bytes("bf16", 12288, 4096) == 12288 * 4096 * 2
    assert binding.spa_packed_weight_bytes("bf16", 100, 80) == 128 * 128 * 2          # rows to 32, cols to 64
    assert binding.spa_packed_weight_bytes("bf16", 33, 64) == 64 * 64 * 2
    assert binding.spa_packed_weight_bytes("f32", 16, 256) == 32 * 256 * 4
    assert binding.spa_packed_weight_bytes("bf16", 2 * 688, 256, 1) == 2 * 704 * 256 * 2   # gate/up: 2 F_pad rows
    out = ctypes.c_size_t(0)
    assert lib.spa_packed_weight_bytes(1, 100, 81, 0, ctypes.byref(out)) == -2          # cols % 16
    assert lib.spa_packed_weight_bytes(1, 101, 80, 1, ctypes.byref(out)) == -1          # odd gate/up rows
    assert lib.spa_packed_weight_bytes(5, 100, 80, 0, ctypes.byref(out)) == -2          # dtype
    assert lib.spa_packed_weight_bytes(1, 100, 80, 3, ctypes.byref(out)) == -1          # kind
    assert lib.spa_pack_weight(1, 64, 64, 0, _fake(0x1000), None, _fake(0x1000 + 64), None) == -3
    assert lib.spa_pack_weight(1, 64, 64, 0, _fake(0x1008), None, _fake(0x100000), None) == -4
    assert lib.spa_pack_weight(1, 64, 64, 0, _fake(0x1000), _fake(0x200008), _fake(0x100000), None) == -4  # scale
    assert lib.spa_pack_weight(1, 64, 64, 0, _fake(0x1000), _fake(0x100040), _fake(0x100000), None) == -3  # scale
    assert lib.spa_pack_weight(1, 64, 64, 0, None, None, _fake(0x100000), None) == -1


def test_alias_checks_of_every_written_buffer(lib):
    """Each buffer a call writes must be disjoint from the others it writes and from what it only
    reads: outputs over the caches, the workspace, h_in or a weight are refused before any launch."""
    s = _shape()
    w, c = _weights(), _cache()
    WS = 0xA0000000
    ws_bytes = _ws_bytes(lib, s, 256)[1]
    cache_base = 0x40000000
    # spa_layer_step: idx_out / scores_out over H^c, K^c, over the workspace, over each other
    assert _step(lib, s, w, c, X, idx=cache_base + 0x20000000) == -3           # idx_out inside H^c
    assert _step(lib, s, w, c, X, scores=cache_base) == -3                       # scores_out inside K^c
    assert _step(lib, s, w, c, X, scores=WS + 4096, ws_bytes=ws_bytes) == -3    # scores_out inside the workspace
    assert _step(lib, s, w, c, X, idx=WS, ws_bytes=ws_bytes) == -3              # idx_out inside the workspace
    assert _step(lib, s, w, c, X, idx=0x90000000, scores=0x90000000 + 512) == -3  # idx_out over scores_out
    assert _step(lib, s, w, c, X, scores=X + 64) == -3                          # scores_out over h_in
    assert _step(lib, s, w, c, X, idx=0x100000) == -3                           # idx_out over packed w_r
    assert _step(lib, s, w, c, X, ws=cache_base + 0x30000000, ws_bytes=ws_bytes) == -3   # workspace over P^c
    assert _step(lib, s, _weights(base=cache_base + 0x20000000), c, X) == -3   # a weight inside H^c
    # spa_layer_full: the workspace over a cache
    assert lib.spa_layer_full(ctypes.byref(s), ctypes.byref(w), ctypes.byref(c), _fake(X), _fake(cache_base),
                              1 << 40, None) == -3
    # spa_sparse_update: idx inside H^c (written), workspace over K^c
    assert lib.spa_sparse_update(ctypes.byref(s), ctypes.byref(w), ctypes.byref(c), _fake(X),
                                 _fake(cache_base + 0x20000000), 5, _fake(WS), 1 << 40, None) == -3
    assert lib.spa_sparse_update(ctypes.byref(s), ctypes.byref(w), ctypes.byref(c), _fake(X), _fake(0x90000000), 5,
                                 _fake(cache_base), 1 << 40, None) == -3
    # spa_identify: scores_out over h_in, over the workspace, over p_out, p_out over w_r
    P = 0xB0000000
    ident = lambda pc, po, so, ws=WS: lib.spa_identify(ctypes.byref(s), _fake(X), _fake(P), _fake(pc) if pc else None,
                                                       _fake(po) if po else None, _fake(so) if so else None,
                                                       _fake(ws), 1 << 40, None)
    assert ident(0xC0000000, None, X) == -3
    assert ident(0xC0000000, None, WS) == -3
    assert ident(0xC0000000, 0xD0000000, 0xD0000000 + 1024) == -3
    assert ident(0xC0000000, P, 0xE0000000) == -3
    assert ident(0xC0000000, 0xD0000000, 0xE0000000, ws=0xD0000000 + 4096) == -3
    # spa_topk: idx_out over the scores
    assert lib.spa_topk(2, 100, _fake(P), 10, _fake(P + 256), None) == -3


def test_noalloc_step_validation(lib):
    """spa_layer_step_noalloc validates like spa_layer_step, and refuses a call whose exact layout
    exceeds its 64 MiB of static scratch before touching the device."""
    s = _shape()
    w, c = _weights(), _cache()
    call = lambda s, w, c, x, k=256, idx=0x90000000: lib.spa_layer_step_noalloc(
        ctypes.byref(s), ctypes.byref(w) if w is not None else None, ctypes.byref(c), _fake(x) if x else None, k, 0,
        _fake(idx) if idx else None, None, None)
    assert call(s, None, c, X) == -1
    assert call(s, _weights(misalign=1), c, X) == -4
    assert call(s, w, _cache(h=X + 4096), X) == -3
    assert call(s, w, c, X, k=2000) == -1
    assert call(s, w, c, X, idx=0) == -1
    big = _shape(batch=8, n_tokens=4096)
    assert call(big, w, _cache(), X, k=1024, idx=0xF0000000) == -5
