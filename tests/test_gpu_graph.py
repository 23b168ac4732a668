"""The cached layer step captured in a HIP graph: every replay must equal the same step launched
eagerly. Replays run with new inputs copied in eagerly between them (the graph reads its captured
input buffer), and each replay is checked, not only the first."""
import numpy as np
import pytest

import synth
from helpers import dev, has_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs an MI355X")]


def test_step_graph_replays_match_eager():
    import torch
    import adaptive_hidden_state_amd as spa
    spa.load_library()
    shape = synth.LayerShape(1, 333, 512, 8, 2, 128, 1024, 64, "bf16")
    s = shape
    w = synth.random_weights(shape, seed=5, std=0.1, gains="random")
    from adaptive_hidden_state_amd.offline import singular_proxy_weights
    w_r = synth.to_storage(singular_proxy_weights(w["w_v"], w["g_attn"], s.rank), s.dtype)
    dw = spa.upload_weights(w, w_r, s.dtype)
    x0 = synth.random_hidden(shape, seed=6)
    rng = np.random.default_rng([78, 5])
    xs = [x0]
    for _ in range(3):
        xs.append(synth.drift_step(xs[-1], 60, rng, s.dtype)[0])
    k = 83

    def fresh():
        c = spa.alloc_cache(s)
        spa.spa_layer_full(s, dw, c, dev(x0, s.dtype), spa.alloc_workspace(s, s.n_tokens))
        return c

    cg, ce = fresh(), fresh()
    xbuf = dev(xs[1], s.dtype)
    ws_g, ws_e = spa.alloc_workspace(s, k), spa.alloc_workspace(s, k)
    idx_g = torch.empty(s.batch, k, dtype=torch.int32, device="cuda")
    idx_e = torch.empty_like(idx_g)
    sc_g = torch.empty(s.batch, s.n_tokens, dtype=torch.float32, device="cuda")
    sc_e = torch.empty_like(sc_g)
    torch.cuda.synchronize()

    # one eager step on a scratch cache first, so every kernel has run once before the capture
    scratch = fresh()
    spa.spa_layer_step(s, dw, scratch, xbuf, k, spa.SPA_PROXY_WRITE_ALL, idx_g, sc_g, ws_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()   # capturing does not execute: cg is still the warm-up state
    with torch.cuda.graph(g):
        spa.spa_layer_step(s, dw, cg, xbuf, k, spa.SPA_PROXY_WRITE_ALL, idx_g, sc_g, ws_g)
    torch.cuda.synchronize()

    for t in range(1, 4):
        xbuf.copy_(dev(xs[t], s.dtype))       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        spa.spa_layer_step(s, dw, ce, dev(xs[t], s.dtype), k, spa.SPA_PROXY_WRITE_ALL, idx_e, sc_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(idx_g, idx_e), t
        assert torch.equal(sc_g, sc_e), t
        for a, b in ((cg.k, ce.k), (cg.v, ce.v), (cg.h, ce.h), (cg.p, ce.p)):
            assert np.array_equal(host(a), host(b)), t
