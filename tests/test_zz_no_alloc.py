"""spa_layer_step_noalloc (the library's static device scratch, no workspace argument) against
spa_layer_step (the caller's workspace) through the C ABI: two calls in a row on one GPU, the second
with a smaller input than the first, so the second runs on scratch that holds the first call's data.
Both entry points run the same kernels with the same plans and reductions in a fixed order, so the
update sets, scores and caches must be bit-identical."""
import numpy as np
import pytest

import synth
from helpers import dev, has_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs an MI355X")]


def _pair(spa, s, w, x0, x1, k):
    """Warm two cache sets identically, then one cached step through each entry point."""
    import torch
    caches = [spa.alloc_cache(s) for _ in range(2)]
    ws_full = spa.alloc_workspace(s, s.n_tokens)
    for c in caches:
        spa.spa_layer_full(s, w, c, x0, ws_full)
    idx = [torch.full((s.batch, k), -1, dtype=torch.int32, device="cuda") for _ in range(2)]
    sc = [torch.full((s.batch, s.n_tokens), -7.0, dtype=torch.float32, device="cuda") for _ in range(2)]
    spa.spa_layer_step(s, w, caches[0], x1, k, spa.SPA_PROXY_WRITE_ALL, idx[0], sc[0], spa.alloc_workspace(s, k))
    spa.spa_layer_step_noalloc(s, w, caches[1], x1, k, spa.SPA_PROXY_WRITE_ALL, idx[1], sc[1])
    torch.cuda.synchronize()
    assert torch.equal(idx[0], idx[1])
    assert torch.equal(sc[0], sc[1])
    for a, b in zip(caches[0], caches[1]):
        assert torch.equal(a, b)
    return idx[1]


def test_noalloc_step_equals_workspace_step_twice():
    import torch
    import adaptive_hidden_state_amd as spa
    spa.load_library()
    # first call: the llada-shaped layer (N = 1024, d = 4096, F = 12288, k = 256; ~33 MiB of scratch)
    wl = synth.WORKLOADS["llada-layer"]
    s = wl.shape
    pair = synth.haar_pair(wl, s)
    wd = synth.layer_weights_device(wl, 0, pair, shape=s)
    w_r = spa.singular_proxy_from_factors(wd["v_lambda"], wd["v_right"], s.rank, wd["g_attn"])
    w = spa.upload_weights(wd, w_r.to(torch.bfloat16), s.dtype)
    del wd
    x0 = synth.normal_device((s.batch, s.n_tokens, s.d_model), 2, 0, synth.STREAM_X0)
    x1 = x0.clone()
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    rows = torch.randperm(s.n_tokens, generator=g, device="cuda")[:300]
    x1[:, rows] = (x1[:, rows].float() + 0.5 * torch.randn(s.batch, 300, s.d_model, generator=g, device="cuda")).to(
        torch.bfloat16)
    i1 = _pair(spa, s, w, x0, x1, 256)
    assert set(i1[0].tolist()) <= set(rows.tolist())   # the 256 selected rows are drifted ones
    # second call, smaller: two sequences of 200 tokens, d = 256, GQA-free, k = 37
    s2 = synth.LayerShape(2, 200, 256, 4, 4, 64, 688, 32, "bf16")
    w2h = synth.random_weights(s2, seed=11, std=0.1, gains="random")
    from adaptive_hidden_state_amd.offline import singular_proxy_weights
    w_r2 = synth.to_storage(singular_proxy_weights(w2h["w_v"], w2h["g_attn"], s2.rank), s2.dtype)
    w2 = spa.upload_weights(w2h, w_r2, s2.dtype)
    x20 = synth.random_hidden(s2, seed=12)
    x21, _ = synth.drift_step(x20, 40, np.random.default_rng([79, 1]), s2.dtype)
    _pair(spa, s2, w2, dev(x20, "bf16"), dev(x21, "bf16"), 37)


def test_noalloc_refuses_calls_past_the_scratch():
    """The batched layer (B = 8, N = 4096) needs more than the 64 MiB of scratch: SPA_ERR_WORKSPACE
    before any launch, and nothing was written."""
    import torch
    import adaptive_hidden_state_amd as spa
    spa.load_library()
    s = synth.LayerShape(8, 4096, 4096, 32, 32, 128, 12288, 128, "bf16")
    with pytest.raises(spa.SpaError) as e:
        w = spa.DeviceWeights(*[torch.empty(n // 2, dtype=torch.bfloat16, device="cuda") for n in (
            spa.spa_packed_weight_bytes("bf16", 128, 4096), spa.spa_packed_weight_bytes("bf16", 12288, 4096),
            spa.spa_packed_weight_bytes("bf16", 4096, 4096), spa.spa_packed_weight_bytes("bf16", 24576, 4096, 1),
            spa.spa_packed_weight_bytes("bf16", 4096, 12288))])
        c = spa.alloc_cache(s)
        x = torch.zeros(8, 4096, 4096, dtype=torch.bfloat16, device="cuda")
        idx = torch.full((8, 1024), -1, dtype=torch.int32, device="cuda")
        spa.spa_layer_step_noalloc(s, w, c, x, 1024, spa.SPA_PROXY_WRITE_ALL, idx, None)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool((idx == -1).all())
