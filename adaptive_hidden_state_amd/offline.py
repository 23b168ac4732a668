"""Offline, once-per-model preparation of the singular proxy ([PN] 关键设计 2; [GS] part 1).

W_r = Lambda_r V_r^T is built from the SVD of the layer's Value projection with the attention
RMSNorm gain folded in (W = W_v diag(g_attn)), because the proxy reads the raw hidden state.
This is host-side LAPACK work done once per layer, off the decoding path; the decoding step
itself runs entirely in libspacache.
"""
from __future__ import annotations

import numpy as np


def singular_proxy_weights(w_v, g_attn, r: int) -> np.ndarray:
    """r x d float64 W_r from a full SVD of W_v diag(g_attn) (LAPACK gesdd)."""
    w = np.asarray(w_v, dtype=np.float64) * np.asarray(g_attn, dtype=np.float64)[None, :]
    _, lam, vt = np.linalg.svd(w, full_matrices=False)
    if not 1 <= r <= lam.shape[0]:
        raise ValueError("rank out of range")
    return lam[:r, None] * vt[:r]


def singular_proxy_from_factors(lam, v_right, r: int, g_attn=None) -> np.ndarray:
    """W_r from known singular factors of W_v (values lam, right vectors as rows of v_right).

    Valid only when the gain is 1 everywhere (then W_v diag(g) = W_v and its factors are known).
    """
    def is_torch(a):
        return type(a).__module__.startswith("torch")

    if g_attn is not None:
        ones = bool((g_attn == 1).all()) if is_torch(g_attn) else bool(np.all(np.asarray(g_attn) == 1))
        if not ones:
            raise ValueError("closed-form factors need unit RMSNorm gains; use singular_proxy_weights")
    if is_torch(v_right):  # torch tensor (device-side factors of the large workloads)
        import torch
        lam_t = torch.as_tensor(np.asarray(lam[:r], dtype=np.float64), dtype=torch.float64, device=v_right.device)
        return lam_t[:, None] * v_right[:r].to(torch.float64)
    lam = np.asarray(lam, dtype=np.float64)
    return lam[:r, None] * np.asarray(v_right, dtype=np.float64)[:r]
