"""Shared helpers of the GPU parity tests: device transfer, error norms, the near-tie protocol."""
from __future__ import annotations

import numpy as np

import oracle


def has_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def dev(a, dtype: str):
    """Host float array (already rounded to the storage dtype) -> device tensor of that dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def tol_for(dtype: str) -> float:
    """Block-output tolerance (relative L2 over the updated rows): bf16 2e-2, fp32 1e-5."""
    return 2e-2 if dtype == "bf16" else 1e-5


def kth_boundary(s: np.ndarray, k: int) -> float:
    """Score of the k-th least similar token under the selection order."""
    order = np.lexsort((np.arange(len(s)), oracle.order_key(s)))
    return float(s[order[k - 1]])


def check_near_ties(i_gpu: np.ndarray, i_orc: np.ndarray, s_orc: np.ndarray, k: int, tol: float = 2e-3):
    """The GPU's set may differ from the oracle's only by tokens whose oracle score lies within tol
    of the k-th boundary score (both picks are then correct up to score rounding)."""
    assert len(i_gpu) == k and len(set(i_gpu.tolist())) == k
    assert np.all(np.diff(i_gpu) > 0), "indices must be ascending"
    diff = set(i_gpu.tolist()) ^ set(i_orc.tolist())
    if not diff:
        return 0
    b = kth_boundary(s_orc, k)
    bad = [j for j in diff if not abs(float(s_orc[j]) - b) <= tol]
    assert not bad, f"index sets differ beyond near-ties: {bad[:10]} (boundary {b})"
    return len(diff)
