"""Seeded synthetic inputs for the SPA-Cache layer step: shapes, weights, hidden states, drift.

This module is the only code shared by the CPU oracle's tests and the HIP path's tests and bench.
It holds no arithmetic of the method itself: it draws random numbers, plants a spectrum in the
Value projection, and rounds arrays to their storage dtype. Everything the method computes
(proxy, cosine, Top-k, budget, attention, FFN, SVD of the Value projection) lives elsewhere.

Workloads (synthetic stand-ins for the pages' LLaDA-8B-Instruct and Dream-v0-Instruct-7B runs on
public benchmarks; no dataset item and no trained weight is used anywhere):

  tiny-f32        1 x 64 tokens, d=256, 4 heads x 64, FFN 688, r=16, fp32, rho=0.25
  llada-layer     1 x 1024 tokens, d=4096, 32 heads x 128, FFN 12288, r=128, bf16, rho=0.25
  llada-stack     32 layers of the llada-layer shape, piecewise-Gaussian budget (0.25 at 12; 0.05; 0.08)
  dream-stack     28 layers, d=3584, 28 q / 4 kv heads x 128, FFN 18944, N=2048, r=128, bf16
  batched-stress  8 x 4096 tokens of the llada-layer shape, r in {64,128,512}, rho in {0.08,...,1}

Seeds: numpy.random.default_rng([config_id, layer, stream]) with stream 0 = weights, 1 = the
Haar factors of the planted Value projection, 2 = first hidden state, 3 = drift process.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "LayerShape", "Workload", "WORKLOADS", "layer_weights", "first_hidden", "drift_step",
    "drift_sequence", "to_storage", "storage_np_dtype",
]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    batch: int
    n_tokens: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    rank: int
    dtype: str = "bf16"          # "bf16" or "f32": storage type of X, weights, K/V/H caches
    norm_eps: float = 1e-6
    rope_theta: float = 0.0      # > 1: rotary embedding of q and k (0: none)

    @property
    def d_q(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def d_kv(self) -> int:
        return self.n_kv_heads * self.head_dim

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    config_id: int
    name: str
    shape: LayerShape
    n_layers: int = 1
    rho: Optional[float] = None             # uniform budget (single-layer workloads)
    budget: Optional[tuple] = None          # (rho_peak, l_peak, rho_first, rho_last) for stacks
    spectrum: str = "power1.2"              # planted Value spectrum: "geometric0.9" or "power1.2"
    drift_frac: Optional[float] = None      # fixed fraction of drifting tokens per step
    drift_range: Optional[tuple] = None     # U(lo, hi) fraction per step
    steps: int = 1                          # cached steps after the warm-up
    unmask_per_step: Optional[int] = None
    arch_rope_theta: float = 0.0            # the real layers' rotary base (used with the arch option)
    arch_qkv_bias: bool = False             # the real layers have q/k/v biases


WORKLOADS: Dict[str, Workload] = {
    "tiny-f32": Workload(1, "tiny-f32", LayerShape(1, 64, 256, 4, 4, 64, 688, 16, "f32"),
                         rho=0.25, spectrum="geometric0.9", drift_frac=0.2, steps=1),
    "llada-layer": Workload(2, "llada-layer", LayerShape(1, 1024, 4096, 32, 32, 128, 12288, 128, "bf16"),
                            rho=0.25, spectrum="power1.2", drift_range=(0.1, 0.4), steps=8, arch_rope_theta=5e5),
    "llada-stack": Workload(3, "llada-stack", LayerShape(1, 1024, 4096, 32, 32, 128, 12288, 128, "bf16"),
                            n_layers=32, budget=(0.25, 12, 0.05, 0.08), spectrum="power1.2",
                            steps=64, unmask_per_step=16, arch_rope_theta=5e5),
    "dream-stack": Workload(4, "dream-stack", LayerShape(1, 2048, 3584, 28, 4, 128, 18944, 128, "bf16"),
                            n_layers=28, budget=(0.25, 10, 0.05, 0.08), spectrum="power1.2",
                            steps=32, unmask_per_step=64, arch_rope_theta=1e6, arch_qkv_bias=True),
    "batched-stress": Workload(5, "batched-stress", LayerShape(8, 4096, 4096, 32, 32, 128, 12288, 128, "bf16"),
                               rho=0.25, spectrum="power1.2", drift_frac=0.15, steps=16),
}

STREAM_WEIGHTS, STREAM_HAAR, STREAM_X0, STREAM_DRIFT = 0, 1, 2, 3


def _rng(config_id: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(config_id), int(layer), int(stream)])


def storage_np_dtype(dtype: str):
    return np.float32


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round an array to the storage dtype and return it as float32 (bf16 values are exactly
    representable in float32). bf16 rounding is torch's CPU round-to-nearest-even cast."""
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a32
    if dtype != "bf16":
        raise ValueError(f"unknown storage dtype {dtype!r}")
    import torch
    return torch.from_numpy(a32).to(torch.bfloat16).to(torch.float32).numpy()


def _haar(rng: np.random.Generator, n: int, m: int) -> np.ndarray:
    """n x m matrix with orthonormal columns, Haar-distributed (QR of a Gaussian with the sign fix)."""
    g = rng.standard_normal((n, m))
    q, r = np.linalg.qr(g)
    q *= np.sign(np.diag(r))[None, :]
    return q


def planted_spectrum(kind: str, n: int, d_kv: int, d: int, std: float = 0.02) -> np.ndarray:
    """Singular values planted in the Value projection.

    geometric0.9: lambda_i = 0.9**i exactly (i = 1..n).
    power1.2:     lambda_i proportional to i**-1.2, scaled so that the Frobenius norm equals that of
                  a d_kv x d matrix of N(0, std^2) entries, std * sqrt(d * d_kv).
    """
    i = np.arange(1, n + 1, dtype=np.float64)
    if kind == "geometric0.9":
        return 0.9 ** i
    if kind == "power1.2":
        lam = i ** -1.2
        return lam * (std * math.sqrt(d * d_kv) / np.linalg.norm(lam))
    raise ValueError(kind)


def layer_weights(wl: Workload, layer: int = 0, shape: Optional[LayerShape] = None,
                  std: float = 0.02) -> Dict[str, np.ndarray]:
    """Random-init weights of one layer, rounded to the storage dtype (float32 arrays).

    Matrices are [out][in] row-major (y = x @ W.T). w_v = U diag(lambda) V^T is planted with Haar U, V;
    the planted factors are returned too ("v_lambda", "v_right" = V^T rows) so that callers can form
    the exact singular factors without an SVD. RMSNorm gains are 1 (as at initialisation).
    """
    s = shape or wl.shape
    rng = _rng(wl.config_id, layer, STREAM_WEIGHTS)
    d, dq, dkv, f = s.d_model, s.d_q, s.d_kv, s.d_ffn

    def normal(rows, cols):
        return (rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std))

    w = {}
    w["w_q"] = normal(dq, d)
    w["w_k"] = normal(dkv, d)
    w["w_o"] = normal(d, dq)
    w["w_gate"] = normal(f, d)
    w["w_up"] = normal(f, d)
    w["w_down"] = normal(d, f)
    hr = _rng(wl.config_id, layer, STREAM_HAAR)
    n = min(dkv, d)
    lam = planted_spectrum(wl.spectrum, n, dkv, d, std)
    u = _haar(hr, dkv, n)
    v = _haar(hr, d, n)
    w["w_v"] = ((u * lam[None, :]) @ v.T).astype(np.float32)
    w["v_lambda"] = lam
    w["v_right"] = v.T.copy()        # n x d, rows are right singular vectors of the planted w_v
    w["g_attn"] = np.ones(d, np.float32)
    w["g_ffn"] = np.ones(d, np.float32)
    for key in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_ffn"):
        w[key] = to_storage(w[key], s.dtype)
    return w


def first_hidden(wl: Workload, layer: int = 0, shape: Optional[LayerShape] = None) -> np.ndarray:
    """Hidden states at step 0: B x N x d, N(0, 1), rounded to the storage dtype."""
    s = shape or wl.shape
    rng = _rng(wl.config_id, layer, STREAM_X0)
    x = rng.standard_normal((s.batch, s.n_tokens, s.d_model), dtype=np.float32)
    return to_storage(x, s.dtype)


def drift_step(x: np.ndarray, n_drift: int, rng: np.random.Generator, dtype: str,
               big: float = 0.5, small: float = 1e-3, rows: Optional[np.ndarray] = None) -> (np.ndarray, List[np.ndarray]):
    """One step of the drift process: in each sequence, n_drift rows (random, or the given ones)
    get N(0, big^2) added, every other row N(0, small^2); the result is re-rounded to storage."""
    b, n, d = x.shape
    out = x.astype(np.float32, copy=True)
    chosen = []
    for bi in range(b):
        r = rows[bi] if rows is not None else rng.choice(n, size=n_drift, replace=False)
        r = np.asarray(r, dtype=np.int64)
        noise = rng.standard_normal((n, d), dtype=np.float32) * np.float32(small)
        noise[r] = rng.standard_normal((len(r), d), dtype=np.float32) * np.float32(big)
        out[bi] += noise
        chosen.append(np.sort(r))
    return to_storage(out, dtype), chosen


def drift_sequence(wl: Workload, n_steps: Optional[int] = None, layer: int = 0,
                   shape: Optional[LayerShape] = None):
    """X^0 and X^1..X^T for a single-layer workload, plus the drifted rows of every step.

    Drift count per step: round(f * N) with f fixed (drift_frac) or f ~ U(lo, hi) per step.
    """
    s = shape or wl.shape
    steps = wl.steps if n_steps is None else n_steps
    rng = _rng(wl.config_id, layer, STREAM_DRIFT)
    xs = [first_hidden(wl, layer, s)]
    drifted = []
    for _ in range(steps):
        f = wl.drift_frac if wl.drift_frac is not None else rng.uniform(*wl.drift_range)
        n_drift = int(round(f * s.n_tokens))
        x, rows = drift_step(xs[-1], n_drift, rng, s.dtype)
        xs.append(x)
        drifted.append(rows)
    return xs, drifted


def random_hidden(shape: LayerShape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) hidden states for edge-case tests (any shape), rounded to storage."""
    rng = np.random.default_rng([99, int(seed)])
    x = rng.standard_normal((shape.batch, shape.n_tokens, shape.d_model), dtype=np.float32) * np.float32(scale)
    return to_storage(x, shape.dtype)


def random_weights(shape: LayerShape, seed: int, std: float = 0.02, spectrum: str = "power1.2",
                   gains: str = "ones") -> Dict[str, np.ndarray]:
    """Weights for an arbitrary shape (edge cases, ragged sizes); same recipe as layer_weights.
    gains="random" draws RMSNorm gains from U(0.5, 1.5) to exercise the gain paths."""
    w = layer_weights(Workload(1000 + int(seed), "adhoc", shape, spectrum=spectrum), 0, shape, std)
    if gains == "random":
        rng = np.random.default_rng([98, int(seed)])
        w["g_attn"] = to_storage(rng.uniform(0.5, 1.5, shape.d_model).astype(np.float32), shape.dtype)
        w["g_ffn"] = to_storage(rng.uniform(0.5, 1.5, shape.d_model).astype(np.float32), shape.dtype)
    return w


# ---------------------------------------------------------------------------------------------
# Device-side generation for the multi-layer and batched workloads. A 32-layer stack holds ~13 GB
# of weights, too much to draw with NumPy on the host in a benchmark's set-up, so these draw the
# same distributions with a seeded torch generator on the device. Values differ from the NumPy
# streams above (different generator); shapes, distributions and seeds-by-(config, layer, stream)
# are the same. The planted Value projection reuses one host-drawn Haar pair per shape and gives
# every layer its own signed row permutation of it, which keeps the columns orthonormal and the
# planted spectrum exact while avoiding a 4096 x 4096 QR per layer.
# ---------------------------------------------------------------------------------------------

def _torch_gen(config_id: int, layer: int, stream: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(config_id) * 1_000_003 + int(layer) * 1009 + int(stream))
    return g


def haar_pair(wl: Workload, shape: Optional[LayerShape] = None):
    """Host-drawn orthonormal factors (U: d_kv x n, V: d x n, n = min(d_kv, d)) shared by a workload's
    layers, plus the planted singular values (float64)."""
    s = shape or wl.shape
    hr = _rng(wl.config_id, 0, STREAM_HAAR)
    n = min(s.d_kv, s.d_model)
    return _haar(hr, s.d_kv, n), _haar(hr, s.d_model, n), planted_spectrum(wl.spectrum, n, s.d_kv, s.d_model)


def layer_weights_device(wl: Workload, layer: int, pair, device="cuda", shape: Optional[LayerShape] = None,
                         std: float = 0.02, qkv_bias: bool = False) -> Dict[str, object]:
    """Random-init weights of one layer as device tensors in the storage dtype ([out][in] row-major),
    drawn on the device. w_v = (S P U) diag(lambda) (S' P' V)^T with this layer's random row
    permutations P, P' and sign flips S, S' of the shared Haar pair; "v_lambda" (host float64) and
    "v_right" (device float32, n x d: rows are the right singular vectors) are returned too."""
    import torch
    s = shape or wl.shape
    tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    g = _torch_gen(wl.config_id, layer, STREAM_WEIGHTS, device)
    d, dq, dkv, f = s.d_model, s.d_q, s.d_kv, s.d_ffn

    def normal(rows, cols):
        return (torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32) * std).to(tdt)

    w = {"w_q": normal(dq, d), "w_k": normal(dkv, d), "w_o": normal(d, dq), "w_gate": normal(f, d),
         "w_up": normal(f, d), "w_down": normal(d, f)}
    u0, v0, lam = pair
    gh = _torch_gen(wl.config_id, layer, STREAM_HAAR, device)

    def signed_perm(m):
        rows = torch.randperm(m.shape[0], generator=gh, device=device)
        sign = torch.randint(0, 2, (m.shape[0], 1), generator=gh, device=device).to(torch.float32) * 2 - 1
        return m[rows] * sign

    u = signed_perm(torch.as_tensor(u0, dtype=torch.float32, device=device))
    v = signed_perm(torch.as_tensor(v0, dtype=torch.float32, device=device))
    lam_t = torch.as_tensor(lam, dtype=torch.float32, device=device)
    w["w_v"] = ((u * lam_t[None, :]) @ v.T).to(tdt)
    w["v_lambda"] = np.asarray(lam, dtype=np.float64)
    w["v_right"] = v.T.contiguous()
    if qkv_bias:   # N(0, std^2) q/k/v biases
        w["b_q"], w["b_k"], w["b_v"] = normal(1, dq)[0], normal(1, dkv)[0], normal(1, dkv)[0]
    w["g_attn"] = torch.ones(d, dtype=tdt, device=device)
    w["g_ffn"] = torch.ones(d, dtype=tdt, device=device)
    return w


def normal_device(shape: tuple, config_id: int, layer: int, stream: int, device="cuda", std: float = 1.0,
                  dtype: str = "bf16"):
    """A seeded N(0, std^2) device tensor rounded to the storage dtype (inputs of the large workloads)."""
    import torch
    g = _torch_gen(config_id, layer, stream, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * std
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def unmask_schedule(wl: Workload, shape: Optional[LayerShape] = None, device="cuda", per_step: Optional[int] = None):
    """Denoising schedule of a stack workload: T = N / u steps (u = per_step, default the workload's),
    step t unmasks the u positions
    perm[t u : (t + 1) u] of one seeded permutation of the N positions, and gives them fresh N(0, 1)
    embedding rows. Returns (positions T x u int64, rows T x B x u x d in the storage dtype)."""
    import torch
    s = shape or wl.shape
    u = per_step or wl.unmask_per_step
    t_steps = s.n_tokens // u
    g = _torch_gen(wl.config_id, 0, STREAM_DRIFT, device)
    perm = torch.randperm(s.n_tokens, generator=g, device=device)[: t_steps * u].reshape(t_steps, u)
    rows = normal_device((t_steps, s.batch, u, s.d_model), wl.config_id, 1, STREAM_DRIFT, device, 1.0, s.dtype)
    return perm.contiguous(), rows


def drift_sequence_device(wl: Workload, shape: Optional[LayerShape] = None, n_steps: Optional[int] = None,
                          device="cuda"):
    """Device analogue of drift_sequence for the batched workload: X^0 ~ N(0, 1); at every step each
    sequence gets N(0, 0.5^2) on round(f N) random rows and N(0, (1e-3)^2) elsewhere, re-rounded to
    the storage dtype."""
    import torch
    s = shape or wl.shape
    steps = wl.steps if n_steps is None else n_steps
    tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    xs = [normal_device((s.batch, s.n_tokens, s.d_model), wl.config_id, 0, STREAM_X0, device, 1.0, s.dtype)]
    g = _torch_gen(wl.config_id, 0, STREAM_DRIFT, device)
    n_drift = int(round(wl.drift_frac * s.n_tokens))
    for _ in range(steps):
        noise = torch.randn(s.batch, s.n_tokens, s.d_model, generator=g, device=device) * 1e-3
        for b in range(s.batch):
            rows = torch.randperm(s.n_tokens, generator=g, device=device)[:n_drift]
            noise[b, rows] = torch.randn(n_drift, s.d_model, generator=g, device=device) * 0.5
        xs.append((xs[-1].to(torch.float32) + noise).to(tdt))
        del noise
    return xs
