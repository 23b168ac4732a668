"""ctypes binding of libspacache (include/spacache.h): argument marshalling only.

Every function here has the name of the C entry point it calls. Tensors are torch tensors that live
on the GPU; the binding checks dtype/device/contiguity, passes data_ptr() and the current HIP stream,
and raises SpaError on a non-zero status. No step of the method runs in Python: if the shared
library is missing, every call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional, Sequence, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libspacache.so")

SPA_OK = 0
SPA_F32, SPA_BF16 = 0, 1
SPA_PROXY_WRITE_ALL, SPA_PROXY_WRITE_SELECTED = 0, 1

# Every symbol include/spacache.h declares.
EXPORTS = ("spa_budget", "spa_packed_weight_bytes", "spa_pack_weight", "spa_workspace_bytes", "spa_layer_full",
           "spa_layer_step", "spa_layer_step_timed", "spa_layer_step_noalloc", "spa_identify", "spa_topk",
           "spa_sparse_update", "spa_attend", "spa_status_string")
SPA_PACK_PLAIN, SPA_PACK_GATE_UP = 0, 1


class SpaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {spa_status_string(status)} ({status})")


class spa_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_tokens", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_ffn", ctypes.c_int32), ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class spa_layer_weights(ctypes.Structure):
    _fields_ = [("w_r", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p),
                ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p), ("b_qkv", ctypes.c_void_p)]


class spa_layer_cache(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("h_cache", ctypes.c_void_p),
                ("p_cache", ctypes.c_void_p)]


class spa_timing(ctypes.Structure):
    _fields_ = [("marks", ctypes.c_void_p), ("capacity", ctypes.c_int32), ("count", ctypes.c_int32),
                ("names", ctypes.c_void_p)]


_lib_handle: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspacache.so once; raise if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise RuntimeError(f"libspacache.so not found at {path}; build it with "
                           f"`python -m adaptive_hidden_state_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "spa_budget": ([I32, I32, ctypes.c_double, ctypes.c_double, ctypes.c_double, I32, P, P], ctypes.c_int),
        "spa_packed_weight_bytes": ([I32, I32, I32, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "spa_pack_weight": ([I32, I32, I32, I32, P, P, P, P], ctypes.c_int),
        "spa_workspace_bytes": ([P, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "spa_layer_full": ([P, P, P, P, P, SZ, P], ctypes.c_int),
        "spa_layer_step": ([P, P, P, P, I32, I32, P, P, P, SZ, P], ctypes.c_int),
        "spa_layer_step_timed": ([P, P, P, P, I32, I32, P, P, P, SZ, P, P], ctypes.c_int),
        "spa_layer_step_noalloc": ([P, P, P, P, I32, I32, P, P, P], ctypes.c_int),
        "spa_identify": ([P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "spa_topk": ([I32, I32, P, I32, P, P], ctypes.c_int),
        "spa_sparse_update": ([P, P, P, P, P, I32, P, SZ, P], ctypes.c_int),
        "spa_attend": ([P, P, I32, P, P, P, P], ctypes.c_int),
        "spa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib_handle = lib
    return lib


def spa_status_string(status: int) -> str:
    return load_library().spa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != SPA_OK:
        raise SpaError(status, where)


# ----------------------------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------------------------
def dtype_code(dtype) -> int:
    if dtype in (SPA_F32, "f32", "float32", "fp32"):
        return SPA_F32
    if dtype in (SPA_BF16, "bf16", "bfloat16"):
        return SPA_BF16
    raise ValueError(f"unsupported dtype {dtype!r}")


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype_code(dtype) == SPA_BF16 else torch.float32


def make_shape(s) -> spa_shape:
    """spa_shape from any object with the LayerShape attributes (batch, n_tokens, ..., dtype, norm_eps,
    optionally rope_theta)."""
    return spa_shape(int(s.batch), int(s.n_tokens), int(s.d_model), int(s.n_q_heads), int(s.n_kv_heads),
                     int(s.head_dim), int(s.d_ffn), int(s.rank), dtype_code(s.dtype), float(s.norm_eps),
                     float(getattr(s, "rope_theta", 0.0)))


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


class DeviceWeights(NamedTuple):
    """Layer weights on the device, fragment-packed as spa_layer_weights wants them (the RMSNorm gains
    folded into w_qkv and w_gate_up)."""
    w_r: object        # r x d
    w_qkv: object      # (d_q + 2 d_kv) x d, times diag(g_attn)
    w_o: object        # d x d_q
    w_gate_up: object  # 2F x d, times diag(g_ffn)
    w_down: object     # d x F
    b_qkv: object = None  # optional d_q + 2 d_kv biases [b_q; b_k; b_v] (plain vector, storage dtype)


class DeviceCache(NamedTuple):
    k: object  # B x H_kv x N x hd
    v: object  # B x H_kv x N x hd
    h: object  # B x N x d
    p: object  # B x N x r float32


def _check_bytes(t, need: int, name: str):
    have = t.numel() * t.element_size()
    if have < need:
        raise ValueError(f"{name} holds {have} bytes, needs {need} (weights must be fragment-packed: spa_pack_weight)")


def _weights_struct(w: DeviceWeights, tdt, shape=None) -> spa_layer_weights:
    if shape is not None:   # every matrix must be the packed size the kernels will read
        s = shape
        dq, dkv = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
        need = {"w_r": (s.rank, s.d_model, SPA_PACK_PLAIN), "w_qkv": (dq + 2 * dkv, s.d_model, SPA_PACK_PLAIN),
                "w_o": (s.d_model, dq, SPA_PACK_PLAIN), "w_gate_up": (2 * s.d_ffn, s.d_model, SPA_PACK_GATE_UP),
                "w_down": (s.d_model, s.d_ffn, SPA_PACK_PLAIN)}
        for f, (r, c, kind) in need.items():
            _check_bytes(getattr(w, f), spa_packed_weight_bytes(s.dtype, r, c, kind), f)
    if w.b_qkv is not None and shape is not None:
        s = shape
        need = (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim
        if w.b_qkv.dim() != 1 or w.b_qkv.numel() != need:
            raise ValueError(f"b_qkv must be a vector of {need} biases")
    return spa_layer_weights(*(_ptr(getattr(w, f), tdt, f) for f in DeviceWeights._fields))


def _cache_struct(c: DeviceCache, tdt) -> spa_layer_cache:
    import torch
    return spa_layer_cache(_ptr(c.k, tdt, "k_cache"), _ptr(c.v, tdt, "v_cache"), _ptr(c.h, tdt, "h_cache"),
                           _ptr(c.p, torch.float32, "p_cache"))


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws, None, "workspace"), int(ws.numel() * ws.element_size())


# ----------------------------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------------------------
def spa_budget(n_layers: int, l_peak: int, rho_peak: float, rho_first: float, rho_last: float,
               n_tokens: int) -> Tuple[list, list]:
    lib = load_library()
    rho = (ctypes.c_double * n_layers)()
    k = (ctypes.c_int32 * n_layers)()
    _check(lib.spa_budget(n_layers, l_peak, rho_peak, rho_first, rho_last, n_tokens,
                          ctypes.cast(rho, ctypes.c_void_p), ctypes.cast(k, ctypes.c_void_p)), "spa_budget")
    return list(rho), list(k)


def spa_workspace_bytes(shape, k_max: int) -> int:
    out = ctypes.c_size_t(0)
    s = make_shape(shape)
    _check(load_library().spa_workspace_bytes(ctypes.byref(s), int(k_max), ctypes.byref(out)),
           "spa_workspace_bytes")
    return int(out.value)


def alloc_workspace(shape, k_max: int, device="cuda"):
    import torch
    return torch.empty(spa_workspace_bytes(shape, k_max), dtype=torch.uint8, device=device)


def spa_layer_full(shape, w: DeviceWeights, cache: DeviceCache, h_in, ws, stream=None):
    tdt = torch_dtype(shape.dtype)
    s = make_shape(shape)
    wp, wb = _ws(ws)
    ws_ = _weights_struct(w, tdt, shape)
    cs = _cache_struct(cache, tdt)
    _check(load_library().spa_layer_full(ctypes.byref(s), ctypes.byref(ws_), ctypes.byref(cs), _ptr(h_in, tdt, "h_in"),
                                         wp, wb, _stream(stream)), "spa_layer_full")


def spa_layer_step(shape, w: DeviceWeights, cache: DeviceCache, h_in, k: int, policy: int, idx_out,
                   scores_out, ws, stream=None):
    import torch
    tdt = torch_dtype(shape.dtype)
    s = make_shape(shape)
    wp, wb = _ws(ws)
    ws_ = _weights_struct(w, tdt, shape)
    cs = _cache_struct(cache, tdt)
    _check(load_library().spa_layer_step(ctypes.byref(s), ctypes.byref(ws_), ctypes.byref(cs), _ptr(h_in, tdt, "h_in"),
                                         int(k), int(policy), _ptr(idx_out, torch.int32, "idx_out"),
                                         _ptr(scores_out, torch.float32, "scores_out"), wp, wb, _stream(stream)),
           "spa_layer_step")


def spa_layer_step_noalloc(shape, w: DeviceWeights, cache: DeviceCache, h_in, k: int, policy: int, idx_out,
                           scores_out, stream=None):
    """spa_layer_step on the library's static device scratch (no workspace argument, nothing allocated)."""
    import torch
    tdt = torch_dtype(shape.dtype)
    s = make_shape(shape)
    ws_ = _weights_struct(w, tdt, shape)
    cs = _cache_struct(cache, tdt)
    _check(load_library().spa_layer_step_noalloc(ctypes.byref(s), ctypes.byref(ws_), ctypes.byref(cs),
                                                 _ptr(h_in, tdt, "h_in"), int(k), int(policy),
                                                 _ptr(idx_out, torch.int32, "idx_out"),
                                                 _ptr(scores_out, torch.float32, "scores_out"), _stream(stream)),
           "spa_layer_step_noalloc")


class HipEvents:
    """`n` HIP timing events (created through the HIP runtime) for spa_layer_step_timed."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.n = n
        self.events = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            # no system-scope fence when an event completes: the marks sit between kernels of one
            # stream and are only read back on the host after a synchronize
            if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events[i] = ev
        self.names = (ctypes.c_char_p * max(n - 1, 1))()

    def timing(self) -> spa_timing:
        return spa_timing(ctypes.cast(self.events, ctypes.c_void_p), self.n, 0,
                          ctypes.cast(self.names, ctypes.c_void_p))

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float(0.0)
        if self.hip.hipEventSynchronize(ctypes.c_void_p(self.events[j])) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.events[i]),
                                        ctypes.c_void_p(self.events[j])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(ctypes.c_void_p(self.events[i]))


def spa_layer_step_timed(shape, w: DeviceWeights, cache: DeviceCache, h_in, k: int, policy: int, idx_out,
                         scores_out, ws, events: HipEvents, stream=None):
    """spa_layer_step with an event after every kernel; returns [(kernel name, duration ms), ...]."""
    import torch
    tdt = torch_dtype(shape.dtype)
    s = make_shape(shape)
    wp, wb = _ws(ws)
    ws_ = _weights_struct(w, tdt, shape)
    cs = _cache_struct(cache, tdt)
    t = events.timing()
    _check(load_library().spa_layer_step_timed(ctypes.byref(s), ctypes.byref(ws_), ctypes.byref(cs),
                                               _ptr(h_in, tdt, "h_in"), int(k), int(policy),
                                               _ptr(idx_out, torch.int32, "idx_out"),
                                               _ptr(scores_out, torch.float32, "scores_out"), wp, wb,
                                               _stream(stream), ctypes.byref(t)), "spa_layer_step_timed")
    return [(events.names[i].decode(), events.elapsed_ms(i, i + 1)) for i in range(t.count - 1)]


def spa_identify(shape, h_in, w_r, p_cache, p_out, scores_out, ws, stream=None):
    import torch
    tdt = torch_dtype(shape.dtype)
    s = make_shape(shape)
    wp, wb = _ws(ws)
    _check_bytes(w_r, spa_packed_weight_bytes(shape.dtype, shape.rank, shape.d_model), "w_r")
    _check(load_library().spa_identify(ctypes.byref(s), _ptr(h_in, tdt, "h_in"), _ptr(w_r, tdt, "w_r"),
                                       _ptr(p_cache, torch.float32, "p_cache"), _ptr(p_out, torch.float32, "p_out"),
                                       _ptr(scores_out, torch.float32, "scores_out"), wp, wb, _stream(stream)),
           "spa_identify")


def spa_topk(scores, k: int, idx_out, stream=None):
    import torch
    if scores.dim() != 2:
        raise ValueError("scores must be batch x n")
    b, n = scores.shape
    _check(load_library().spa_topk(int(b), int(n), _ptr(scores, torch.float32, "scores"), int(k),
                                   _ptr(idx_out, torch.int32, "idx_out"), _stream(stream)), "spa_topk")


def spa_sparse_update(shape, w: DeviceWeights, cache: DeviceCache, h_in, idx, ws, stream=None):
    import torch
    tdt = torch_dtype(shape.dtype)
    s = make_shape(shape)
    wp, wb = _ws(ws)
    k = int(idx.shape[-1]) if idx is not None else 0
    ws_ = _weights_struct(w, tdt, shape)
    cs = _cache_struct(cache, tdt)
    _check(load_library().spa_sparse_update(ctypes.byref(s), ctypes.byref(ws_), ctypes.byref(cs),
                                            _ptr(h_in, tdt, "h_in"), _ptr(idx, torch.int32, "idx"), k, wp, wb,
                                            _stream(stream)), "spa_sparse_update")


def spa_attend(shape, q, m_per_seq: int, k_cache, v_cache, o_out, stream=None):
    tdt = torch_dtype(shape.dtype)
    s = make_shape(shape)
    _check(load_library().spa_attend(ctypes.byref(s), _ptr(q, tdt, "q"), int(m_per_seq), _ptr(k_cache, tdt, "k_cache"),
                                     _ptr(v_cache, tdt, "v_cache"), _ptr(o_out, tdt, "o_out"), _stream(stream)),
           "spa_attend")


# ----------------------------------------------------------------------------------------------
# device buffers (plumbing: torch allocates, the library computes)
# ----------------------------------------------------------------------------------------------
def spa_packed_weight_bytes(dtype, rows: int, cols: int, kind: int = SPA_PACK_PLAIN) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().spa_packed_weight_bytes(dtype_code(dtype), int(rows), int(cols), int(kind),
                                                  ctypes.byref(out)), "spa_packed_weight_bytes")
    return int(out.value)


def spa_pack_weight(mat, kind: int = SPA_PACK_PLAIN, col_scale=None, stream=None):
    """Fragment-packed copy (1-D device tensor) of a row-major device matrix [rows][cols] (y = x W^T),
    optionally of W diag(col_scale) (col_scale: device vector of cols entries, same dtype)."""
    import torch
    if mat.dim() != 2:
        raise ValueError("weight must be a matrix")
    dt = "bf16" if mat.dtype == torch.bfloat16 else "f32"
    rows, cols = mat.shape
    if col_scale is not None and (col_scale.dim() != 1 or col_scale.numel() != cols):
        raise ValueError("col_scale must be a vector of one entry per column")
    nbytes = spa_packed_weight_bytes(dt, rows, cols, kind)
    dst = torch.empty(nbytes // mat.element_size(), dtype=mat.dtype, device=mat.device)
    scale_ptr = None if col_scale is None else _ptr(col_scale, mat.dtype, "col_scale")
    _check(load_library().spa_pack_weight(dtype_code(dt), int(rows), int(cols), int(kind), _ptr(mat, None, "weight"),
                                          scale_ptr, _ptr(dst, None, "packed"), _stream(stream)), "spa_pack_weight")
    return dst


def upload_weights(w: dict, w_r, dtype, device="cuda") -> DeviceWeights:
    """Device weights from host arrays (numpy or torch), packed for the GEMMs: [W_q; W_k; W_v] with the
    attention RMSNorm gain folded in, W_o, [W_gate; W_up] (gate/up interleave) with the FFN RMSNorm gain
    folded in, W_down and W_r."""
    import numpy as np
    import torch
    tdt = torch_dtype(dtype)

    def dev(a):
        t = torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)) if not isinstance(a, torch.Tensor) else a
        return t.to(device=device, dtype=tdt).contiguous()

    g_attn, g_ffn = dev(w["g_attn"]), dev(w["g_ffn"])
    qkv = spa_pack_weight(torch.cat([dev(w["w_q"]), dev(w["w_k"]), dev(w["w_v"])], 0).contiguous(),
                          col_scale=g_attn)
    gu = spa_pack_weight(torch.cat([dev(w["w_gate"]), dev(w["w_up"])], 0).contiguous(), SPA_PACK_GATE_UP,
                         col_scale=g_ffn)
    b_qkv = None
    if "b_q" in w:   # q, k, v biases, added after the normalisation (not scaled by the gain)
        b_qkv = torch.cat([dev(w["b_q"]).reshape(-1), dev(w["b_k"]).reshape(-1), dev(w["b_v"]).reshape(-1)]).contiguous()
    out = DeviceWeights(spa_pack_weight(dev(w_r)), qkv, spa_pack_weight(dev(w["w_o"])), gu,
                        spa_pack_weight(dev(w["w_down"])), b_qkv)
    torch.cuda.current_stream().synchronize()   # the row-major staging copies are freed after packing
    return out


def alloc_cache(shape, device="cuda") -> DeviceCache:
    import torch
    tdt = torch_dtype(shape.dtype)
    b, n = shape.batch, shape.n_tokens
    return DeviceCache(torch.zeros(b, shape.n_kv_heads, n, shape.head_dim, dtype=tdt, device=device),
                       torch.zeros(b, shape.n_kv_heads, n, shape.head_dim, dtype=tdt, device=device),
                       torch.zeros(b, n, shape.d_model, dtype=tdt, device=device),
                       torch.zeros(b, n, shape.rank, dtype=torch.float32, device=device))
