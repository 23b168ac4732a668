"""SPA-Cache per-layer decoding step on MI355X (gfx950): HIP kernels behind the libspacache C ABI.

The package holds the kernels (csrc/), the build script (build.py), the ctypes binding (binding.py)
and the offline singular-proxy preparation (offline.py).
"""
from .binding import (  # noqa: F401
    EXPORTS, LIB_PATH, SPA_BF16, SPA_F32, SPA_PACK_GATE_UP, SPA_PACK_PLAIN, SPA_PROXY_WRITE_ALL, SPA_PROXY_WRITE_SELECTED, DeviceCache,
    DeviceWeights, HipEvents, SpaError, alloc_cache, alloc_workspace, load_library, make_shape, spa_attend, spa_budget,
    spa_identify, spa_layer_full, spa_layer_step, spa_layer_step_noalloc, spa_layer_step_timed, spa_pack_weight, spa_packed_weight_bytes, spa_sparse_update, spa_status_string, spa_topk,
    spa_workspace_bytes, torch_dtype, upload_weights,
)
from .offline import singular_proxy_from_factors, singular_proxy_weights  # noqa: F401
