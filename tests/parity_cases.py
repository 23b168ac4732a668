"""Shapes and row counts of the GPU parity tests, in one place.

tests/test_gpu_parity.py parametrizes its tests from these lists, and the host check
tests/test_plan_coverage.py reads the same lists (plus the one-off cases listed in
PARITY_SINGLE_CALLS) to verify that every kernel instance the workloads run is reached by some
parity test.
"""
import synth

SMALL_BF16 = [
    synth.LayerShape(2, 200, 256, 4, 4, 64, 688, 32, "bf16"),      # ragged N, K tail in W_down (688)
    synth.LayerShape(1, 333, 512, 8, 2, 128, 1024, 64, "bf16"),    # GQA, hd 128, ragged N
]
SMALL_STEP_K = [1, 37, 150]

FUSED_TOPK_SHAPES = [SMALL_BF16[0], SMALL_BF16[1],
                     synth.LayerShape(5, 3, 128, 2, 2, 64, 256, 16, "bf16"),
                     synth.LayerShape(3, 1030, 256, 4, 4, 64, 688, 32, "bf16"),
                     synth.LayerShape(2, 3000, 256, 4, 4, 64, 688, 32, "bf16"),
                     synth.LayerShape(1, 4100, 256, 4, 4, 64, 688, 32, "bf16"),
                     # rank 128 (the projection on 32-row tiles): tiles shared by sequences, several
                     # sequences completing in one workgroup of the cosine kernel
                     synth.LayerShape(5, 3, 128, 2, 2, 64, 256, 128, "bf16"),
                     synth.LayerShape(7, 45, 128, 2, 2, 64, 256, 128, "bf16"),
                     synth.LayerShape(3, 1030, 256, 4, 4, 64, 688, 128, "bf16"),
                     synth.LayerShape(2, 1500, 256, 4, 4, 64, 688, 128, "bf16"),
                     synth.LayerShape(1, 4000, 256, 4, 4, 64, 688, 128, "bf16")]


def fused_topk_ks(n):
    return sorted({1, n // 3, n - 1, n} - {0})


ROPE_STEP_CASES = [
    (synth.LayerShape(1, 333, 512, 8, 2, 128, 1024, 64, "bf16", rope_theta=1e6), 100),
    (synth.LayerShape(2, 200, 256, 4, 4, 64, 688, 32, "bf16", rope_theta=1e4), 37),
    (synth.LayerShape(1, 64, 256, 4, 4, 64, 688, 16, "f32", rope_theta=1e4), 16),
]

# spa_attend: (dtype, hd, hq, hkv, n keys, m queries), batch 2
ATTEND_CASES = [("bf16", 128, 4, 4, 1024, 256), ("bf16", 64, 6, 2, 77, 13), ("f32", 64, 4, 4, 64, 16),
                ("f32", 128, 2, 1, 100, 70), ("bf16", 128, 28, 4, 300, 65), ("bf16", 128, 28, 4, 2048, 100),
                ("bf16", 64, 8, 8, 999, 40), ("bf16", 128, 32, 32, 1024, 51),
                ("bf16", 128, 4, 2, 20, 5), ("bf16", 64, 2, 2, 1, 3)]   # fewer keys than one tile
# spa_attend with many packed rows per KV head (the packed kernel): (batch, hd, hq, hkv, n keys, m queries)
ATTEND_MANY_CASES = [(8, 128, 32, 32, 333, 450), (8, 128, 32, 4, 1024, 256), (4, 64, 64, 16, 100, 700),
                     (7, 128, 28, 4, 2047, 1000), (8, 128, 32, 4, 24, 300)]

# full-size workload layers
LLADA_EXACT_K = [51, 87, 123, 130, 200, 256]        # LLaDA stack row counts and the workload's k
DREAM_STACK_K = [102, 143, 163, 256, 311, 334, 360, 372, 428, 512]
BATCHED_EXACT_RHO = [0.08, 0.16]                   # k = 327, 655 at N = 4096
BATCHED_ID_RANKS = [64, 512]
LLADA_ID_RANKS = [64, 256, 512]                    # the LLaDA stack's other proxy ranks
# cached steps at another proxy rank (the stacks' rank sweep): (workload, rank, exactly k drifted rows)
RANK_STEP_CASES = [("llada", 256, 51), ("dream", 256, 102)]

LLADA = synth.WORKLOADS["llada-layer"].shape
DREAM = synth.WORKLOADS["dream-stack"].shape
BATCHED = synth.WORKLOADS["batched-stress"].shape
TINY = synth.WORKLOADS["tiny-f32"].shape

# The other library calls the GPU tests (and smoke) make, as (shape, k, mode): mode "step" (cached step
# with Top-k of k rows), "full" (spa_layer_full), "identify" (spa_identify), "sparse"
# (spa_sparse_update of k rows).
PARITY_SINGLE_CALLS = [
    (TINY, 16, "step"), (TINY, 0, "full"), (TINY, 0, "identify"),              # smoke, tiny-f32 config test
    (SMALL_BF16[0], 40, "step"),                                               # policy SELECTED
    (SMALL_BF16[0], 0, "step"), (SMALL_BF16[0], 200, "step"),                  # k = 0 and k = N
    (SMALL_BF16[0], 0, "full"), (SMALL_BF16[1], 0, "full"),                    # warm-up vs the oracle
    (SMALL_BF16[1], 333, "step"),                                              # rho = 1 vs the full recompute
    (SMALL_BF16[0], 0, "identify"), (SMALL_BF16[1], 0, "identify"),
    (SMALL_BF16[0], 23, "sparse"),                                             # unsorted / out-of-range indices
    (SMALL_BF16[0], 30, "step"),                                               # three-layer chain
    (synth.LayerShape(1, 333, 512, 8, 2, 128, 1024, 64, "bf16"), 83, "step"),  # graph replays
    (synth.LayerShape(1, 8192, 256, 4, 4, 64, 688, 32, "bf16"), 64, "step"),   # RoPE at positions to 8191
    (synth.LayerShape(2, 150, 512, 8, 2, 64, 1024, 32, "bf16"), 0, "full"),    # RoPE and biases, warm-up
    (synth.LayerShape(2, 200, 2048, 16, 16, 128, 1024, 2048, "bf16"), 0, "identify"),   # full Value identifier
    (synth.LayerShape(1, 256, 2048, 16, 16, 128, 1024, 2048, "bf16"), 64, "step"),
    (LLADA, 256, "step"),                                                      # the workload's own drift
    (LLADA.replace(rank=LLADA.d_kv), 0, "identify"),                           # full identifier, r = 4096
    (LLADA, 0, "full"),                                                        # the vanilla full recompute
    (DREAM, 512, "step"), (DREAM, 0, "full"),
    (DREAM.replace(rank=DREAM.d_kv), 102, "step"),                             # full identifier, r = 512
    (BATCHED, 1024, "step"),
]


def parity_calls():
    """Every (shape, k, mode) the GPU parity tests run through the library, plus the spa_attend calls
    as (shape, m, "attend")."""
    calls = list(PARITY_SINGLE_CALLS)
    for s in SMALL_BF16:
        calls += [(s, k, "step") for k in SMALL_STEP_K]
    for s in FUSED_TOPK_SHAPES:
        calls += [(s, k, "step") for k in fused_topk_ks(s.n_tokens)]
    calls += [(s, k, "step") for s, k in ROPE_STEP_CASES]
    calls += [(LLADA, k, "step") for k in LLADA_EXACT_K]
    calls += [(DREAM, k, "step") for k in DREAM_STACK_K]
    calls += [(BATCHED, int(BATCHED.n_tokens * rho + 1e-9), "step") for rho in BATCHED_EXACT_RHO]
    calls += [(BATCHED.replace(rank=r), 0, "identify") for r in BATCHED_ID_RANKS]
    calls += [(LLADA.replace(rank=r), 0, "identify") for r in LLADA_ID_RANKS]
    calls += [({"llada": LLADA, "dream": DREAM}[wl].replace(rank=r), k, "step") for wl, r, k in RANK_STEP_CASES]
    for dtype, hd, hq, hkv, n, m in ATTEND_CASES:
        calls.append((synth.LayerShape(2, n, 256, hq, hkv, hd, 256, 16, dtype), m, "attend"))
    for b, hd, hq, hkv, n, m in ATTEND_MANY_CASES:
        calls.append((synth.LayerShape(b, n, 256, hq, hkv, hd, 256, 16, "bf16"), m, "attend"))
    return calls
