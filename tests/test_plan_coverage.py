"""Every kernel instance the workloads run is reached by a GPU parity test (host logic, no GPU).

The kernel planners (tests/planner_check.hip, built with hipcc and run on the CPU) list, for each
library call, the instances it launches: GEMM kernel and tile, split-K or not, one or several column
tiles, a ragged last row tile or not; the identification variant (Top-k fused into the cosine kernel
or separate, keys per thread, ranks past one pass per wave); the attention kernel, dtype, head dim,
GQA and ragged query blocks. The workloads' calls are those the bench runs (every layer's k_l of the
stacks under the adaptive and the uniform budget, every proxy rank it sweeps or offers, the full
recomputes); the parity calls are those of tests/test_gpu_parity.py (tests/parity_cases.py).
"""
import os
import shutil
import subprocess

import pytest

import oracle
import synth
from parity_cases import parity_calls

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("plan") / "planner_check")
    subprocess.run([hipcc, "-O1", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-o", exe, os.path.join(HERE, "planner_check.hip")], check=True,
                   capture_output=True, timeout=600)
    return exe


def _line(tag, s, k, mode):
    return (f"{tag} {s.dtype} {s.batch} {s.n_tokens} {s.d_model} {s.n_q_heads} {s.n_kv_heads} {s.head_dim} "
            f"{s.d_ffn} {s.rank} {k} {mode}")


def instance_keys(exe, calls):
    """{key: [tag of a call that reaches it, ...]} for calls (shape, k, mode)."""
    text = "\n".join(_line(f"c{i}", s, k, m) for i, (s, k, m) in enumerate(calls)) + "\n"
    out = subprocess.run([exe, "instances"], input=text, capture_output=True, text=True, timeout=120, check=True).stdout
    keys = {}
    for ln in out.splitlines():
        assert not ln.startswith("BAD"), ln
        tag, *ks = ln.split()
        for key in ks:
            keys.setdefault(key, []).append(int(tag[1:]))
    return keys


def workload_calls():
    """The library calls of the five workloads as the bench runs them."""
    calls = []
    for name in ("tiny-f32", "llada-layer"):
        wl = synth.WORKLOADS[name]
        k = int(oracle.budget(1, 1, wl.rho, wl.rho, wl.rho, wl.shape.n_tokens)[1][0])
        calls += [(wl.shape, k, "step"), (wl.shape, 0, "full")]
    for name, ranks in (("llada-stack", (64, 128, 256, 512)), ("dream-stack", (128, 256))):
        wl = synth.WORKLOADS[name]
        s = wl.shape
        rho_p, l_p, rho_1, rho_l = wl.budget
        rho, ks = oracle.budget(wl.n_layers, l_p, rho_p, rho_1, rho_l, s.n_tokens)
        mean = float(rho.mean())
        k_uniform = int(oracle.budget(1, 1, mean, mean, mean, s.n_tokens)[1][0])
        for r in list(ranks) + [s.d_kv]:           # the proxy ranks and the full Value identifier
            sr = s.replace(rank=r)
            calls += [(sr, int(k), "step") for k in sorted(set(ks.tolist()) | {k_uniform})]
            calls.append((sr, 0, "full"))
    wl = synth.WORKLOADS["batched-stress"]
    for r in (64, 128, 512):
        sr = wl.shape.replace(rank=r)
        for rho in (0.08, 0.16, 0.25, 1.0):
            calls.append((sr, int(oracle.budget(1, 1, rho, rho, rho, sr.n_tokens)[1][0]), "step"))
        calls.append((sr, 0, "full"))
    return calls


@pytest.mark.slow
def test_every_workload_instance_has_a_parity_test(checker):
    work = workload_calls()
    par = parity_calls()
    wk = instance_keys(checker, work)
    pk = instance_keys(checker, par)
    missing = sorted(set(wk) - set(pk))
    detail = []
    for key in missing:
        s, k, mode = work[wk[key][0]]
        detail.append(f"{key}  (e.g. {mode} k={k} of B={s.batch} N={s.n_tokens} d={s.d_model} r={s.rank})")
    assert not missing, "kernel instances no parity test reaches:\n" + "\n".join(detail)
