"""Host logic of bench.py (no GPU): the graph replay bookkeeping of the layer bench, the identification
summary and the roofline arithmetic."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


class _Graph:
    def __init__(self, log, steps):
        self.log, self.steps = log, steps

    def replay(self):
        self.log.extend(self.steps)


@pytest.mark.parametrize("R,n_in", [(4, 8), (4, 7), (1, 5), (3, 2)])
@pytest.mark.parametrize("windows_on", [True, False])
def test_range_runner_replays_exactly_the_steps_in_order(R, n_in, windows_on):
    period = R * n_in

    def which(i):  # the bench's rotation: instance, input step
        return i % R, 1 + (i // R) % n_in

    log = []
    single = [_Graph(log, [which(g)]) for g in range(period)]  # graph g captured step g
    windows = [_Graph(log, [which(w + q) for q in range(R)]) for w in range(period)] if windows_on else None
    run = bench.range_runner(single, windows, None, R, n_in)
    for i0, n in [(0, 0), (0, 1), (3, 10), (5, 40), (10, 37), (period - 1, 2 * period + 3)]:
        log.clear()
        run(i0, n)
        assert log == [which(i) for i in range(i0, i0 + n)]


def test_range_runner_eager_fallback():
    seen = []
    run = bench.range_runner(None, None, seen.append, 4, 8)
    run(6, 9)
    assert seen == list(range(6, 15))


def test_consecutive_steps_visit_distinct_instances():
    R, n_in = 4, 8
    log = []
    single = [_Graph(log, [g % R]) for g in range(R * n_in)]
    bench.range_runner(single, None, None, R, n_in)(0, 3 * R * n_in)
    assert all(a != b for a, b in zip(log, log[1:]))


def test_identification_summary_arithmetic():
    work = {"proxy_gemm": (8_000_000, 1.0e9), "cosine_topk": (2_000_000, 0.0), "qkv_gemm_scatter": (1e8, 1e10)}
    per_us = {"proxy_gemm": 6.0, "cosine_topk": 4.0, "qkv_gemm_scatter": 40.0}
    out = bench.identification_summary(per_us, work, 0.2, 10.0)
    assert out["kernels"] == ["proxy_gemm", "cosine_topk"]
    assert out["us"] == 10.0 and out["share_of_step"] == 0.05
    assert out["GB/s"] == pytest.approx(1000.0)  # 10 MB in 10 us
    assert out["hbm_frac"] == pytest.approx(1000.0 / bench.PEAK_HBM_GBS, abs=1e-4)
    assert out["target_us"] == 10.0 and out["hbm_frac_target"] == 0.6
    assert bench.identification_summary({"qkv_gemm_scatter": 1.0}, work, 0.2) is None
