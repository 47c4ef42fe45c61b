"""The launch tracer (mok_trace_enable / mok_trace_collect) that bench.py uses
for per-kernel times: every launch of a step is recorded under its name, the
times are positive and together stay within the elapsed time (consecutive
launches of one call share the event between them), and tracing does not
change any result."""
import numpy as np
import pytest

from synthetic import make_dy, problem
from test_gpu_forward import device_inputs
from test_gpu_graph import Step, _bits

pytestmark = pytest.mark.gpu


def test_trace_counts_launches_and_times_fit_the_step():
    import torch
    import mixture_experts_layer_30_amd as mok
    p = problem(300, 256, 384, 16, 4, seed=71)
    step = Step(p, device_inputs(p), make_dy(p), mx=False)
    step.run()
    torch.cuda.synchronize()
    ref = _bits(step.outputs())

    mok.trace_collect()                               # drop anything recorded before
    n = 3
    mok.trace_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        step.run()
    e1.record()
    torch.cuda.synchronize()
    mok.trace_enable(False)
    stats = mok.trace_collect()
    elapsed = e0.elapsed_time(e1)

    expect = {"schedule", "gateup_gemm", "down_gemm", "combine", "reverse_combine",
              "bwd_dh_gemm", "bwd_dwd_gemm", "bwd_dwgu_gemm", "bwd_dx_gemm", "reverse_dispatch"}
    assert expect <= set(stats), sorted(stats)
    for name in expect:
        launches, total, mx = stats[name]
        assert launches == n, (name, launches)      # one ring group: one launch per step
        assert total > 0 and mx > 0 and mx <= total + 1e-9, (name, total, mx)
    traced = sum(v[1] for v in stats.values())
    # the chained events cover each call's launches back to back, so the
    # per-kernel times are disjoint pieces of the elapsed time (the gaps
    # between calls are not traced)
    assert 0 < traced <= elapsed * 1.02, (traced, elapsed)
    assert mok.trace_collect() == {}, "collect clears the record"

    for u, v in zip(_bits(step.outputs()), ref):
        assert np.array_equal(u, v), "tracing must not change the results"
