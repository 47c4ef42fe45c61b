"""The layer step (schedule, forward with saved context, backward) enqueues
only kernels on the caller's stream, with no allocation, memset or host sync,
so it can be captured in a HIP graph and replayed. Every replay must give
bitwise the results of the eager step; replays are interleaved with eager
work and synchronisations, and one replay follows an in-place change of the
inputs (the graph reads the buffers it was captured with). Also with the
persistent driver and with the single-launch forward."""
import numpy as np
import pytest

from moe_testlib import to_dev_bf16
from synthetic import make_dy, problem
from test_gpu_forward import device_inputs

pytestmark = pytest.mark.gpu


class Step:
    """Buffers of one layer step; run() enqueues schedule + forward + backward."""

    def __init__(self, p, d, dy_bits, mx, kind="default"):
        import torch
        import mixture_experts_layer_30_amd as mok
        from mixture_experts_layer_30_amd import functional as F
        self.mok = mok
        self.kind = kind
        dtype = mok.MOK_MXFP8 if mx else mok.MOK_BF16
        cfg = dict(driver=2) if kind == "persistent" else {}
        self.ws = F.get_workspace(p.T, p.H, p.I, p.E, p.k, dtype=dtype, training=True, **cfg)
        self.d = d
        if mx:
            self.wts = F.quantize_weights(*d["weights"]) + F.quantize_weights_backward(*d["weights"])
        else:
            self.wts = d["weights"]
        self.dy = to_dev_bf16(dy_bits)
        wg, wu, wd = d["weights"]
        self.y = torch.empty_like(d["x"])
        self.dx = torch.empty_like(d["x"])
        self.dwg, self.dwu, self.dwd = torch.empty_like(wg), torch.empty_like(wu), torch.empty_like(wd)
        self.dtw = torch.empty_like(d["w"])

    def run(self):
        mok, ws, d = self.mok, self.ws, self.d
        if self.kind == "single-launch":
            mok.forward_fused(ws.problem, d["ids"], ws.schedule, d["x"], d["w"], self.wts, self.y, ws.workspace,
                              ws.fwd_ctx, ws.config)
        else:
            mok.build_schedule(ws.problem, d["ids"], ws.schedule, ws.config)
            mok.forward(ws.problem, ws.schedule, d["x"], d["w"], self.wts, self.y, ws.workspace, ws.fwd_ctx,
                        ws.config)
        mok.backward(ws.problem, ws.schedule, ws.fwd_ctx, d["x"], d["w"], self.wts, self.dy, self.dx,
                     self.dwg, self.dwu, self.dwd, self.dtw, ws.workspace, ws.config)

    def outputs(self):
        return [t.clone() for t in (self.y, self.dx, self.dwg, self.dwu, self.dwd, self.dtw)]


def _bits(ts):
    import torch
    return [t.contiguous().view(-1).view(torch.uint8).cpu().numpy().copy() for t in ts]


@pytest.mark.parametrize("mx,kind", [(False, "default"), (True, "default"), (False, "persistent"),
                                     (False, "single-launch")],
                         ids=["bf16", "mxfp8", "bf16-persistent", "bf16-single-launch"])
def test_step_replays_bitwise_in_a_hip_graph(mx, kind):
    """(persistent, single-launch: the forward's counters are cleared by fill
    kernels captured with it, so every replay starts from zero counters)"""
    import torch
    p = problem(300, 256, 384, 16, 4, seed=61)
    print(f"[graph] mx={mx} {kind}", flush=True)
    d = device_inputs(p)
    step = Step(p, d, make_dy(p), mx, kind)

    step.run()
    torch.cuda.synchronize()
    ref = _bits(step.outputs())

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step.run()

    for rep in range(3):
        for t in (step.y, step.dx, step.dwg, step.dwu, step.dwd, step.dtw):
            t.zero_()                                # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _bits(step.outputs())
        for i, (u, v) in enumerate(zip(got, ref)):
            assert np.array_equal(u, v), f"replay {rep}: output {i} differs from the eager step"

    # new inputs in the captured buffers: the replay must follow them
    x2 = to_dev_bf16(make_dy(problem(300, 256, 384, 16, 4, seed=62)))
    d["x"].copy_(x2)
    step.run()
    torch.cuda.synchronize()
    ref2 = _bits(step.outputs())
    assert any(not np.array_equal(u, v) for u, v in zip(ref2, ref)), "new x must change the step"
    for t in (step.y, step.dx, step.dwg, step.dwu, step.dwd, step.dtw):
        t.zero_()
    g.replay()
    torch.cuda.synchronize()
    for i, (u, v) in enumerate(zip(_bits(step.outputs()), ref2)):
        assert np.array_equal(u, v), f"replay after new x: output {i} differs from the eager step"
