"""GPU parity of the bf16 backward (dx, dWg, dWu, dWd, d topk_w) against the fp64
oracle, plus bitwise determinism. Small cases compare every output; the
large-hidden workload compares sampled tokens and a few whole experts."""
import numpy as np
import pytest

import oracle
from moe_testlib import ExpertsF64, assert_close_bf16, f64, from_dev_bf16, to_dev_bf16
from synthetic import CONFIGS, make_dy, problem
from test_gpu_forward import device_inputs, host_inputs, sampled_tokens

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(p, d, dy_bits, **cfg):
    import torch
    from mixture_experts_layer_30_amd import functional as F
    ws = F.get_workspace(p.T, p.H, p.I, p.E, p.k, training=True, **cfg)
    F.run_schedule(ws, d["ids"])
    y = F.run_forward(ws, d["x"], d["w"], d["weights"])
    out = F.run_backward(ws, d["x"], d["w"], d["weights"], to_dev_bf16(dy_bits))
    torch.cuda.synchronize()
    return y, out


SMALL = [
    problem(37, 256, 256, 5, 2, seed=41),
    problem(300, 128, 384, 16, 4, seed=42),
    problem(200, 384, 256, 12, 3, seed=43),
    problem(300, 128, 128, 512, 8, seed=46),    # the most experts: ~5 rows each, many empty
    problem(37, 256, 128, 4, 4, seed=47),       # k = E: every token routed to every expert
]


@pytest.mark.parametrize("p", SMALL, ids=lambda p: p.name)
def test_small_backward_matches_oracle(p):
    x, ids, w, wg, wu, wd = host_inputs(p)
    dy = make_dy(p)
    _, (dx, dwg, dwu, dwd, dtw) = gpu_fwd_bwd(p, device_inputs(p), dy)
    ref = oracle.backward(f64(x), ids, w.astype(np.float64), ExpertsF64(wg, wu, wd), f64(dy))
    assert_close_bf16(from_dev_bf16(dx), ref["dx"], "dx")
    assert_close_bf16(dtw.cpu().numpy().astype(np.float64), ref["dw"], "d topk_w")
    for e in range(p.E):
        for name, got in (("dWg", dwg), ("dWu", dwu), ("dWd", dwd)):
            g = from_dev_bf16(got[e])
            if not ref[name][e].any():
                assert not g.any(), f"{name}[{e}] of an empty expert must be exactly zero"
            else:
                assert_close_bf16(g, ref[name][e], f"{name}[{e}]")


def test_empty_experts_exact_zero_gradients():
    p = problem(64, 128, 128, 6, 2, seed=44)
    x, ids, w, wg, wu, wd = host_inputs(p)
    ids2 = np.stack([np.full(64, 1), np.where(np.arange(64) % 2 == 0, 3, 4)], axis=1)
    dy = make_dy(p)
    d = device_inputs(p, ids2)
    _, (dx, dwg, dwu, dwd, dtw) = gpu_fwd_bwd(p, d, dy)
    for e in (0, 2, 5):
        for t in (dwg, dwu, dwd):
            assert not from_dev_bf16(t[e]).any()
    ref = oracle.backward(f64(x), ids2, w.astype(np.float64), ExpertsF64(wg, wu, wd), f64(dy))
    assert_close_bf16(from_dev_bf16(dx), ref["dx"], "dx")


def test_backward_one_hot_expert_invalid_ids_and_ragged_token_axis():
    """The weight-gradient GEMMs read x and dY rows in place through the
    schedule's token table, 64 token rows per pair: experts here hold 199
    rows (3 full pairs + 7), 64 and 65 rows (a pair boundary and one row past
    it), 1 row, 69 rows, and none. Two ids are out of range: their rows get
    no expert output, d topk_w 0 and no dx contribution."""
    p = problem(200, 256, 384, 7, 2, seed=45)
    x, ids, w, wg, wu, wd = host_inputs(p)
    j1 = np.full(200, 6)
    j1[:64] = 2
    j1[64:129] = 3
    j1[129] = 5
    ids2 = np.stack([np.full(200, 4), j1], axis=1)
    ids2[180, 1] = 99
    ids2[150, 0] = -1
    dy = make_dy(p)
    _, (dx, dwg, dwu, dwd, dtw) = gpu_fwd_bwd(p, device_inputs(p, ids2), dy)
    ref = oracle.backward(f64(x), ids2, w.astype(np.float64), ExpertsF64(wg, wu, wd), f64(dy))
    got_dw = dtw.cpu().numpy()
    assert got_dw[180, 1] == 0.0 and got_dw[150, 0] == 0.0
    assert_close_bf16(from_dev_bf16(dx), ref["dx"], "dx")
    assert_close_bf16(got_dw.astype(np.float64), ref["dw"], "d topk_w")
    for e in range(p.E):
        for name, got in (("dWg", dwg), ("dWu", dwu), ("dWd", dwd)):
            g = from_dev_bf16(got[e])
            if not ref[name][e].any():
                assert not g.any(), f"{name}[{e}] of an empty expert must be exactly zero"
            else:
                assert_close_bf16(g, ref[name][e], f"{name}[{e}]")


@pytest.mark.timeout(900)
def test_large_hidden_fwd_bwd_sampled():
    """T=16384, H=7168, E=32, top-4, I=2048, Zipf(0.8) loads."""
    p = CONFIGS[4]
    x, ids, w, wg, wu, wd = host_inputs(p)
    dy = make_dy(p)
    d = device_inputs(p)
    y, (dx, dwg, dwu, dwd, dtw) = gpu_fwd_bwd(p, d, dy)
    ex = ExpertsF64(wg, wu, wd)
    toks = sampled_tokens(p.T, 12, 4)
    yref, _ = oracle.forward_tokens(f64(x[toks]), ids[toks], w[toks].astype(np.float64), ex)
    assert_close_bf16(from_dev_bf16(y)[toks], yref, "y[sampled]")
    dxr, dwr = oracle.backward_tokens(f64(x[toks]), ids[toks], w[toks].astype(np.float64), ex,
                                      f64(dy[toks]))
    assert_close_bf16(from_dev_bf16(dx)[toks], dxr, "dx[sampled]")
    assert_close_bf16(dtw.cpu().numpy()[toks].astype(np.float64), dwr, "d topk_w[sampled]")
    # the least, a middle and the most loaded expert: the weight-gradient
    # GEMMs run K = the expert's rows (about 270 to 12000 here), so the
    # hottest expert takes the longest K loop the kernels ever run
    counts = np.bincount(ids.reshape(-1), minlength=p.E)
    order = np.argsort(counts, kind="stable")
    for e in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        print(f"expert {e}: {counts[e]} rows", flush=True)
        dg, du, dd = oracle.backward_expert_weights(e, f64(x), ids, w.astype(np.float64), ex, f64(dy))
        assert_close_bf16(from_dev_bf16(dwg[e]), dg, f"dWg[{e}]")
        assert_close_bf16(from_dev_bf16(dwu[e]), du, f"dWu[{e}]")
        assert_close_bf16(from_dev_bf16(dwd[e]), dd, f"dWd[{e}]")


@pytest.mark.timeout(900)
def test_large_hidden_step_bitwise_deterministic_10_runs():
    """The whole bf16 step (schedule, forward with context, backward) on
    T=16384, H=7168, E=32, top-4, I=2048 with Zipf(0.8) loads, run 10 times
    on the same buffers: every output bitwise equal to the first run's."""
    import torch
    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    p = CONFIGS[4]
    d = device_inputs(p)
    ddy = to_dev_bf16(make_dy(p))
    ws = F.get_workspace(p.T, p.H, p.I, p.E, p.k, training=True)
    wg, wu, wd = d["weights"]
    outs = [torch.empty_like(d["x"]), torch.empty_like(d["x"]), torch.empty_like(wg), torch.empty_like(wu),
            torch.empty_like(wd), torch.empty_like(d["w"])]
    ref = None
    for run in range(10):
        for o in outs:
            o.fill_(7)
        y, dx, dwg, dwu, dwd, dtw = outs
        F.run_schedule(ws, d["ids"])
        mok.forward(ws.problem, ws.schedule, d["x"], d["w"], d["weights"], y, ws.workspace, ws.fwd_ctx, ws.config)
        mok.backward(ws.problem, ws.schedule, ws.fwd_ctx, d["x"], d["w"], d["weights"], ddy, dx, dwg, dwu, dwd,
                     dtw, ws.workspace, ws.config)
        torch.cuda.synchronize()
        if ref is None:
            ref = [o.clone() for o in outs]
        else:
            for o, r in zip(outs, ref):
                assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"run {run} differs"


@pytest.mark.parametrize("p", [problem(300, 128, 384, 16, 4, seed=42), CONFIGS[4]], ids=lambda p: p.name)
def test_ring_configuration_leaves_every_output_bitwise_unchanged(p):
    """Each routed row's arithmetic does not depend on the minibatch, ring slot
    or tile it lands in, so y and every gradient are bitwise the same for any
    minibatch size and slot count: one minibatch (M = R), the default ring,
    many minibatches through one slot, and a ragged size through three."""
    import torch
    dy = make_dy(p)
    d = device_inputs(p)
    y0, out0 = gpu_fwd_bwd(p, d, dy, minibatch_rows=p.R, ring_slots=1)
    ref = [y0.clone()] + [t.clone() for t in out0]
    small = max(256, p.R // 16)
    for cfg in ({}, dict(minibatch_rows=small, ring_slots=1), dict(minibatch_rows=small + 128 * 3 + 64,
                                                                   ring_slots=3)):
        print(f"[ring] {p.name} {cfg}", flush=True)
        y, out = gpu_fwd_bwd(p, d, dy, **cfg)
        for name, a, b in zip(("y", "dx", "dWg", "dWu", "dWd", "d topk_w"), [y] + list(out), ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (cfg, name)


def test_backward_bitwise_deterministic():
    import torch
    p = problem(2048, 512, 256, 16, 4, seed=45, zipf_s=1.0)
    dy = make_dy(p)
    d = device_inputs(p)
    _, first = gpu_fwd_bwd(p, d, dy)
    ref = [t.clone() for t in first]
    for _ in range(9):
        _, out = gpu_fwd_bwd(p, d, dy)
        for a, b in zip(out, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_empty_input_forward_backward():
    """T = 0: the forward writes nothing (y is empty, passed as NULL) and the
    backward writes exact-zero weight gradients for every expert (all empty),
    over buffers that held other bytes."""
    import torch
    from mixture_experts_layer_30_amd import functional as F
    T, H, I, E, k = 0, 128, 256, 4, 2
    print("[backward] T=0", flush=True)
    ws = F.get_workspace(T, H, I, E, k, training=True)
    x = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, k), dtype=torch.int32, device="cuda")
    w = torch.empty((0, k), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(5)
    wts = tuple(torch.randn(s, generator=g).to(torch.bfloat16).cuda() for s in ((E, I, H), (E, I, H), (E, H, I)))
    F.run_schedule(ws, ids)
    y = F.run_forward(ws, x, w, wts)
    dy = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    dx, dtw = torch.empty_like(x), torch.empty_like(w)
    dwg, dwu, dwd = (torch.full_like(t, 3.0) for t in wts)
    F.backward(ws.problem, ws.schedule, ws.fwd_ctx, x, w, wts, dy, dx, dwg, dwu, dwd, dtw, ws.workspace, ws.config)
    torch.cuda.synchronize()
    assert y.shape == (0, H) and dx.shape == (0, H) and dtw.shape == (0, k)
    for name, t in (("dWg", dwg), ("dWu", dwu), ("dWd", dwd)):
        assert not t.view(torch.int16).any(), f"{name} of an empty layer must be exactly zero"
