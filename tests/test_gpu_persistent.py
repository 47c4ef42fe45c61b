"""The persistent minibatch driver (driver=2) on the GPU: one resident grid
consumes the minibatches in order through the ring, gate/up and down tiles
waking each other through device counters ([MoK clip] Key points bullets 3-5,
How-to items 3-4; the plan is checked on the host by test_persist_plan.py).

Its results must be bitwise those of the one-launch-per-stage driver (which
workgroup runs a tile never changes what the tile computes) and match the
oracle; the status word must not carry the give-up bit. Small cases stress
slot reuse (one slot, many minibatches); the full-size cases run the bench
workload's forward with saved context, bf16 and MXFP8. The give-up path
itself is forced from the host with a zero wait limit: every workgroup must
leave, the bit must be set, and the next call must be exact again."""
import functools

import numpy as np
import pytest

import oracle
from moe_testlib import ExpertsF64, assert_close_bf16, f64, from_dev_bf16, to_dev_bf16
from synthetic import CONFIGS, make_all_experts, make_routing, make_x, problem

pytestmark = pytest.mark.gpu

GIVE_UP = 0x2      # MOK_STATUS_WATCHDOG


@functools.lru_cache(maxsize=2)
def host_inputs(p):
    x = make_x(p)
    ids, w = make_routing(p, x)
    wg, wu, wd = make_all_experts(p)
    return x, ids, w, wg, wu, wd


def device_inputs(p):
    import torch
    x, ids, w, wg, wu, wd = host_inputs(p)
    return dict(x=to_dev_bf16(x), ids=torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
                w=torch.from_numpy(w).cuda(), weights=(to_dev_bf16(wg), to_dev_bf16(wu), to_dev_bf16(wd)))


def run(p, d, training=False, dtype=None, weights=None, **cfg):
    import torch
    from mixture_experts_layer_30_amd import functional as F
    kw = {} if dtype is None else dict(dtype=dtype)
    ws = F.get_workspace(p.T, p.H, p.I, p.E, p.k, training=training, **kw, **cfg)
    F.run_schedule(ws, d["ids"])
    y = F.run_forward(ws, d["x"], d["w"], weights if weights is not None else d["weights"])
    torch.cuda.synchronize()
    status = F.read_schedule(ws)["status"]
    return y, ws, status


def same_bits(a, b):
    import torch
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


SMALL = [
    problem(37, 256, 256, 5, 2, seed=11),
    problem(300, 128, 384, 16, 4, seed=12),
    problem(1, 128, 128, 3, 3, seed=13),
    problem(64, 512, 128, 1, 1, seed=14),
]


@pytest.mark.parametrize("p", SMALL, ids=lambda p: p.name)
@pytest.mark.parametrize("cfg", [dict(), dict(minibatch_rows=64, ring_slots=1),
                                 dict(minibatch_rows=48, ring_slots=3)],
                         ids=["default", "M64-ring1", "M48-ring3"])
def test_small_persistent_matches_launch_per_stage_and_oracle(p, cfg):
    print(f"[persistent] {p.name} {cfg}", flush=True)
    d = device_inputs(p)
    y1, _, s1 = run(p, d, driver=1, **cfg)
    y2, _, s2 = run(p, d, driver=2, **cfg)
    assert not (s2 & GIVE_UP), f"status {s2:#x}"
    assert same_bits(y1, y2)
    x, ids, w, wg, wu, wd = host_inputs(p)
    ref, _ = oracle.forward(f64(x), ids, w.astype(np.float64), ExpertsF64(wg, wu, wd))
    assert_close_bf16(from_dev_bf16(y2), ref, "y")


def test_ring_reuse_many_minibatches_one_slot():
    # 1200 routed rows in 20 minibatches of 64 rows through one ring slot
    p = problem(300, 256, 256, 7, 4, seed=41)
    print(f"[persistent] {p.name} M64 ring1", flush=True)
    d = device_inputs(p)
    y1, _, _ = run(p, d, driver=1, minibatch_rows=64, ring_slots=1)
    y2, _, s2 = run(p, d, driver=2, minibatch_rows=64, ring_slots=1)
    assert not (s2 & GIVE_UP)
    assert same_bits(y1, y2)


@pytest.mark.timeout(900)
def test_full_size_persistent_bitwise_equal_with_context():
    # the bench workload: 8 minibatches of 8192 rows through 4 ring slots
    p = CONFIGS[4]
    print(f"[persistent] {p.name}", flush=True)
    d = device_inputs(p)
    y1, ws1, _ = run(p, d, training=True, driver=1)
    c1 = ws1.fwd_ctx.clone()
    y2, ws2, s2 = run(p, d, training=True, driver=2)
    assert not (s2 & GIVE_UP)
    assert same_bits(y1, y2)
    assert same_bits(c1, ws2.fwd_ctx)
    x, ids, w, wg, wu, wd = host_inputs(p)
    toks = np.array([0, 1, 4097, 9000, p.T - 1])
    ref, _ = oracle.forward_tokens(f64(x[toks]), ids[toks], w[toks].astype(np.float64), ExpertsF64(wg, wu, wd))
    assert_close_bf16(from_dev_bf16(y2)[toks], ref, "y[sampled]")


@pytest.mark.timeout(900)
def test_full_size_persistent_mxfp8_bitwise_equal():
    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    p = CONFIGS[4]
    print(f"[persistent] {p.name} mxfp8", flush=True)
    d = device_inputs(p)
    qw = F.quantize_weights(*d["weights"])
    y1, _, _ = run(p, d, dtype=mok.MOK_MXFP8, weights=qw, driver=1)
    y2, _, s2 = run(p, d, dtype=mok.MOK_MXFP8, weights=qw, driver=2)
    assert not (s2 & GIVE_UP)
    assert same_bits(y1, y2)


def test_persistent_bitwise_deterministic_10_runs():
    import torch
    p = CONFIGS[2]
    print(f"[persistent] {p.name} x10", flush=True)
    d = device_inputs(p)
    y0, _, _ = run(p, d, driver=2)
    ref = y0.view(torch.int16).clone()
    for _ in range(9):
        y, _, s = run(p, d, driver=2)
        assert not (s & GIVE_UP)
        assert torch.equal(y.view(torch.int16), ref)


@pytest.mark.parametrize("p", [SMALL[0], SMALL[1], CONFIGS[1]], ids=lambda p: p.name)
def test_agent_scope_sync_path_matches(p, monkeypatch):
    """The synchronisation a grid takes when some workgroup does not run on the
    XCD of its queue (every signal releases, every wait acquires at agent
    scope), forced on: driver 2 and the single launch stay bitwise equal to
    driver 1, the give-up bit clear."""
    import torch
    from mixture_experts_layer_30_amd import functional as F
    print(f"[persistent] {p.name} agent-scope sync", flush=True)
    d = device_inputs(p)
    cfg = dict(minibatch_rows=64, ring_slots=2) if p.T < 1000 else {}
    y1, ws1, _ = run(p, d, training=True, driver=1, **cfg)
    monkeypatch.setenv("MOK_PERSIST_AGENT_SYNC", "1")
    y2, ws2, s2 = run(p, d, training=True, driver=2, **cfg)
    assert not (s2 & GIVE_UP)
    assert same_bits(y1, y2)
    assert same_bits(ws1.fwd_ctx, ws2.fwd_ctx)
    ws3 = F.get_workspace(p.T, p.H, p.I, p.E, p.k, training=True, **cfg)
    y3 = F.run_forward_fused(ws3, d["ids"], d["x"], d["w"], d["weights"])
    torch.cuda.synchronize()
    assert not (F.read_schedule(ws3)["status"] & GIVE_UP)
    assert same_bits(y1, y3)
    assert same_bits(ws1.fwd_ctx, ws3.fwd_ctx)


def test_forced_give_up_ends_every_workgroup_and_recovers(monkeypatch):
    """Failure handling, forced from the host: with the wait limit set to 0
    ticks of the real-time counter (MOK_PERSIST_SPIN_TICKS=0), the first wait
    that is not met at once gives up. Every workgroup of driver 2 and of the
    single launch must then leave (the call completes), the status word must
    carry the give-up bit, and the next calls with the normal limit must give
    driver 1's results bitwise (the counters are cleared before each launch)."""
    import torch
    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    p = SMALL[1]
    print(f"[persistent] {p.name} forced give-up", flush=True)
    d = device_inputs(p)
    y1, _, _ = run(p, d, driver=1)
    monkeypatch.setenv("MOK_PERSIST_SPIN_TICKS", "0")
    _, _, s2 = run(p, d, driver=2)
    assert s2 & GIVE_UP, f"status {s2:#x}"
    ws3 = F.get_workspace(p.T, p.H, p.I, p.E, p.k)
    F.run_forward_fused(ws3, d["ids"], d["x"], d["w"], d["weights"])
    torch.cuda.synchronize()
    # (the schedule itself may be incomplete: read only its status word)
    off = mok.schedule_layout(ws3.problem, ws3.config).status
    assert int(ws3.schedule[off:off + 4].cpu().view(torch.int32)[0]) & GIVE_UP
    monkeypatch.delenv("MOK_PERSIST_SPIN_TICKS")
    y4, _, s4 = run(p, d, driver=2)
    assert not (s4 & GIVE_UP)
    assert same_bits(y1, y4)
    y5 = F.run_forward_fused(ws3, d["ids"], d["x"], d["w"], d["weights"])
    torch.cuda.synchronize()
    assert not (F.read_schedule(ws3)["status"] & GIVE_UP)
    assert same_bits(y1, y5)


def test_persistent_invalid_ids_match_launch_per_stage():
    """Rows with expert ids outside [0, E) are left out of every tile: driver 2
    stays bitwise equal to driver 1 (one slot, many minibatches), the bad-id
    bit set and the give-up bit clear."""
    import torch
    p = problem(200, 256, 128, 6, 2, seed=23)
    print(f"[persistent] {p.name} invalid ids", flush=True)
    d = device_inputs(p)
    ids = d["ids"].clone()
    ids[7, 1] = 99
    ids[150, 0] = -1
    ids[33, 0] = 6
    d = dict(d, ids=ids)
    y1, _, s1 = run(p, d, driver=1, minibatch_rows=64, ring_slots=1)
    y2, _, s2 = run(p, d, driver=2, minibatch_rows=64, ring_slots=1)
    assert s1 & 1 and s2 & 1 and not (s2 & GIVE_UP), f"status {s1:#x} {s2:#x}"
    assert same_bits(y1, y2)
    x, ids_h, w, wg, wu, wd = host_inputs(p)
    ids_h = ids.cpu().numpy()
    ref, _ = oracle.forward(f64(x), ids_h, w.astype(np.float64), ExpertsF64(wg, wu, wd))
    assert_close_bf16(from_dev_bf16(y2), ref, "y")
