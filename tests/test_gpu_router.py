"""GPU parity of the router front end against the fp64 oracle, through the C
ABI. The expert selection is an integer decision taken on fp32 logits, so the
device's ids must equal the oracle's wherever the oracle's scores separate
the k-th and (k+1)-th choice (and neighbours inside the selection) by more
than fp32 rounding can move them; inside such near-ties the device's choice
only has to be a valid top-k. Weights, d_sel and d_w_router are compared with
fp32 tolerances, dx (bf16) with the layer's bf16 bar; repeated runs must be
bitwise equal, and exact ties must go to the lower expert id."""
import numpy as np
import pytest

import oracle
from moe_testlib import assert_close_bf16, from_dev_bf16, rel_fro, to_dev_bf16
from synthetic import CONFIGS, bf16_to_f32, make_x, problem, router_weights

pytestmark = pytest.mark.gpu

# separation (relative to the scores' scale) above which the fp32 logits of
# the device cannot reorder two experts: |logit| error <= H * 2^-24 * sum|x||w|
TIE_MARGIN = 1e-4


def _inputs(p, with_bias):
    x = make_x(p)
    wr, bias = router_weights(p)                 # Wr [H][E] fp32, bias fp64 (zipf / empty experts)
    if not with_bias:
        bias = np.zeros(p.E)
    elif not bias.any():                         # a balancing-style bias of the logits' scale
        bias = 0.5 * np.random.default_rng(p.seed + 7).standard_normal(p.E)
    bias = np.where(np.isfinite(bias), bias, -1e30)   # the device takes finite fp32 biases
    return x, np.ascontiguousarray(wr.T), bias.astype(np.float32)


def _run(p, x, wr_eh, bias32):
    import torch
    import mixture_experts_layer_30_amd as mok
    prob = mok.make_problem(p.T, p.H, 128, p.E, p.k)
    dx_ = to_dev_bf16(x)
    dwr = torch.from_numpy(wr_eh).cuda()
    db = torch.from_numpy(bias32).cuda()
    ids = torch.empty((p.T, p.k), dtype=torch.int32, device="cuda")
    w = torch.empty((p.T, p.k), dtype=torch.float32, device="cuda")
    mok.router_forward(prob, dx_, dwr, db, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _check_selection(ids, w, logits, bias, k):
    score = logits + bias[None, :].astype(np.float64)
    scale = np.abs(logits).max(axis=1) + np.abs(bias[bias > -1e29]).max(initial=0.0) + 1e-30
    order = np.argsort(-score, axis=1, kind="stable")
    n_exact = 0
    for t in range(ids.shape[0]):
        s = score[t]
        got = ids[t].tolist()
        assert len(set(got)) == k and all(0 <= e < len(s) for e in got)
        # every pick scores at least the best non-pick, up to the margin
        rest = [e for e in range(len(s)) if e not in got]
        if rest:
            assert min(s[got]) >= max(s[rest]) - TIE_MARGIN * scale[t]
        # descending order up to the margin
        assert all(s[a] >= s[b] - TIE_MARGIN * scale[t] for a, b in zip(got, got[1:]))
        srt = np.sort(s)[::-1]
        gaps = np.diff(srt[:min(k + 1, len(s))])
        if len(gaps) == 0 or (-gaps).min() > TIE_MARGIN * scale[t]:
            assert got == order[t, :k].tolist(), (t, got, order[t, :k].tolist())
            n_exact += 1
    # weights: the softmax of the device-selected logits (fp64 oracle values)
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    ref_w = ex / ex.sum(axis=1, keepdims=True)
    assert np.allclose(w, ref_w, rtol=2e-5, atol=1e-7), float(np.abs(w - ref_w).max())
    return n_exact


CASES = [problem(37, 256, 128, 5, 2, seed=61), problem(300, 128, 128, 64, 8, seed=62),
         problem(200, 384, 128, 12, 3, seed=63), problem(64, 512, 128, 512, 8, seed=64),
         problem(129, 256, 128, 32, 4, seed=66, zipf_s=1.2, empty_den=4), problem(9, 128, 128, 6, 6, seed=67),
         problem(40, 256, 128, 128, 64, seed=68),      # E > 64 (round-based selection), maximum k
         problem(100, 256, 128, 100, 4, seed=70)]      # 64 < E <= 128 with k <= 8: the widest dense dWr tile


@pytest.mark.parametrize("with_bias", [False, True], ids=["nobias", "bias"])
@pytest.mark.parametrize("p", CASES, ids=lambda p: p.name)
def test_router_forward_matches_oracle(p, with_bias):
    x, wr_eh, bias = _inputs(p, with_bias)
    ids, w = _run(p, x, wr_eh, bias)
    logits, _, _ = oracle.router_forward(bf16_to_f32(x).astype(np.float64), wr_eh.astype(np.float64), None, p.k)
    n = _check_selection(ids, w, logits, bias, p.k)
    if p.k <= 8:                                 # with k = 64 of 128 some gap is often tiny
        assert n >= 0.8 * p.T                    # almost every token is far from a tie


def test_router_forward_full_size_and_deterministic():
    """Workload T=4096 H=2048 E=64 top-8: selections and weights as the oracle,
    bitwise the same over repeated runs."""
    p = CONFIGS[1]
    x, wr_eh, bias = _inputs(p, False)
    ids, w = _run(p, x, wr_eh, bias)
    for _ in range(3):
        ids2, w2 = _run(p, x, wr_eh, bias)
        assert np.array_equal(ids, ids2) and np.array_equal(w.view(np.uint32), w2.view(np.uint32))
    logits, _, _ = oracle.router_forward(bf16_to_f32(x).astype(np.float64), wr_eh.astype(np.float64), None, p.k)
    assert _check_selection(ids, w, logits, bias, p.k) >= 0.95 * p.T


@pytest.mark.parametrize("E,k", [(48, 6), (128, 8)])   # rank-count and round-based selection
def test_router_forward_64_token_workgroups_equal_16(E, k):
    """T >= 16384 with E <= 128 runs 64-token workgroups: every logit is the
    same sum in the same order as with 16-token workgroups, so ids and
    weights are bitwise those of the 16-token path (run on the first 16000
    tokens, below the switch), and match the oracle."""
    import dataclasses
    p = problem(16384, 1024, 128, E, k, seed=69)
    x, wr_eh, bias = _inputs(p, True)
    ids, w = _run(p, x, wr_eh, bias)
    q = dataclasses.replace(p, T=16000)
    ids16, w16 = _run(q, x[:16000], wr_eh, bias)
    assert np.array_equal(ids[:16000], ids16)
    assert np.array_equal(w[:16000].view(np.uint32), w16.view(np.uint32))
    ids2, w2 = _run(p, x, wr_eh, bias)
    assert np.array_equal(ids, ids2) and np.array_equal(w.view(np.uint32), w2.view(np.uint32))
    sub = np.r_[0:1000, 16000:16384]             # both kinds of workgroup, and the last one
    logits, _, _ = oracle.router_forward(bf16_to_f32(x[sub]).astype(np.float64), wr_eh.astype(np.float64), None, k)
    assert _check_selection(ids[sub], w[sub], logits, bias, k) >= 0.8 * len(sub)


@pytest.mark.parametrize("E,k", [(10, 3), (100, 40)])   # rank-count and round-based selection
def test_router_exact_ties_go_to_the_lower_id(E, k):
    import torch
    import mixture_experts_layer_30_amd as mok
    T, H = 16, 128
    rng = np.random.default_rng(65)
    x = make_x(problem(T, H, 128, E, k, seed=65))
    wr = rng.standard_normal((E, H)).astype(np.float32)
    wr[7] = wr[2]                                # experts 2 and 7 always tie
    wr[5] = wr[2]                                # ... and 5
    wr[2] *= 0                                   # (2 is now zero, 5 and 7 equal)
    wr[9] = wr[4]
    prob = mok.make_problem(T, H, 128, E, k)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    mok.router_forward(prob, to_dev_bf16(x), torch.from_numpy(wr).cuda(), None, ids, w)
    got = ids.cpu().numpy()
    n_tied = 0
    for t in range(T):
        sel = got[t].tolist()
        if 7 in sel:
            assert 5 in sel and sel.index(5) < sel.index(7)
        if 9 in sel:
            assert 4 in sel and sel.index(4) < sel.index(9)
        n_tied += (5 in sel and 7 in sel) + (4 in sel and 9 in sel)
    assert n_tied > 0                            # the tied pairs were reached


@pytest.mark.parametrize("p", CASES + [CONFIGS[1]], ids=lambda p: p.name)
def test_router_backward_matches_oracle(p):
    import torch
    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    x, wr_eh, bias = _inputs(p, True)
    ids, w = _run(p, x, wr_eh, bias)
    g = np.random.default_rng(p.seed + 100).standard_normal((p.T, p.k)).astype(np.float32)
    ws = F.get_workspace(p.T, p.H, 128, p.E, p.k, training=False)
    F.run_schedule(ws, torch.from_numpy(ids).cuda())
    prob = mok.make_problem(p.T, p.H, 128, p.E, p.k)
    d_sel = torch.empty((p.T, p.k), dtype=torch.float32, device="cuda")
    dx = torch.empty((p.T, p.H), dtype=torch.bfloat16, device="cuda")
    dwr = torch.empty((p.E, p.H), dtype=torch.float32, device="cuda")
    args = (prob, ws.schedule, to_dev_bf16(x), torch.from_numpy(wr_eh).cuda(), torch.from_numpy(ids).cuda(),
            torch.from_numpy(w).cuda(), torch.from_numpy(g).cuda(), d_sel, dx, dwr)
    mok.router_backward(*args, config=ws.config)
    torch.cuda.synchronize()
    ref_sel, _, ref_dwr, ref_dx = oracle.router_backward(bf16_to_f32(x).astype(np.float64),
                                                         wr_eh.astype(np.float64), ids, w.astype(np.float64),
                                                         g.astype(np.float64))
    assert np.allclose(d_sel.cpu().numpy(), ref_sel, rtol=1e-5, atol=1e-6)
    assert rel_fro(dwr.cpu().numpy(), ref_dwr) < 1e-5
    assert_close_bf16(from_dev_bf16(dx), ref_dx, "router dx")
    # bitwise reproducible
    d_sel2, dx2, dwr2 = torch.empty_like(d_sel), torch.empty_like(dx), torch.empty_like(dwr)
    mok.router_backward(*args[:7], d_sel2, dx2, dwr2, config=ws.config)
    torch.cuda.synchronize()
    assert torch.equal(d_sel, d_sel2) and torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dwr.view(torch.int32), dwr2.view(torch.int32))


def test_router_backward_full_size():
    """The fwd+bwd workload's router (T=16384 H=7168 E=32 top-4, Zipf(0.8)
    selection bias): d_sel, dWr (the dense contraction over all 16384 tokens)
    and every dx row against the oracle, bitwise the same on a second call."""
    import torch
    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    p = CONFIGS[4]
    print(f"[router] backward {p.name}", flush=True)
    x, wr_eh, bias = _inputs(p, True)
    ids, w = _run(p, x, wr_eh, bias)
    g = np.random.default_rng(p.seed + 100).standard_normal((p.T, p.k)).astype(np.float32)
    ws = F.get_workspace(p.T, p.H, 128, p.E, p.k, training=False)
    F.run_schedule(ws, torch.from_numpy(ids).cuda())
    prob = mok.make_problem(p.T, p.H, 128, p.E, p.k)
    d_sel = torch.empty((p.T, p.k), dtype=torch.float32, device="cuda")
    dx = torch.empty((p.T, p.H), dtype=torch.bfloat16, device="cuda")
    dwr = torch.empty((p.E, p.H), dtype=torch.float32, device="cuda")
    args = (prob, ws.schedule, to_dev_bf16(x), torch.from_numpy(wr_eh).cuda(), torch.from_numpy(ids).cuda(),
            torch.from_numpy(w).cuda(), torch.from_numpy(g).cuda())
    mok.router_backward(*args, d_sel, dx, dwr, config=ws.config)
    torch.cuda.synchronize()
    ref_sel, _, ref_dwr, ref_dx = oracle.router_backward(bf16_to_f32(x).astype(np.float64),
                                                         wr_eh.astype(np.float64), ids, w.astype(np.float64),
                                                         g.astype(np.float64))
    assert np.allclose(d_sel.cpu().numpy(), ref_sel, rtol=1e-5, atol=1e-6)
    assert rel_fro(dwr.cpu().numpy(), ref_dwr) < 1e-5
    assert_close_bf16(from_dev_bf16(dx), ref_dx, "router dx")
    d_sel2, dx2, dwr2 = torch.empty_like(d_sel), torch.empty_like(dx), torch.empty_like(dwr)
    mok.router_backward(*args, d_sel2, dx2, dwr2, config=ws.config)
    torch.cuda.synchronize()
    assert torch.equal(d_sel, d_sel2) and torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dwr.view(torch.int32), dwr2.view(torch.int32))


def test_router_empty_input():
    """T = 0: the forward writes nothing; the backward writes dWr = 0 exactly
    (over a buffer that held other values), the token arrays being empty."""
    import torch
    import mixture_experts_layer_30_amd as mok
    from mixture_experts_layer_30_amd import functional as F
    T, H, E, k = 0, 256, 16, 4
    print("[router] T=0", flush=True)
    prob = mok.make_problem(T, H, 128, E, k)
    x = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    wr = torch.randn((E, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((0, k), dtype=torch.int32, device="cuda")
    w = torch.empty((0, k), dtype=torch.float32, device="cuda")
    mok.router_forward(prob, x, wr, None, ids, w)
    ws = F.get_workspace(T, H, 128, E, k, training=False)
    F.run_schedule(ws, ids)
    dwr = torch.full((E, H), 3.0, dtype=torch.float32, device="cuda")
    mok.router_backward(prob, ws.schedule, x, wr, ids, w, torch.empty_like(w), torch.empty_like(w),
                        torch.empty_like(x), dwr, config=ws.config)
    torch.cuda.synchronize()
    assert not dwr.view(torch.int32).any()
