"""Pins for the oracle's forward pass (CPU only).

Forward = dispatch rows to experts, SwiGLU FFN per expert, weighted combine
([MoK clip] Conclusion and key chart). Pinned against: scalar loops on a tiny
case, the dense-FFN closed form when all experts are equal, torch's own dense
SwiGLU for E = k = 1, and symmetries of the definition.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def rand_case(T, H, I, E, k, seed, distinct=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    if distinct:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    else:
        ids = rng.integers(0, E, size=(T, k))
    w = rng.random((T, k))
    experts = [(rng.standard_normal((I, H)) / math.sqrt(H),
                rng.standard_normal((I, H)) / math.sqrt(H),
                rng.standard_normal((H, I)) / math.sqrt(I)) for _ in range(E)]
    return x, ids, w, experts


def scalar_forward(x, ids, w, experts):
    """Pure-Python loops, one token and one pick at a time."""
    T, H = x.shape
    k = ids.shape[1]
    y = [[0.0] * H for _ in range(T)]
    for t in range(T):
        for j in range(k):
            Wg, Wu, Wd = experts[int(ids[t][j])]
            I = Wg.shape[0]
            h = []
            for i in range(I):
                a = sum(float(x[t][c]) * float(Wg[i][c]) for c in range(H))
                b = sum(float(x[t][c]) * float(Wu[i][c]) for c in range(H))
                h.append(a / (1.0 + math.exp(-a)) * b)
            for c in range(H):
                o = sum(h[i] * float(Wd[c][i]) for i in range(I))
                y[t][c] += float(w[t][j]) * o
    return np.array(y)


def test_scalar_loops_tiny():
    x, ids, w, ex = rand_case(T=4, H=8, I=16, E=3, k=2, seed=0)
    y, _ = oracle.forward(x, ids, w, ex)
    np.testing.assert_allclose(y, scalar_forward(x, ids, w, ex), rtol=0, atol=1e-12)


def test_identical_experts_closed_form():
    # all experts equal => y[t] = (sum_j w[t, j]) * FFN(x[t]); with softmax weights = dense FFN
    x, ids, w, ex = rand_case(T=20, H=16, I=24, E=5, k=3, seed=1)
    ex = [ex[0]] * 5
    y, _ = oracle.forward(x, ids, w, ex)
    Wg, Wu, Wd = ex[0]
    a, b = x @ Wg.T, x @ Wu.T
    dense = (a / (1 + np.exp(-a)) * b) @ Wd.T
    np.testing.assert_allclose(y, w.sum(1, keepdims=True) * dense, rtol=1e-12, atol=1e-12)
    ws = np.exp(w) / np.exp(w).sum(1, keepdims=True)
    y2, _ = oracle.forward(x, ids, ws, ex)
    np.testing.assert_allclose(y2, dense, rtol=1e-12, atol=1e-12)


def test_single_expert_matches_torch_dense_swiglu():
    x, ids, w, ex = rand_case(T=9, H=32, I=48, E=1, k=1, seed=2)
    w = np.ones_like(w)
    y, _ = oracle.forward(x, ids, w, ex)
    Wg, Wu, Wd = (torch.from_numpy(m) for m in ex[0])
    xt = torch.from_numpy(x)
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(xt, Wg)) * torch.nn.functional.linear(xt, Wu), Wd)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_token_permutation_equivariance():
    x, ids, w, ex = rand_case(T=30, H=16, I=8, E=6, k=2, seed=3)
    y, _ = oracle.forward(x, ids, w, ex)
    pi = np.random.default_rng(0).permutation(30)
    y2, _ = oracle.forward(x[pi], ids[pi], w[pi], ex)
    np.testing.assert_allclose(y2, y[pi], rtol=1e-12, atol=1e-13)


def test_linear_in_combine_weights():
    x, ids, w, ex = rand_case(T=10, H=8, I=8, E=4, k=2, seed=4)
    w2 = np.random.default_rng(1).random(w.shape)
    y1, _ = oracle.forward(x, ids, w, ex)
    y2, _ = oracle.forward(x, ids, w2, ex)
    y3, _ = oracle.forward(x, ids, 2.0 * w - 3.0 * w2, ex)
    np.testing.assert_allclose(y3, 2.0 * y1 - 3.0 * y2, rtol=1e-10, atol=1e-12)


def test_expert_relabelling_invariance():
    x, ids, w, ex = rand_case(T=12, H=8, I=8, E=5, k=2, seed=5)
    y, _ = oracle.forward(x, ids, w, ex)
    sigma = np.array([3, 0, 4, 1, 2])          # expert e is renamed sigma[e]
    ex2 = [None] * 5
    for e in range(5):
        ex2[sigma[e]] = ex[e]
    y2, _ = oracle.forward(x, sigma[ids], w, ex2)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-13)


def test_forward_tokens_matches_forward():
    x, ids, w, ex = rand_case(T=25, H=8, I=16, E=4, k=3, seed=6, distinct=False)
    y, ctx = oracle.forward(x, ids, w, ex)
    sub = np.array([0, 3, 7, 24])
    ys, outs = oracle.forward_tokens(x[sub], ids[sub], w[sub], ex)
    np.testing.assert_allclose(ys, y[sub], rtol=1e-12, atol=1e-13)
    ob = ctx["obuf"].reshape(25, 3, 8)
    np.testing.assert_allclose(outs, ob[sub], rtol=1e-12, atol=1e-13)


def test_saved_activations_are_permuted_rows():
    x, ids, w, ex = rand_case(T=6, H=8, I=4, E=3, k=2, seed=7)
    _, ctx = oracle.forward(x, ids, w, ex)
    s = ctx["sched"]
    for p in range(12):
        i = s["perm"][p]
        e = ids.reshape(-1)[i]
        np.testing.assert_allclose(ctx["a"][p], ex[e][0] @ x[i // 2], rtol=1e-12)
        np.testing.assert_allclose(ctx["b"][p], ex[e][1] @ x[i // 2], rtol=1e-12)


def test_invalid_expert_rows_contribute_zero():
    x, ids, w, ex = rand_case(T=4, H=8, I=8, E=3, k=2, seed=8)
    bad = ids.copy()
    bad[1, 0] = 7
    y, ctx = oracle.forward(x, bad, w, ex)
    assert ctx["sched"]["status"] == oracle.STATUS_BAD_EXPERT_ID
    w2 = w.copy()
    w2[1, 0] = 0.0
    y2, _ = oracle.forward(x, ids, w2, ex)
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1])
def test_generator_routing_weights_are_softmax(seed):
    from synthetic import make_routing, make_x, problem
    p = problem(64, 32, 16, 8, 2, seed=seed)
    ids, w = make_routing(p, make_x(p))
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-6)
    assert np.all(w[:, 0] >= w[:, 1])    # picks come in descending score order
