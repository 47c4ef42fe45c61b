"""Pins for the oracle's backward pass (CPU only).

Pinned against central finite differences of the oracle's own forward, against
torch.autograd on an independent per-token formulation, and against the dense
closed form when all experts are equal.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from test_oracle_forward import rand_case


def loss(x, ids, w, ex, dy):
    y, _ = oracle.forward(x, ids, w, ex)
    return float(np.sum(y * dy))


def fd(fun, arr, idx, h=1e-6):
    old = arr[idx]
    arr[idx] = old + h
    lp = fun()
    arr[idx] = old - h
    lm = fun()
    arr[idx] = old
    return (lp - lm) / (2 * h)


def test_finite_differences_all_inputs():
    x, ids, w, ex = rand_case(T=5, H=6, I=4, E=3, k=2, seed=11)
    ex = [tuple(m.copy() for m in t) for t in ex]
    dy = np.random.default_rng(3).standard_normal((5, 6))
    g = oracle.backward(x, ids, w, ex, dy)
    f = lambda: loss(x, ids, w, ex, dy)  # noqa: E731
    rng = np.random.default_rng(4)
    checks = []
    for _ in range(6):
        idx = (rng.integers(5), rng.integers(6))
        checks.append((fd(f, x, idx), g["dx"][idx]))
        idx = (rng.integers(5), rng.integers(2))
        checks.append((fd(f, w, idx), g["dw"][idx]))
        e = int(rng.integers(3))
        i, c = rng.integers(4), rng.integers(6)
        checks.append((fd(f, ex[e][0], (i, c)), g["dWg"][e, i, c]))
        checks.append((fd(f, ex[e][1], (i, c)), g["dWu"][e, i, c]))
        checks.append((fd(f, ex[e][2], (c, i)), g["dWd"][e, c, i]))
    for num, ana in checks:
        assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (num, ana)


def torch_per_token_loss(x, ids, w, ex, dy):
    """Independent formulation: a loop over tokens and picks in torch fp64."""
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    params = [tuple(torch.tensor(m, requires_grad=True) for m in t) for t in ex]
    T, k = ids.shape
    total = 0.0
    for t in range(T):
        yt = 0.0
        for j in range(k):
            Wg, Wu, Wd = params[int(ids[t, j])]
            h = torch.nn.functional.silu(Wg @ xt[t]) * (Wu @ xt[t])
            yt = yt + wt[t, j] * (Wd @ h)
        total = total + torch.dot(yt, torch.tensor(dy[t]))
    total.backward()
    return xt.grad.numpy(), wt.grad.numpy(), [[m.grad for m in t] for t in params]


def test_matches_torch_autograd_per_token():
    x, ids, w, ex = rand_case(T=7, H=8, I=12, E=4, k=2, seed=12)
    dy = np.random.default_rng(5).standard_normal((7, 8))
    g = oracle.backward(x, ids, w, ex, dy)
    dx, dw, dW = torch_per_token_loss(x, ids, w, ex, dy)
    np.testing.assert_allclose(g["dx"], dx, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dw"], dw, rtol=1e-11, atol=1e-12)
    for e in range(4):
        for name, m in zip(("dWg", "dWu", "dWd"), dW[e]):
            ref = np.zeros(g[name][e].shape) if m is None else m.numpy()
            np.testing.assert_allclose(g[name][e], ref, rtol=1e-11, atol=1e-12)


def test_identical_experts_sum_to_dense_gradient():
    x, ids, w, ex = rand_case(T=16, H=8, I=6, E=4, k=2, seed=13)
    ex = [ex[0]] * 4
    dy = np.random.default_rng(6).standard_normal((16, 8))
    g = oracle.backward(x, ids, w, ex, dy)
    # dense reference: y = s * FFN(x) with s = sum_j w[t, j]
    Wg, Wu, Wd = (torch.tensor(m, requires_grad=True) for m in ex[0])
    xt = torch.tensor(x)
    s = torch.tensor(w.sum(1, keepdims=True))
    ffn = torch.nn.functional.linear(
        torch.nn.functional.silu(xt @ Wg.T) * (xt @ Wu.T), Wd)
    (torch.sum(s * ffn * torch.tensor(dy))).backward()
    np.testing.assert_allclose(g["dWg"].sum(0), Wg.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dWu"].sum(0), Wu.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dWd"].sum(0), Wd.grad.numpy(), rtol=1e-11, atol=1e-12)
    # dw[t, j] = <dY[t], FFN(x[t])> for every j
    ref = np.sum(dy * ffn.detach().numpy(), axis=1)
    for j in range(2):
        np.testing.assert_allclose(g["dw"][:, j], ref, rtol=1e-11, atol=1e-12)


def test_empty_experts_get_exact_zero():
    x, ids, w, ex = rand_case(T=6, H=8, I=4, E=5, k=2, seed=14)
    ids = np.where(ids >= 3, ids % 3, ids)       # experts 3 and 4 unused
    ids[:, 1] = (ids[:, 0] + 1) % 3
    dy = np.random.default_rng(7).standard_normal((6, 8))
    g = oracle.backward(x, ids, w, ex, dy)
    for e in (3, 4):
        for name in ("dWg", "dWu", "dWd"):
            assert np.all(g[name][e] == 0.0)


def test_sampled_helpers_match_full_backward():
    x, ids, w, ex = rand_case(T=20, H=8, I=8, E=4, k=3, seed=15, distinct=False)
    dy = np.random.default_rng(8).standard_normal((20, 8))
    g = oracle.backward(x, ids, w, ex, dy)
    sub = np.array([1, 4, 19])
    dx, dw = oracle.backward_tokens(x[sub], ids[sub], w[sub], ex, dy[sub])
    np.testing.assert_allclose(dx, g["dx"][sub], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dw, g["dw"][sub], rtol=1e-11, atol=1e-12)
    for e in range(4):
        dg, du, dd = oracle.backward_expert_weights(e, x, ids, w, ex, dy)
        np.testing.assert_allclose(dg, g["dWg"][e], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(du, g["dWu"][e], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dd, g["dWd"][e], rtol=1e-11, atol=1e-12)


def test_swiglu_derivative_closed_form():
    a = np.linspace(-6, 6, 101)
    b = np.cos(a)
    h = 1e-6
    dA, dB = oracle.moe_oracle._swiglu_backward(np.ones_like(a), a, b)
    num_a = (oracle.swiglu(a + h, b) - oracle.swiglu(a - h, b)) / (2 * h)
    num_b = (oracle.swiglu(a, b + h) - oracle.swiglu(a, b - h)) / (2 * h)
    np.testing.assert_allclose(dA, num_a, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(dB, num_b, rtol=1e-7, atol=1e-9)
    sig = 1.0 / (1.0 + math.exp(-2.0))
    assert abs(oracle.silu(np.array(2.0)) - 2.0 * sig) < 1e-15
