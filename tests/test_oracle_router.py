"""Pins of the oracle's router front end (logits, top-k with ties to the lower
expert id, softmax over the selected unbiased logits, and the backward from
d topk_w), each against something other than the oracle's own formula."""
import numpy as np
import pytest

import oracle
from synthetic import CONFIGS, bf16_to_f32, make_routing, make_x, router_weights


def _rand(T, H, E, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, H)), rng.standard_normal((E, H)) / np.sqrt(H)


def test_selection_dominates_the_rest_and_is_ordered():
    """Checked by pairwise dominance, not by sorting: every selected expert
    beats every unselected one (higher score, or equal score and lower id),
    and the k picks come in descending score, equal scores by ascending id."""
    x, wr = _rand(7, 16, 9, 1)
    bias = np.random.default_rng(2).standard_normal(9)
    for k in (1, 3, 9):
        logits, ids, _ = oracle.router_forward(x, wr, bias, k)
        score = logits + bias
        for t in range(7):
            sel = list(ids[t])
            assert len(set(sel)) == k
            for a in sel:
                for b in set(range(9)) - set(sel):
                    assert score[t, a] > score[t, b] or (score[t, a] == score[t, b] and a < b)
            for a, b in zip(sel, sel[1:]):
                assert score[t, a] > score[t, b] or (score[t, a] == score[t, b] and a < b)


def test_exact_ties_go_to_the_lower_expert_id():
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    wr = np.array([[1.0, 0.0], [2.0, 0.0], [2.0, 0.0], [0.0, 3.0], [0.0, 3.0]])
    _, ids, w = oracle.router_forward(x, wr, None, 2)
    assert ids.tolist() == [[1, 2], [3, 4]]
    assert np.allclose(w, 0.5)                   # equal logits -> equal weights


def test_bias_moves_the_selection_but_not_the_weights():
    x, wr = _rand(5, 8, 6, 3)
    bias = np.zeros(6)
    bias[4] = 1e6                                # expert 4 is always picked first
    logits, ids, w = oracle.router_forward(x, wr, bias, 2)
    assert (ids[:, 0] == 4).all()
    # weights of the two picks: the closed form of a 2-way softmax of the
    # *unbiased* logits
    l0 = logits[np.arange(5), ids[:, 0]]
    l1 = logits[np.arange(5), ids[:, 1]]
    assert np.allclose(w[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-14, atol=0)


def test_weights_are_a_softmax_of_the_selected_logits():
    x, wr = _rand(6, 12, 10, 4)
    logits, ids, w = oracle.router_forward(x, wr, None, 4)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15) and (w > 0).all()
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    # ratio of two weights = exp of the logit difference
    assert np.allclose(w[:, 1] / w[:, 0], np.exp(sel[:, 1] - sel[:, 0]), rtol=1e-13)


def test_backward_matches_central_differences():
    """L = sum(g * topk_w) with the selection held fixed (margins far above the
    step), differentiated numerically in x and Wr."""
    T, H, E, k = 4, 6, 5, 2
    x, wr = _rand(T, H, E, 5)
    g = np.random.default_rng(6).standard_normal((T, k))
    _, ids, w = oracle.router_forward(x, wr, None, k)
    d_sel, d_logits, d_wr, dx = oracle.router_backward(x, wr, ids, w, g)

    def loss(xx, ww):
        lg = xx @ ww.T
        sel = np.take_along_axis(lg, ids.astype(np.int64), axis=1)
        ex = np.exp(sel - sel.max(axis=1, keepdims=True))
        return float((g * ex / ex.sum(axis=1, keepdims=True)).sum())

    h = 1e-6
    for (arr, grad) in ((x, dx), (wr, d_wr)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a0 = arr[idx]
            arr[idx] = a0 + h
            lp = loss(x, wr)
            arr[idx] = a0 - h
            lm = loss(x, wr)
            arr[idx] = a0
            num[idx] = (lp - lm) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-9)
    # the softmax Jacobian's rows sum to zero, and unselected logits get none
    assert np.allclose(d_sel.sum(axis=1), 0.0, atol=1e-15)
    mask = np.zeros((T, E), bool)
    mask[np.arange(T)[:, None], ids] = True
    assert (d_logits[~mask] == 0).all()


@pytest.mark.parametrize("cid", [0, 2])
def test_agrees_with_the_workload_router(cid):
    """The seeded workloads draw their routing with their own code: the
    oracle, given the same Wr and bias, picks the same experts and weights."""
    p = CONFIGS[cid]
    T = min(p.T, 512)
    x = make_x(p)
    ids_ref, w_ref = make_routing(p, x)
    wr, bias = router_weights(p)
    _, ids, w = oracle.router_forward(bf16_to_f32(x[:T]).astype(np.float64), wr.T.astype(np.float64), bias, p.k)
    assert np.array_equal(ids, ids_ref[:T])
    assert np.allclose(w, w_ref[:T], rtol=1e-6, atol=0)
