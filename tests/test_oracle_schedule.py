"""Pins for the oracle's routing schedule (CPU only).

The schedule is the stable counting sort of the flat top-k expert ids
([MoK card] "Using the functional API": build_schedule from the top-k expert
choices; [MoK clip] How-to item 2: one schedule for all exchange passes).
"""
import itertools

import numpy as np
import pytest

import oracle
from synthetic import CONFIGS, make_routing, make_x, problem


def brute_force_schedule(f, E):
    """Position of each row by definition: rows of lower experts first, then
    earlier rows of the same expert. O(R^2) pure-Python loops."""
    R = len(f)
    counts = [0] * E
    for v in f:
        counts[v] += 1
    dest = []
    for i in range(R):
        before = sum(1 for i2 in range(R) if f[i2] < f[i])
        same_earlier = sum(1 for i2 in range(i) if f[i2] == f[i])
        dest.append(before + same_earlier)
    perm = [None] * R
    for i, p in enumerate(dest):
        perm[p] = i
    return counts, perm, dest


def test_hand_worked_example():
    # Worked by hand from the definition: T=4, k=2, E=3.
    ids = np.array([[2, 0], [1, 2], [0, 1], [2, 1]])
    s = oracle.schedule(ids, 3)
    assert s["counts"].tolist() == [2, 3, 3]
    assert s["offsets"].tolist() == [0, 2, 5, 8]
    assert s["perm"].tolist() == [1, 4, 2, 5, 7, 0, 3, 6]
    assert s["dest"].tolist() == [5, 0, 2, 6, 1, 3, 7, 4]
    assert s["status"] == 0
    # minibatches of M=2 rows in a ring of 2 slots
    assert oracle.minibatch_count(8, 2) == 4
    assert oracle.ring_row(np.arange(8), 2, 2).tolist() == [0, 1, 2, 3, 0, 1, 2, 3]


def test_brute_force_all_top2_choices_T4_E3():
    pairs = [(a, b) for a in range(3) for b in range(3) if a != b]   # 6 ordered picks
    n = 0
    for choice in itertools.product(pairs, repeat=4):                 # 6^4 = 1296
        ids = np.array(choice)
        f = ids.reshape(-1).tolist()
        counts, perm, dest = brute_force_schedule(f, 3)
        s = oracle.schedule(ids, 3)
        assert s["counts"].tolist() == counts
        assert s["perm"].tolist() == perm
        assert s["dest"].tolist() == dest
        n += 1
    assert n == 1296


def check_invariants(ids, E):
    s = oracle.schedule(ids, E)
    f = np.asarray(ids).reshape(-1)
    R = f.size
    assert s["counts"].sum() == R
    assert sorted(s["perm"].tolist()) == list(range(R))
    assert np.array_equal(s["perm"][s["dest"]], np.arange(R))
    fp = f[s["perm"]]
    assert np.all(np.diff(fp) >= 0)
    for e in range(E):
        seg = s["perm"][s["offsets"][e]:s["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(f[seg] == e)
    return s


@pytest.mark.parametrize("T,E,k,seed", [(1, 4, 1, 0), (7, 5, 3, 1), (300, 16, 4, 2), (1000, 128, 8, 3)])
def test_invariants_random(T, E, k, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    check_invariants(ids, E)


def test_invariants_generator_routing():
    p = CONFIGS[0]
    x = make_x(p)
    ids, w = make_routing(p, x)
    s = check_invariants(ids, p.E)
    assert s["status"] == 0
    # every token picks k distinct experts
    assert all(len(set(r)) == p.k for r in ids.tolist())


def test_repeated_expert_in_one_token():
    # a token may pick the same expert twice: two rows ordered by j
    ids = np.array([[1, 1], [0, 1]])
    s = oracle.schedule(ids, 2)
    assert s["counts"].tolist() == [1, 3]
    assert s["perm"].tolist() == [2, 0, 1, 3]


def test_invalid_ids_set_status_and_sort_last():
    ids = np.array([[0, 5], [-1, 1], [1, 0]])
    s = oracle.schedule(ids, 3)
    assert s["status"] == oracle.STATUS_BAD_EXPERT_ID
    assert s["counts"].tolist() == [2, 2, 0]
    assert s["offsets"].tolist() == [0, 2, 4, 4]
    assert s["perm"].tolist() == [0, 5, 3, 4, 1, 2]
    assert np.array_equal(s["perm"][s["dest"]], np.arange(6))


def test_minibatches_partition_rows():
    R, M, Ns = 1001, 64, 3
    p = np.arange(R)
    nmb = oracle.minibatch_count(R, M)
    assert nmb == 16
    rows = oracle.ring_row(p, M, Ns)
    assert rows.max() < Ns * M
    # inside one minibatch the ring rows are distinct and contiguous
    for m in range(nmb):
        seg = rows[m * M:(m + 1) * M]
        assert np.array_equal(seg, (m % Ns) * M + np.arange(len(seg)))


def test_empty_and_single_expert():
    s = oracle.schedule(np.zeros((5, 1), np.int64), 4)
    assert s["counts"].tolist() == [5, 0, 0, 0]
    assert s["perm"].tolist() == [0, 1, 2, 3, 4]
    s = oracle.schedule(np.zeros((0, 2), np.int64), 4)
    assert s["counts"].tolist() == [0, 0, 0, 0] and s["perm"].size == 0
