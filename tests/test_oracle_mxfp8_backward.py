"""Pins for the oracle's MXFP8 backward (CPU only).

Reading pinned (every backward GEMM operand blocked by 32 along that GEMM's
contraction axis: H for dh, I for dX rows, the expert's rows from its first
permuted row for the weight gradients):
  * block-relative scaling: scaling dy by a power of two scales every
    gradient by exactly that power;
  * block structure: permuting H (or I) inside each aligned 32-block, the
    same way in every tensor, only permutes the outputs, while a swap across
    two blocks changes them; permuting an expert's tokens inside one of its
    32-row blocks (counted from the expert's first row) leaves its weight
    gradients unchanged, a swap across two of its blocks changes them;
  * it stays within the MXFP8 error of the exact fp64 backward (a dropped
    term or a wrong sign would be off by order one).
"""
import numpy as np

import oracle
from test_oracle_forward import rand_case

KEYS = ("dx", "dWg", "dWu", "dWd", "dw")


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def mxb(x, ids, w, ex, dy):
    return oracle.backward_mxfp8(x, ids, w, ex, dy)


def test_power_of_two_scaling_is_exact():
    x, ids, w, ex = rand_case(24, 64, 64, 3, 2, seed=11)
    dy = np.random.default_rng(12).standard_normal((24, 64))
    g1 = mxb(x, ids, w, ex, dy)
    g8 = mxb(x, ids, w, ex, 8.0 * dy)
    for key in KEYS:
        assert np.array_equal(g8[key], 8.0 * g1[key]), key


def _within_block_perm(n, rng):
    p = np.arange(n)
    for b in range(0, n, 32):
        p[b:b + 32] = b + rng.permutation(32)
    return p


def _apply_h(x, ex, dy, p):
    return x[:, p], [(Wg[:, p], Wu[:, p], Wd[p, :]) for Wg, Wu, Wd in ex], dy[:, p]


def test_h_blocks():
    x, ids, w, ex = rand_case(20, 64, 64, 3, 2, seed=21)
    dy = np.random.default_rng(22).standard_normal((20, 64))
    g = mxb(x, ids, w, ex, dy)
    p = _within_block_perm(64, np.random.default_rng(23))
    x2, ex2, dy2 = _apply_h(x, ex, dy, p)
    g2 = mxb(x2, ids, w, ex2, dy2)
    assert rel(g2["dx"], g["dx"][:, p]) < 1e-12
    assert rel(g2["dWg"], g["dWg"][:, :, p]) < 1e-12
    assert rel(g2["dWu"], g["dWu"][:, :, p]) < 1e-12
    assert rel(g2["dWd"], g["dWd"][:, p, :]) < 1e-12
    assert rel(g2["dw"], g["dw"]) < 1e-12
    q = np.arange(64)
    q[3], q[40] = 40, 3                      # across the two blocks of H
    x3, ex3, dy3 = _apply_h(x, ex, dy, q)
    g3 = mxb(x3, ids, w, ex3, dy3)
    assert rel(g3["dx"], g["dx"][:, q]) > 1e-6


def _apply_i(ex, p):
    return [(Wg[p, :], Wu[p, :], Wd[:, p]) for Wg, Wu, Wd in ex]


def test_i_blocks():
    x, ids, w, ex = rand_case(20, 64, 64, 3, 2, seed=31)
    dy = np.random.default_rng(32).standard_normal((20, 64))
    g = mxb(x, ids, w, ex, dy)
    p = _within_block_perm(64, np.random.default_rng(33))
    g2 = mxb(x, ids, w, _apply_i(ex, p), dy)
    assert rel(g2["dx"], g["dx"]) < 1e-12
    assert rel(g2["dWg"], g["dWg"][:, p, :]) < 1e-12
    assert rel(g2["dWu"], g["dWu"][:, p, :]) < 1e-12
    assert rel(g2["dWd"], g["dWd"][:, :, p]) < 1e-12
    assert rel(g2["dw"], g["dw"]) < 1e-12
    q = np.arange(64)
    q[5], q[50] = 50, 5
    g3 = mxb(x, ids, w, _apply_i(ex, q), dy)
    # I blocks enter where I is contracted (dX rows) and through h in the
    # forward (d topk_w); the weight gradients only see I as an output axis
    assert rel(g3["dx"], g["dx"]) > 1e-6
    assert rel(g3["dw"], g["dw"]) > 1e-6


def test_token_blocks_counted_from_the_expert_start():
    # k = 1; tokens 0..39 pick expert 0, tokens 40..79 expert 1, so expert 1's
    # rows are permuted rows 40..79: its blocks are rows 40..71 and 72..79
    # (from its own start), not 32..63 / 64..95.
    T, H, I = 80, 64, 64
    x, _, _, ex = rand_case(T, H, I, 2, 1, seed=41)
    ids = np.array([[0]] * 40 + [[1]] * 40)
    w = np.random.default_rng(42).random((T, 1))
    dy = np.random.default_rng(43).standard_normal((T, H))
    g = mxb(x, ids, w, ex, dy)

    def swapped(a, b):
        p = np.arange(T)
        p[a], p[b] = b, a
        return mxb(x[p], ids[p], w[p], ex, dy[p]), p

    g2, p = swapped(41, 70)                  # same block of expert 1 (rows 1 and 30)
    for key in ("dWg", "dWu", "dWd"):
        assert rel(g2[key], g[key]) < 1e-12, key
    assert rel(g2["dx"], g["dx"][p]) < 1e-12
    g3, _ = swapped(41, 75)                  # rows 1 and 35: different blocks
    assert rel(g3["dWg"][1], g["dWg"][1]) > 1e-6


def test_close_to_exact_backward():
    x, ids, w, ex = rand_case(48, 128, 96, 4, 2, seed=51)
    dy = np.random.default_rng(52).standard_normal((48, 128))
    g = mxb(x, ids, w, ex, dy)
    ref = oracle.backward(x, ids, w, ex, dy)
    for key in KEYS:
        err = rel(g[key], ref[key])
        # each operand carries ~2-3% relative RMS error from E4M3, a few
        # quantized operands sit on each path: well under 0.25; a sign or term
        # error would be of order one
        assert err < 0.25, (key, err)
        assert err > 1e-4, (key, err)         # it does quantize


def test_empty_expert_exact_zero():
    x, ids, w, ex = rand_case(16, 64, 64, 4, 1, seed=61)
    ids = np.where(ids == 3, 2, ids)
    dy = np.random.default_rng(62).standard_normal((16, 64))
    g = mxb(x, ids, w, ex, dy)
    for key in ("dWg", "dWu", "dWd"):
        assert not g[key][3].any()


def test_sampled_helpers_match_full():
    x, ids, w, ex = rand_case(40, 64, 64, 5, 2, seed=71)
    dy = np.random.default_rng(72).standard_normal((40, 64))
    g = mxb(x, ids, w, ex, dy)
    for e in range(5):
        dWg, dWu, dWd = oracle.backward_mxfp8_expert_weights(e, x, ids, w, ex, dy)
        assert rel(dWg, g["dWg"][e]) < 1e-12 and rel(dWu, g["dWu"][e]) < 1e-12
        assert rel(dWd, g["dWd"][e]) < 1e-12
    toks = np.array([0, 7, 19, 33])
    dx, dw = oracle.backward_mxfp8_tokens(x[toks], ids[toks], w[toks], ex, dy[toks])
    assert rel(dx, g["dx"][toks]) < 1e-12
    assert rel(dw, g["dw"][toks]) < 1e-12


def test_channel_slice_matches_full():
    """The GPU tests take the weight gradients of a hot expert on a range of
    intermediate channels (moe_testlib.ExpertsSliceI): that range of the
    full computation, up to fp64 rounding, for aligned and unaligned ranges
    (no block of the weight-gradient path runs along I)."""
    from moe_testlib import ExpertsSliceI
    x, ids, w, ex = rand_case(40, 64, 128, 3, 2, seed=73)
    dy = np.random.default_rng(74).standard_normal((40, 64))
    for e in range(3):
        dWg, dWu, dWd = oracle.backward_mxfp8_expert_weights(e, x, ids, w, ex, dy)
        for i0, i1 in ((32, 96), (16, 80), (0, 128)):
            sg, su, sd = oracle.backward_mxfp8_expert_weights(e, x, ids, w, ExpertsSliceI(ex, i0, i1), dy)
            assert rel(sg, dWg[i0:i1]) < 1e-12 and rel(su, dWu[i0:i1]) < 1e-12
            assert rel(sd, dWd[:, i0:i1]) < 1e-12
