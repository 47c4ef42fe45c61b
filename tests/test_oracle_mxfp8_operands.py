"""Per-operand pins of the oracle's MXFP8 backward (CPU only).

Each quantization point of the MXFP8 backward is pinned on its own: a case is
built where every operand of every GEMM is exactly representable in MXFP8
along every axis it is quantized on -- except one element of one operand,
which exactly one quantizer changes, by a value derived here by hand from the
E4M3 rules. The expected gradients are then the plain closed forms of the
backward with that one element replaced, so leaving out that quantization
(or applying it along the wrong axis, or to the wrong operand) fails.

The regime: one expert, one pick per token (k = 1, w = 1), T = H = I = 32,
so every quantization axis (H, I, 2I = two blocks of I, and the expert's 32
rows) is one block of 32. The gate pre-activation a is 60 or more
everywhere, where sigmoid(a) is exactly 1.0 in float64 (exp(-60) < 2^-53),
so silu(a) = a and the SwiGLU and its backward become bilinear:
    h = a*b,  dA = dh*b,  dB = dh*a.
All values are dyadic with at most four significant bits, so every product
and sum in the closed forms is exact in float64.

E4M3 facts used (OCP OFP8, with the MX block scale X = 2^(floor(log2 amax) - 8)):
a block maximum whose significand is 1.875 scales to 480 > 448 and saturates
to 448, i.e. 1.875 * 2^e -> 1.75 * 2^e; the same value is exact when a larger
element (2 * 2^e) sets the scale (it scales to 240, a code). 1.0625 lies
halfway between the codes for 1.0 and 1.125 at exponent 0 and rounds to the
even one, 1.0.
"""
import numpy as np
import pytest

import oracle

T = H = I = 32
T0, T1, T2, T3 = 5, 9, 17, 23          # tokens with planted values (T2 has a = 128)
I0, I1, I3 = 7, 12, 20                 # columns with planted values
KEYS = ("y", "dx", "dWg", "dWu", "dWd", "dw")


def rows_q(V):
    """Quantize-dequantize each row of V in 32-blocks (along the last axis)."""
    return oracle.mxfp8_roundtrip(V)


def cols_q(V):
    return oracle.mxfp8_roundtrip(np.asarray(V).T).T


def base():
    """Inputs where every operand is exactly representable (see the module
    docstring). Returns dict X, Wg, Wu, Wd, dY, w."""
    rng = np.random.default_rng(7)
    X = np.zeros((T, H))
    X[:, 0] = 8.0                                   # a = 8 * Wg[:, 0] = 64 ...
    X[T2, 0] = 16.0                                 # ... and 128 on token T2
    X[:, 1] = rng.choice([-1.5, -1.0, -0.75, -0.5, 0.5, 0.75, 1.0, 1.5], T)   # passive column
    X[:, 3] = rng.choice([-1.0, -0.5, -0.25, 0.25, 0.5, 1.0], T)              # v: b = v * beta
    X[T2, 3] = 1.0
    Wg = np.zeros((I, H))
    Wg[:, 0] = 8.0
    Wu = np.zeros((I, H))
    Wu[:, 3] = rng.choice([-1.5, -1.0, -0.5, 0.5, 1.0, 1.5], I)              # beta
    Wu[I1, 3] = 2.0
    Wd = np.eye(H, I)
    dY = rng.choice([-1.5, -1.0, -0.75, -0.5, -0.25, 0.0, 0.25, 0.5, 0.75, 1.0, 1.5], (T, H))
    return dict(X=X, Wg=Wg, Wu=Wu, Wd=Wd, dY=dY, w=np.ones(T))


def closed_forms(c, sub=None):
    """The backward of one expert with k = 1 in the bilinear regime, with
    optional per-use substitutions sub[name](value) -> value of the operand
    that one GEMM reads. Returns (outputs, operands)."""
    sub = sub or {}
    S = lambda name, v: sub[name](v) if name in sub else v  # noqa: E731
    X, Wg, Wu, Wd, dY, w = c["X"], c["Wg"], c["Wu"], c["Wd"], c["dY"], c["w"]
    a, b = X @ Wg.T, X @ Wu.T
    assert (a >= 60).all(), "sigmoid(a) must be exactly 1"
    out = S("h_I", a * b) @ S("Wd_I", Wd).T         # the forward quantizes the unrounded h
    a, b = S("a_bf16", a), S("b_bf16", b)             # the bf16 a, b saved for the backward
    h = S("h_bf16", a * b)
    dO = S("dO_bf16", w[:, None] * dY)
    dh = S("dO_H", dO) @ S("Wd_H", Wd)
    dA, dB = S("dA_bf16", dh * b), S("dB_bf16", dh * a)
    Xt = S("X_t", X)
    res = {"y": w[:, None] * out, "dw": (dY * out).sum(1)[:, None],
           "dx": S("dA_2I", dA) @ S("Wg_2I", Wg) + S("dB_2I", dB) @ S("Wu_2I", Wu),
           "dWg": (S("dA_t", dA).T @ Xt)[None], "dWu": (S("dB_t", dB).T @ Xt)[None],
           "dWd": (S("dO_t", dO).T @ S("h_t", h))[None]}
    ops = {"X_H": (X, rows_q), "Wg_H": (Wg, rows_q), "Wu_H": (Wu, rows_q), "h_I": (X @ Wg.T * (X @ Wu.T), rows_q),
           "Wd_I": (Wd, rows_q), "dO_H": (dO, rows_q), "Wd_H": (Wd, cols_q), "dA_2I": (dA, rows_q),
           "dB_2I": (dB, rows_q), "Wg_2I": (Wg, cols_q), "Wu_2I": (Wu, cols_q), "dO_t": (dO, cols_q),
           "h_t": (h, cols_q), "dA_t": (dA, cols_q), "dB_t": (dB, cols_q), "X_t": (X, cols_q)}
    return res, ops


def put(idx, val):
    def f(V):
        V = np.array(V, np.float64)
        V[idx] = val
        return V
    return f


def run_oracle(c):
    ex = [(c["Wg"], c["Wu"], c["Wd"])]
    ids = np.zeros((T, 1), np.int64)
    return oracle.backward_mxfp8(c["X"], ids, c["w"][:, None], ex, c["dY"])


def check_case(c, targets, affected):
    """targets: {operand: (index, value it quantizes to)} for a quantized
    operand, {name_bf16: (index, value) or function} for a bf16 rounding the
    case states by hand; affected: outputs the quantizations must change."""
    sub = {name: (t if callable(t) else put(*t)) for name, t in targets.items()}
    exp, ops = closed_forms(c, sub)
    # preconditions: exactly the planted element changes under its quantizer
    for name, (V, q) in ops.items():
        changed = q(V) != V
        if name in targets and not callable(targets[name]):
            idx, val = targets[name]
            assert changed.sum() == 1 and changed[idx], (name, np.argwhere(changed))
            assert q(V)[idx] == val, (name, q(V)[idx], val)
        else:
            assert not changed.any(), (name, np.argwhere(changed))
    got = run_oracle(c)
    for key in KEYS:
        assert np.array_equal(got[key], exp[key]), (key, np.abs(got[key] - exp[key]).max())
    # leaving the quantization out gives something else
    plain, _ = closed_forms(c, {k: v for k, v in sub.items() if k.endswith("_bf16")})
    for key in KEYS:
        same = np.array_equal(plain[key], exp[key])
        assert same == (key not in affected), (key, same)


def test_bilinear_closed_forms_equal_the_exact_backward():
    """The closed forms above are the exact backward in this regime (the exact
    backward is pinned by finite differences and torch autograd), and with
    every operand representable the MXFP8 backward equals it exactly."""
    c = base()
    exp, ops = closed_forms(c)
    for name, (V, q) in ops.items():
        assert np.array_equal(q(V), V), name
    ex = [(c["Wg"], c["Wu"], c["Wd"])]
    ids = np.zeros((T, 1), np.int64)
    ref = oracle.backward(c["X"], ids, c["w"][:, None], ex, c["dY"])
    for key in KEYS:
        assert np.allclose(ref[key], exp[key], rtol=0, atol=1e-12), key
    got = run_oracle(c)
    for key in KEYS:
        assert np.array_equal(got[key], exp[key]), key


def test_dO_quantized_along_H_for_dh():
    c = base()
    c["dY"][T0] = np.clip(c["dY"][T0], -1.5, 1.5)
    c["dY"][T0, I0] = 1.875                          # the largest of its row ...
    c["dY"][T1, I0] = 2.0                            # ... but not of its column
    c["X"][T0, 3] = 1.0
    c["Wu"][I0, 3] = 1.0
    check_case(c, {"dO_H": ((T0, I0), 1.75)}, affected={"dx", "dWg", "dWu"})


def test_dO_quantized_along_tokens_for_dWd():
    c = base()
    c["dY"][:, I0] = np.clip(c["dY"][:, I0], -1.5, 1.5)
    c["dY"][T0] = 0.0
    c["dY"][T0, I0] = 1.875                          # the largest of its column ...
    c["dY"][T0, I1] = 2.0                            # ... but not of its row
    c["X"][T0, 3] = 0.5
    c["dY"][T2, I0] = 1.5                            # dA, dB of column I0 peak on T2
    c["Wu"][I0, 3] = 1.0
    check_case(c, {"dO_t": ((T0, I0), 1.75)}, affected={"dWd"})


def test_h_quantized_along_tokens_for_dWd():
    c = base()
    c["Wu"][:, 3] = np.where(np.abs(c["Wu"][:, 3]) == 1.5, np.sign(c["Wu"][:, 3]), c["Wu"][:, 3])
    c["X"][T0, 3] = 1.25                             # h[T0, I0] = 64 * 1.25 * 1.5 = 120 ...
    c["Wu"][I0, 3] = 1.5                             # ... the only 1.5 of beta
    c["X"][T2, 3] = 0.25                             # keeps T2's h below 120 in column I0
    c["dY"][T0] = 0.0
    c["dY"][T0, I1] = 1.0
    check_case(c, {"h_t": ((T0, I0), 112.0)}, affected={"dWd"})


def test_dA_quantized_along_tokens_for_dWg():
    c = base()
    c["Wu"][:, 3] = np.where(np.abs(c["Wu"][:, 3]) == 1.5, np.sign(c["Wu"][:, 3]), c["Wu"][:, 3])
    c["Wu"][I1, 3] = 2.0
    c["Wu"][I0, 3] = 1.0
    c["X"][T0, 3] = 1.25
    c["dY"][T0] = 0.0
    c["dY"][T0, I0] = 1.5                            # dA[T0, I0] = 1.5 * 1.25 = 1.875 ...
    c["dY"][T0, I1] = 1.0                            # ... dA[T0, I1] = 2.5 leads its row
    check_case(c, {"dA_t": ((T0, I0), 1.75)}, affected={"dWg"})


def _gate_60_on_column(c, i):
    """a[:, i] = 60 (120 on token T2): Wg[i, 0] = 7.5, with a larger entry on
    a passive column (x there is 0) so that 7.5 is not its row's maximum;
    beta_i = 0 makes b, h and dA of column i zero, and Wu[i] reads another
    passive column so that dB of column i still reaches dx."""
    c["Wg"][i, 0] = 7.5
    c["Wg"][i, 2] = 8.0
    c["Wu"][i, 3] = 0.0
    c["Wu"][i, 4] = 1.0


def test_dB_quantized_along_tokens_for_dWu():
    c = base()
    _gate_60_on_column(c, I0)
    c["dY"][:, I0] = 0.0
    c["dY"][T2, I0] = 0.25                           # dB[T2, I0] = 30 ...
    c["dY"][T2, I1] = 1.0                            # ... under T2's row maximum 128
    c["dY"][T0, I0] = 1.0                            # dB[T0, I0] = 60, its column's largest
    c["dY"][T0, I1] = 1.0                            # dB[T0, I1] = 64 leads the row
    check_case(c, {"dB_t": ((T0, I0), 56.0)}, affected={"dWu"})


def test_dA_quantized_along_2I_for_dx():
    c = base()
    c["Wu"][I0, 3] = 1.0
    c["X"][T0, 3] = 1.25
    c["dY"][T0] = 0.0
    c["dY"][T0, I0] = 1.5                            # dA[T0, I0] = 1.875 leads its row ...
    c["dY"][T0, I1] = 0.25
    c["dY"][T3, I0] = 2.0                            # ... but not its column
    c["X"][T3, 3] = 1.0
    check_case(c, {"dA_2I": ((T0, I0), 1.75)}, affected={"dx"})


def test_dB_quantized_along_2I_for_dx():
    c = base()
    _gate_60_on_column(c, I0)
    c["dY"][:, I0] = 0.0
    c["dY"][T0] = np.clip(c["dY"][T0], -0.75, 0.75)
    c["dY"][T0, I0] = 1.0                            # dB[T0, I0] = 60 leads its row ...
    c["X"][T3, 2] = 0.5                              # ... not its column: a[T3, I0] = 60 + 4 = 64
    c["dY"][T3, I0] = 1.0                            # and dB[T3, I0] = 64
    check_case(c, {"dB_2I": ((T0, I0), 56.0)}, affected={"dx"})


def test_x_quantized_along_tokens_for_dWg_dWu():
    c = base()
    c["X"][T0, 1] = 1.875                            # the passive column's largest
    check_case(c, {"X_t": ((T0, 1), 1.75)}, affected={"dWg", "dWu"})


def test_Wd_quantized_along_H_for_dh():
    c = base()
    c["Wd"][I0, I0] = 1.875                          # its column's only entry ...
    c["Wd"][I0, I3] = 2.0                            # ... its row's second, larger one
    c["Wd"][I3, I3] = 0.0
    c["dY"][:, I0] = np.where(np.abs(c["dY"][:, I0]) >= 0.75, np.sign(c["dY"][:, I0]), 0.5 * np.sign(c["dY"][:, I0]))
    c["Wu"][I0, 3] = 1.0
    check_case(c, {"Wd_H": ((I0, I0), 1.75)}, affected={"dx", "dWg", "dWu"})


def test_Wg_quantized_along_2I_for_dx():
    c = base()
    c["Wg"][I0, 2] = 1.875                           # passive column 2: only dX reads it
    check_case(c, {"Wg_2I": ((I0, 2), 1.75)}, affected={"dx"})


def test_dO_rounded_to_bf16_before_it_is_quantized():
    """dO = w * dy is stored in bf16 before either quantization: with
    w = 1 + 2^-10 and dy = 1.0625, w * dy = 1.06354 rounds to the bf16 value
    1.0625, an E4M3 midpoint that rounds to even (1.0); quantizing w * dy
    directly would give 1.125."""
    c = base()
    c["w"][T0] = 1.0 + 2.0 ** -10
    c["dY"][T0] = np.clip(c["dY"][T0], -1.0, 1.0)
    c["dY"][T0, I1] = 1.5                            # row maximum: exponent 0
    c["dY"][:, I0] = np.clip(c["dY"][:, I0], -1.0, 1.0)
    c["dY"][T3, I0] = 1.5                            # column maximum: exponent 0
    c["dY"][T0, I0] = 1.0625
    assert np.array_equal(oracle.bf16_round(c["w"][:, None] * c["dY"]), c["dY"])
    assert rows_q(np.array([[1.0625 * (1 + 2.0 ** -10), 1.5] + [0.0] * 30]))[0, 0] == 1.125
    check_case(c, {"dO_bf16": lambda V: c["dY"], "dO_H": ((T0, I0), 1.0), "dO_t": ((T0, I0), 1.0)},
               affected={"dx", "dWg", "dWu", "dWd"})
    # quantizing w * dy without the bf16 rounding gives something else
    alt, _ = closed_forms(c, {"dO_H": rows_q, "dO_t": cols_q})
    got = run_oracle(c)
    for key in ("dx", "dWg", "dWu", "dWd"):
        assert not np.allclose(got[key], alt[key], rtol=1e-6), key


def test_dA_dB_rounded_to_bf16_before_they_are_quantized():
    """dh[T0, I0] = 1 + 2^-4 + 2^-9 from three exact products (Wd[H1, I0] =
    2^-4 and Wd[H2, I0] = 2^-9 are exact in both Wd blocks they sit in); with
    b = 1 and a = 64, dA = 1.064453125 and dB = 68.125 round to the bf16
    values 1.0625 and 68, both E4M3 midpoints that go to the even code (1.0
    and 64); quantized unrounded they would give 1.125 and 72."""
    c = base()
    H1, H2 = 27, 29
    c["Wd"][H1, I0], c["Wd"][H2, I0] = 2.0 ** -4, 2.0 ** -9
    c["dY"][:, [H1, H2]] = 0.0
    c["X"][T0, 3] = 1.0
    c["Wu"][I0, 3] = 1.0
    c["dY"][T0] = np.clip(c["dY"][T0], -1.0, 1.0)
    c["dY"][T0, I1] = 0.5
    c["dY"][:, I0] = np.clip(c["dY"][:, I0], -1.0, 1.0)
    c["dY"][T2, I0] = 0.5
    c["dY"][T0, [I0, H1, H2]] = 1.0
    check_case(c, {"dA_bf16": ((T0, I0), 1.0625), "dB_bf16": ((T0, I0), 68.0),
                   "dA_t": ((T0, I0), 1.0), "dA_2I": ((T0, I0), 1.0),
                   "dB_t": ((T0, I0), 64.0), "dB_2I": ((T0, I0), 64.0)},
               affected={"dx", "dWg", "dWu"})
    alt, _ = closed_forms(c, {"dA_t": cols_q, "dA_2I": rows_q, "dB_t": cols_q, "dB_2I": rows_q})
    got = run_oracle(c)
    for key in ("dx", "dWg", "dWu"):
        assert not np.allclose(got[key], alt[key], rtol=1e-6), key


def test_saved_a_and_h_rounded_to_bf16_before_h_is_quantized():
    """a[T0, I0] = 64 + 3.5 + 0.234375 = 67.734375 rounds to the bf16 value
    67.5; with b = 1 + 2^-7, h = 67.5 * b = 68.02734375 rounds to 68, an E4M3
    midpoint at exponent 6 that goes to the even code, 64. Without the
    rounding of a, h would be bf16(68.2635) = 68.5, and without the rounding
    of h, 68.027: both quantize to 72. The forward quantizes its own,
    unrounded h = 68.2635 along I: 72."""
    c = base()
    c["X"][T0, 6], c["Wg"][I0, 6] = 3.5, 1.0          # a[T0, I0] = 64 + 3.5 ...
    c["X"][T0, 7], c["Wg"][I0, 7] = 1.0, 0.234375     # ... + 0.234375
    c["Wg"][I3, 7] = 0.5                              # (a[T0, I3] = 64.5, b there is 0)
    c["Wu"][I3, 3] = 0.0
    c["X"][T0, 5], c["Wu"][I0, 5] = 2.0 ** -7, 1.0    # b[T0, I0] = 1 + 2^-7
    c["X"][T0, 3], c["Wu"][I0, 3] = 1.0, 1.0
    c["X"][T2, 3] = 0.25
    c["dY"][T0] = 0.0
    c["dY"][T0, I1] = 1.0
    a_r = lambda V: put((T0, I0), 67.5)(put((T0, I3), 64.5)(V))   # noqa: E731
    check_case(c, {"a_bf16": a_r, "h_bf16": ((T0, I0), 68.0), "h_t": ((T0, I0), 64.0),
                   "h_I": ((T0, I0), 72.0)},
               affected={"dWd", "y"})


# ------------------------------------------------------------------ bf16 rounding
def test_bf16_round_hand_values():
    r = oracle.bf16_round
    assert r(1.0 + 2.0 ** -8) == 1.0                      # tie -> even
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6      # tie -> even (upwards)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7   # above the tie: no double rounding
    assert r(-1.0 - 2.0 ** -8 - 2.0 ** -30) == -(1.0 + 2.0 ** -7)
    assert r(255.5) == 256.0 and r(255.0) == 255.0
    assert r(2.0 ** -133) == 2.0 ** -133 and r(3 * 2.0 ** -134) == 2.0 ** -132   # subnormals
    assert r(3.38e38) == 1.984375 * 2.0 ** 127 and r(3.39e38) == 1.9921875 * 2.0 ** 127   # largest finite
    assert np.isinf(r(3.4e38)) and np.isinf(r(-1.9961 * 2.0 ** 127))
    assert np.signbit(r(-0.0))


@pytest.mark.parametrize("scale", [1e-3, 1.0, 1e4])
def test_bf16_round_matches_torch_on_float32_values(scale):
    import torch
    v = (np.random.default_rng(3).standard_normal(20000) * scale).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(v), ref)
