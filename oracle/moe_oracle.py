"""Plain, slow, obviously-correct CPU fp64 oracle of the deterministic MoE layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
the CPU-baseline leg of bench.py, never by the product path.

Sources (cited by title and section):
  [MoK card] "Mixture-Of-Kittens (MoK)" project card,
             agentlenshq.com/zh-CN/projects/ghp:cursor/mixture-of-kittens
  [MoK clip] "Mixture-of-Kittens: Cursor open-sources an MoE training
             megakernel", miguoliang.com/clip/mixture-of-kittens
  [OCP MX]   OCP Microscaling Formats (MX) Specification v1.0 (the MXFP8 block
             format the card names but does not define).

Everything is float64. Inputs that are bf16/fp32 on the device are passed in
already widened to float64 (exact). Expert weights are passed as a sequence
`experts` with experts[e] -> (Wg [I][H], Wu [I][H], Wd [H][I]) float64, so a
caller can convert one expert at a time.

Notation: T tokens, H hidden, I expert intermediate size, E experts, k picks
per token, R = T*k routed rows, flat row i = t*k + j, permuted row p.

Readings where the pages are silent (each stated where it is used):
  * the expert FFN is SwiGLU with no biases: h = silu(x.Wg^T) * (x.Wu^T),
    out = h.Wd^T, silu(a) = a*sigmoid(a);
  * "stable" permutation = sort rows by expert id, ties by flat index i;
  * an expert id outside [0, E) sets status bit 0; such rows are placed after
    all valid rows (ascending i), are not counted in any expert, and their
    expert output is zero;
  * the combine uses topk_w as given (no renormalisation), j ascending;
  * minibatch m holds permuted rows [m*M, (m+1)*M) and lives in ring slot
    m mod N_s;
  * the gradient "of the router weights" is d y / d topk_w.
"""
from __future__ import annotations

import numpy as np

STATUS_BAD_EXPERT_ID = 1


# ============================================================================ schedule
def schedule(topk_ids, E):
    """Routing schedule built from the top-k choices.

    [MoK card] "Using the functional API": the schedule is built from the
    top-k expert choices and is shared by forward and backward.
    [MoK clip] Key points, bullet 4: routed-token counts stay on the device;
    How-to item 2: one schedule table serves all four exchange passes.

    counts[e]  = #{i : f[i] = e}
    offsets    = exclusive prefix sum of counts, offsets[E] = #valid rows
    perm[p]    = flat row i placed at permuted position p (stable by i)
    dest[i]    = p with perm[p] = i
    """
    f = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    R = f.size
    valid = (f >= 0) & (f < E)
    status = 0 if valid.all() else STATUS_BAD_EXPERT_ID
    key = np.where(valid, f, E)                      # invalid rows sort last
    counts = np.bincount(key, minlength=E + 1)[:E].astype(np.int64)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(key, kind="stable").astype(np.int64)
    dest = np.empty(R, np.int64)
    dest[perm] = np.arange(R, dtype=np.int64)
    return {"counts": counts, "offsets": offsets, "perm": perm, "dest": dest,
            "status": status, "R": R, "E": E}


def minibatch_count(R, M):
    """Number of fixed-size minibatches of M permuted rows ([MoK clip] Key
    points, bullet 3: a tunable minibatch is the unit of overlap)."""
    return (R + M - 1) // M


def ring_row(p, M, n_slots):
    """Row of the ring token buffer that permuted row p occupies.

    [MoK clip] Key points, bullet 4 and How-to item 4: a fixed-size ring
    ("macrobatch") of token slots reused on the device. Minibatch m = p // M
    goes to slot m mod n_slots; the row keeps its offset inside the minibatch.
    """
    p = np.asarray(p, dtype=np.int64)
    return ((p // M) % n_slots) * M + p % M


# ============================================================================ expert FFN
def sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def silu(a):
    return a * sigmoid(a)


def swiglu(a, b):
    """SwiGLU gate: silu(a) * b ([MoK clip] Key points, bullet 5 and the key
    chart name the expert FFN "SwiGLU"; gate = a, up = b)."""
    return silu(a) * b


def expert_ffn(X, Wg, Wu, Wd):
    """One expert's SwiGLU FFN on rows X [n][H] -> (out [n][H], a, b, h)."""
    a = X @ Wg.T
    b = X @ Wu.T
    h = swiglu(a, b)
    return h @ Wd.T, a, b, h


# ============================================================================ forward
def forward(x, topk_ids, topk_w, experts):
    """MoE layer forward: dispatch -> per-expert SwiGLU FFN -> weighted combine.

    [MoK clip] Conclusion and the key chart: router top-k -> dispatch of token
    rows to their experts -> expert FFN (SwiGLU) -> combine -> weighted sum.
    [MoK clip] How-to item 6: a fixed accumulation order; here the combine
    adds j = 0..k-1 in ascending order.

    Returns y [T][H] and ctx = {sched, obuf [R][H] (flat row order),
    a, b [R][I] (permuted order)}.
    """
    x = np.asarray(x, np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids).reshape(T, -1)
    k = ids.shape[1]
    E = len(experts)
    s = schedule(ids, E)
    R = T * k
    obuf = np.zeros((R, H), np.float64)
    I = np.asarray(experts[0][0]).shape[0] if E else 0
    a_all = np.zeros((R, I), np.float64)
    b_all = np.zeros((R, I), np.float64)
    for e in range(E):
        lo, hi = s["offsets"][e], s["offsets"][e + 1]
        if hi == lo:
            continue
        P = s["perm"][lo:hi]
        Wg, Wu, Wd = experts[e]
        out, a, b, _ = expert_ffn(x[P // k], Wg, Wu, Wd)
        obuf[P] = out
        a_all[lo:hi] = a
        b_all[lo:hi] = b
    w = np.asarray(topk_w, np.float64).reshape(T, k)
    y = np.zeros((T, H), np.float64)
    ob = obuf.reshape(T, k, H)
    for j in range(k):
        y += w[:, j:j + 1] * ob[:, j, :]
    return y, {"sched": s, "obuf": obuf, "a": a_all, "b": b_all}


def forward_tokens(x_rows, ids_rows, w_rows, experts):
    """y for a subset of tokens, straight from the definition
    y[t] = sum_j w[t, j] * FFN_{ids[t, j]}(x[t]) (rows with an invalid id add 0).
    Also returns the per-(t, j) expert outputs [n][k][H]."""
    x_rows = np.asarray(x_rows, np.float64)
    n, H = x_rows.shape
    ids_rows = np.asarray(ids_rows).reshape(n, -1)
    w_rows = np.asarray(w_rows, np.float64).reshape(n, -1)
    k = ids_rows.shape[1]
    E = len(experts)
    outs = np.zeros((n, k, H), np.float64)
    for e in sorted(set(int(v) for v in ids_rows.reshape(-1) if 0 <= v < E)):
        sel = np.argwhere(ids_rows == e)
        Wg, Wu, Wd = experts[e]
        out, _, _, _ = expert_ffn(x_rows[sel[:, 0]], Wg, Wu, Wd)
        outs[sel[:, 0], sel[:, 1]] = out
    y = np.zeros((n, H), np.float64)
    for j in range(k):
        y += w_rows[:, j:j + 1] * outs[:, j, :]
    return y, outs


# ============================================================================ backward
def _swiglu_backward(dh, a, b):
    """d/da and d/db of silu(a)*b:
    dA = dh * b * sig(a) * (1 + a * (1 - sig(a))),  dB = dh * a * sig(a)."""
    sg = sigmoid(a)
    return dh * b * sg * (1.0 + a * (1.0 - sg)), dh * a * sg


def backward(x, topk_ids, topk_w, experts, dy):
    """Backward of the layer for upstream gradient dy [T][H].

    [MoK card] "What it is" and "Using the functional API": forward and
    backward are both provided, backward reuses the schedule.
    [MoK clip] How-to item 2: backward is reverse-combine (dY to the routed
    rows) then reverse-dispatch (row gradients back to their token).

    Returns dict dx [T][H], dWg/dWu [E][I][H], dWd [E][H][I], dw [T][k].
    An expert with no rows gets exact zero weight gradients.
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids).reshape(T, -1)
    k = ids.shape[1]
    E = len(experts)
    w = np.asarray(topk_w, np.float64).reshape(T, k)
    y, ctx = forward(x, ids, w, experts)
    s = ctx["sched"]
    R = T * k
    I = np.asarray(experts[0][0]).shape[0]
    ob = ctx["obuf"].reshape(T, k, H)
    dw = np.einsum("th,tjh->tj", dy, ob)           # reverse-combine: d w[t, j]
    wf = w.reshape(-1)
    dxrows = np.zeros((R, H), np.float64)
    dWg = np.zeros((E, I, H))
    dWu = np.zeros((E, I, H))
    dWd = np.zeros((E, H, I))
    for e in range(E):
        lo, hi = s["offsets"][e], s["offsets"][e + 1]
        if hi == lo:
            continue
        P = s["perm"][lo:hi]
        Wg, Wu, Wd = experts[e]
        X = x[P // k]
        a, b = ctx["a"][lo:hi], ctx["b"][lo:hi]
        h = swiglu(a, b)
        dO = wf[P][:, None] * dy[P // k]           # reverse-combine: dY to rows
        dh = dO @ Wd
        dWd[e] = dO.T @ h
        dA, dB = _swiglu_backward(dh, a, b)
        dWg[e] = dA.T @ X
        dWu[e] = dB.T @ X
        dxrows[P] = dA @ Wg + dB @ Wu
    dx = dxrows.reshape(T, k, H).sum(axis=1)       # reverse-dispatch
    return {"dx": dx, "dWg": dWg, "dWu": dWu, "dWd": dWd, "dw": dw, "y": y}


def backward_tokens(x_rows, ids_rows, w_rows, experts, dy_rows):
    """dx and dw for a subset of tokens, from the per-row definition:
    dw[t,j] = <dy[t], FFN_e(x[t])>; dx[t] = sum_j (dA Wg_e + dB Wu_e) with
    dO = w[t,j] dy[t]."""
    x_rows = np.asarray(x_rows, np.float64)
    dy_rows = np.asarray(dy_rows, np.float64)
    n, H = x_rows.shape
    ids_rows = np.asarray(ids_rows).reshape(n, -1)
    w_rows = np.asarray(w_rows, np.float64).reshape(n, -1)
    k = ids_rows.shape[1]
    E = len(experts)
    dx = np.zeros((n, H))
    dw = np.zeros((n, k))
    for e in sorted(set(int(v) for v in ids_rows.reshape(-1) if 0 <= v < E)):
        sel = np.argwhere(ids_rows == e)
        t, j = sel[:, 0], sel[:, 1]
        Wg, Wu, Wd = experts[e]
        out, a, b, _ = expert_ffn(x_rows[t], Wg, Wu, Wd)
        dw[t, j] = np.sum(dy_rows[t] * out, axis=1)
        dh = (w_rows[t, j][:, None] * dy_rows[t]) @ Wd
        dA, dB = _swiglu_backward(dh, a, b)
        np.add.at(dx, t, dA @ Wg + dB @ Wu)
    return dx, dw


def backward_expert_weights(e, x, topk_ids, topk_w, experts, dy):
    """(dWg[e], dWu[e], dWd[e]) for one expert from all rows routed to it."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids).reshape(T, -1)
    k = ids.shape[1]
    w = np.asarray(topk_w, np.float64).reshape(T, k)
    sel = np.argwhere(ids == e)                     # ascending flat index
    Wg, Wu, Wd = experts[e]
    I = Wg.shape[0]
    if sel.size == 0:
        return np.zeros((I, H)), np.zeros((I, H)), np.zeros((H, I))
    t, j = sel[:, 0], sel[:, 1]
    X = x[t]
    _, a, b, h = expert_ffn(X, Wg, Wu, Wd)
    dO = w[t, j][:, None] * np.asarray(dy, np.float64)[t]
    dh = dO @ Wd
    dA, dB = _swiglu_backward(dh, a, b)
    return dA.T @ X, dB.T @ X, dO.T @ h


# ============================================================================ MXFP8
# [MoK card] "Core concepts" table and "Limits": MXFP8 is a low-precision
# weight format, weights are pre-quantized by an op before the kernel sees
# them. The block format is the one [OCP MX] defines: 32 elements share one
# E8M0 scale (2^(s-127)); each element is FP8 E4M3 (bias 7, no infinities,
# S.1111.111 = NaN, largest finite 448).

E4M3_MAX = 448.0


def e4m3_decode(code):
    """Value of an E4M3 code (vectorised). NaN for S.1111.111."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    v = np.where(e == 0, sub, nrm)
    v = np.where((e == 0xF) & ((c & 7) == 7), np.nan, v)
    return sign * v


def _round_half_even(q):
    return np.round(q)                               # numpy rounds half to even


def e4m3_encode(v):
    """Round float64 values to E4M3, nearest-even, saturating at +-448.
    The sign bit is copied from the input, so -0.0 and negative values that
    round to zero give 0x80."""
    v = np.asarray(v, np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    code = np.zeros(a.shape, np.int64)
    # subnormal range |v| < 2^-6: step 2^-9; a quotient of 8 is code 0x08 (2^-6)
    sub = a < 2.0 ** -6
    code = np.where(sub, _round_half_even(a * 2.0 ** 9).astype(np.int64), code)
    # normal range: exponent from frexp, 3 mantissa bits
    mant, ex = np.frexp(np.where(sub, 1.0, a))      # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                                       # a = (2*mant) * 2^e
    q = _round_half_even((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    ncode = ((e + 7) << 3) | q
    ncode = np.where(a > E4M3_MAX, 0x7E, np.minimum(ncode, 0x7E))
    code = np.where(sub, code, ncode)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def mxfp8_quantize(v):
    """Quantize along the last axis in blocks of 32 ([OCP MX] scale rule).

    Per block: amax = max |v|; e = floor(log2 amax) - 8 (8 = largest E4M3
    exponent); scale byte s = clamp(e + 127, 0, 254), s = 0 for an all-zero
    block; code = E4M3(v / 2^(s - 127)), round to nearest even, saturating.
    Returns (codes uint8 [..., K], scales uint8 [..., K/32]).
    """
    v = np.asarray(v, np.float64)
    K = v.shape[-1]
    assert K % 32 == 0
    blocks = v.reshape(v.shape[:-1] + (K // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    s = np.clip(ex - 1 - 8 + 127, 0, 254)
    s = np.where(amax > 0, s, 0).astype(np.int64)
    scale = np.exp2(s.astype(np.float64) - 127.0)
    codes = e4m3_encode(blocks / scale[..., None])
    return codes.reshape(v.shape), s.astype(np.uint8)


def mxfp8_dequantize(codes, scales):
    codes = np.asarray(codes)
    K = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (K // 32, 32))
    scale = np.exp2(np.asarray(scales, np.float64) - 127.0)
    return (vals * scale[..., None]).reshape(codes.shape)


def mxfp8_roundtrip(v):
    return mxfp8_dequantize(*mxfp8_quantize(v))


def _mx_experts(experts):
    """Expert weights as the MXFP8 kernel sees them: each matrix quantized
    along its contraction axis (H for Wg/Wu, I for Wd) and dequantized."""
    class _Q:
        def __len__(self):
            return len(experts)

        def __getitem__(self, e):
            Wg, Wu, Wd = experts[e]
            return mxfp8_roundtrip(Wg), mxfp8_roundtrip(Wu), mxfp8_roundtrip(Wd)
    return _Q()


def _mx_ffn(X, Wg, Wu, Wd, with_ab=False):
    a = mxfp8_roundtrip(X) @ Wg.T
    b = mxfp8_roundtrip(X) @ Wu.T
    h = mxfp8_roundtrip(swiglu(a, b))
    out = h @ Wd.T
    return (out, a, b) if with_ab else out


def forward_mxfp8(x, topk_ids, topk_w, experts):
    """MXFP8 forward: both GEMMs take MXFP8 operands. Weights are quantized
    along their contraction axis, each gathered x row along H, and the SwiGLU
    output h along I; accumulation and the combine are exact (fp64)."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids).reshape(T, -1)
    k = ids.shape[1]
    qexp = _mx_experts(experts)
    s = schedule(ids, len(experts))
    obuf = np.zeros((T * k, H))
    for e in range(len(experts)):
        lo, hi = s["offsets"][e], s["offsets"][e + 1]
        if hi == lo:
            continue
        P = s["perm"][lo:hi]
        obuf[P] = _mx_ffn(x[P // k], *qexp[e])
    w = np.asarray(topk_w, np.float64).reshape(T, k)
    y = np.einsum("tj,tjh->th", w, obuf.reshape(T, k, H))
    return y, {"sched": s, "obuf": obuf}


def forward_mxfp8_tokens(x_rows, ids_rows, w_rows, experts):
    """forward_mxfp8 restricted to a subset of tokens (per-row definition)."""
    x_rows = np.asarray(x_rows, np.float64)
    n, H = x_rows.shape
    ids_rows = np.asarray(ids_rows).reshape(n, -1)
    w_rows = np.asarray(w_rows, np.float64).reshape(n, -1)
    k = ids_rows.shape[1]
    qexp = _mx_experts(experts)
    outs = np.zeros((n, k, H))
    for e in sorted(set(int(v) for v in ids_rows.reshape(-1) if 0 <= v < len(experts))):
        sel = np.argwhere(ids_rows == e)
        outs[sel[:, 0], sel[:, 1]] = _mx_ffn(x_rows[sel[:, 0]], *qexp[e])
    return np.einsum("tj,tjh->th", w_rows, outs), outs



# ============================================================================ MXFP8 backward
# [MoK card] "What it is": the layer supports BF16 and MXFP8, forward and
# backward; "Limits": MXFP8 needs the weights pre-quantized by the op. The
# pages do not say which backward operands are quantized along which axis;
# the reading here (every operand of every backward GEMM is MXFP8, blocked
# along that GEMM's contraction axis, because the scaled MFMA takes 8-bit A
# and B with scales along K):
#   dh        = Q_H(dO)       . Q_H(Wd)          K = H
#   dXrows    = Q_I([dA|dB])  . Q_I([Wg; Wu])    K = 2I
#   dWd[e]    = Q_t(dO)^T     . Q_t(h)           K = the expert's rows
#   dWg|u[e]  = Q_t(dA|dB)^T  . Q_t(X)           K = the expert's rows
# Q_H / Q_I quantize along H / I; Q_t quantizes along the expert's rows in
# blocks of 32 counted from its first permuted row (the last block is padded
# with zeros, which changes no block maximum). Storage precision (the reading
# that intermediates are kept in bf16, applied to the MXFP8 backward): the
# forward saves a, b as bf16 values; h = silu(a)*b from those, dO = w*dy and
# the SwiGLU gradients dA, dB are each rounded to bf16 once, and it is these
# bf16 values that every quantization above takes (x is bf16 already). d
# topk_w and dx are as in the bf16 backward.


def bf16_round(v):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps float32's 8-bit exponent and 8 significant bits (7 stored),
    so a normal value m * 2^e with 0.5 <= |m| < 1 rounds to a multiple of
    2^(e - 8); below 2^-126 the step is 2^-133 (subnormals). The rounding is
    done once, straight from float64 (no double rounding through float32).
    Magnitudes that round to 2^128 or beyond become infinite.
    """
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)
    r = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)
    r = np.where(np.abs(v) < 2.0 ** -126, np.round(v * 2.0 ** 133) * 2.0 ** -133, r)
    with np.errstate(invalid="ignore"):
        return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)


def _mx_along_rows(V):
    """Quantize-dequantize V [n][K] along K (each row, blocks of 32)."""
    return mxfp8_roundtrip(V)


def _mx_along_cols(V):
    """Quantize-dequantize V [K][n] along K (each column, blocks of 32)."""
    return mxfp8_roundtrip(np.asarray(V, np.float64).T).T


def _mx_along_tokens(V):
    """Quantize-dequantize V [c][n] along its c rows in blocks of 32 starting
    at row 0; rows past c (up to a multiple of 32) are zero padding."""
    V = np.asarray(V, np.float64)
    c = V.shape[0]
    cp = -(-c // 32) * 32
    Vp = np.zeros((cp,) + V.shape[1:])
    Vp[:c] = V
    return _mx_along_cols(Vp)[:c]


def _mx_backward_rows(X, dYr, wr, W, Q):
    """One expert's rows in permuted order: X [c][H] their x rows, dYr [c][H]
    the upstream gradient of their tokens, wr [c] their combine weights; W the
    expert's exact (Wg, Wu, Wd), Q its dequantized forward copies.
    Returns the rows' expert outputs and dX rows (both row-local), and the
    expert's dWg, dWu, dWd (which need all of its rows)."""
    Wg, Wu, Wd = W
    out, a, b = _mx_ffn(X, *Q, with_ab=True)
    a, b = bf16_round(a), bf16_round(b)            # saved by the forward in bf16
    h = bf16_round(swiglu(a, b))
    dO = bf16_round(wr[:, None] * dYr)
    dh = _mx_along_rows(dO) @ _mx_along_cols(Wd)
    dA, dB = (bf16_round(g) for g in _swiglu_backward(dh, a, b))
    dAB = _mx_along_rows(np.concatenate([dA, dB], axis=1))
    dxr = dAB @ _mx_along_cols(np.concatenate([Wg, Wu], axis=0))
    Xt = _mx_along_tokens(X)
    dWg = _mx_along_tokens(dA).T @ Xt
    dWu = _mx_along_tokens(dB).T @ Xt
    dWd = _mx_along_tokens(dO).T @ _mx_along_tokens(h)
    return out, dxr, dWg, dWu, dWd


def backward_mxfp8(x, topk_ids, topk_w, experts, dy):
    """MXFP8 backward (readings above). Returns the same dict as backward()."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids).reshape(T, -1)
    k = ids.shape[1]
    E = len(experts)
    w = np.asarray(topk_w, np.float64).reshape(T, k)
    s = schedule(ids, E)
    R = T * k
    I = np.asarray(experts[0][0]).shape[0]
    qexp = _mx_experts(experts)
    wf = w.reshape(-1)
    obuf = np.zeros((R, H))
    dxrows = np.zeros((R, H))
    dWg = np.zeros((E, I, H))
    dWu = np.zeros((E, I, H))
    dWd = np.zeros((E, H, I))
    for e in range(E):
        lo, hi = s["offsets"][e], s["offsets"][e + 1]
        if hi == lo:
            continue
        P = s["perm"][lo:hi]
        obuf[P], dxrows[P], dWg[e], dWu[e], dWd[e] = _mx_backward_rows(
            x[P // k], dy[P // k], wf[P], experts[e], qexp[e])
    y = np.einsum("tj,tjh->th", w, obuf.reshape(T, k, H))
    dw = np.einsum("th,tjh->tj", dy, obuf.reshape(T, k, H))
    dx = dxrows.reshape(T, k, H).sum(axis=1)
    return {"dx": dx, "dWg": dWg, "dWu": dWu, "dWd": dWd, "dw": dw, "y": y}


def backward_mxfp8_expert_weights(e, x, topk_ids, topk_w, experts, dy):
    """(dWg[e], dWu[e], dWd[e]) of the MXFP8 backward for one expert, from all
    rows routed to it (in permuted order: ascending flat index)."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids).reshape(T, -1)
    w = np.asarray(topk_w, np.float64).reshape(ids.shape)
    sel = np.argwhere(ids == e)
    Wg, Wu, Wd = experts[e]
    I = Wg.shape[0]
    if sel.size == 0:
        return np.zeros((I, H)), np.zeros((I, H)), np.zeros((H, I))
    t, j = sel[:, 0], sel[:, 1]
    _, _, dWg, dWu, dWd = _mx_backward_rows(x[t], np.asarray(dy, np.float64)[t], w[t, j], experts[e],
                                            _mx_experts(experts)[e])
    return dWg, dWu, dWd


def backward_mxfp8_tokens(x_rows, ids_rows, w_rows, experts, dy_rows):
    """dx and d topk_w of the MXFP8 backward for a subset of tokens (their
    parts are row-local: per-row quantization along H and 2I)."""
    x_rows = np.asarray(x_rows, np.float64)
    dy_rows = np.asarray(dy_rows, np.float64)
    n, H = x_rows.shape
    ids_rows = np.asarray(ids_rows).reshape(n, -1)
    w_rows = np.asarray(w_rows, np.float64).reshape(n, -1)
    qexp = _mx_experts(experts)
    dx = np.zeros((n, H))
    dw = np.zeros(ids_rows.shape)
    for e in sorted(set(int(v) for v in ids_rows.reshape(-1) if 0 <= v < len(experts))):
        sel = np.argwhere(ids_rows == e)
        t, j = sel[:, 0], sel[:, 1]
        out, dxr, _, _, _ = _mx_backward_rows(x_rows[t], dy_rows[t], w_rows[t, j], experts[e], qexp[e])
        dw[t, j] = np.sum(dy_rows[t] * out, axis=1)
        np.add.at(dx, t, dxr)
    return dx, dw


# ============================================================================ router front end
# [MoK clip] key chart, "Router picks top-k": the router scores every expert
# for a token and hands the layer its k experts and their combine weights.
# The pages give no formula; the plainest reading, the one the workloads use:
#   * logits = x . Wr^T with Wr [E][H] (one row per expert), no bias term in
#     the logits themselves;
#   * an optional per-expert bias shifts the selection score only
#     (score = logit + bias_e), as the skewed workloads shape expert loads;
#   * the k experts with the largest scores, in descending score, equal scores
#     in ascending expert id;
#   * combine weights = softmax over the k selected *unbiased* logits.
# The backward runs from d topk_w: the selection is piecewise constant, so
# only the selected logits get gradients, through the softmax Jacobian.

def router_forward(x, wr, bias, k):
    """(logits [T][E], topk_ids int32 [T][k], topk_w [T][k]) in float64."""
    logits = x @ wr.T
    score = logits if bias is None else logits + np.asarray(bias)[None, :]
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        # descending score, ties to the lower id: sort on (-score, id)
        order = sorted(range(E), key=lambda e: (-score[t, e], e))
        ids[t] = order[:k]
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    return logits, ids, ex / ex.sum(axis=1, keepdims=True)


def router_backward(x, wr, topk_ids, topk_w, d_topk_w):
    """d of sum(d_topk_w * topk_w) through the softmax of the selected logits.

    Returns (d_sel [T][k]: gradient of each selected logit,
             d_logits [T][E]: the same scattered, zero for unselected experts,
             d_wr [E][H] = d_logits^T . x, dx [T][H] = d_logits . Wr)."""
    w = np.asarray(topk_w, np.float64)
    g = np.asarray(d_topk_w, np.float64)
    d_sel = w * (g - (w * g).sum(axis=1, keepdims=True))
    T, k = topk_ids.shape
    d_logits = np.zeros((T, wr.shape[0]))
    for t in range(T):
        for j in range(k):
            d_logits[t, topk_ids[t, j]] += d_sel[t, j]
    return d_sel, d_logits, d_logits.T @ x, d_logits @ wr
