"""Helpers shared by the GPU parity tests: moving synthetic bf16 bit patterns to
and from the device, fp64 views of expert weights for the oracle, and the
tolerance checks."""
from __future__ import annotations

import numpy as np

from synthetic import bf16_to_f32

# Parity bar for bf16 results against the fp64 oracle.
REL_FRO_BF16 = 1e-2
MAX_ABS_FRAC_BF16 = 5e-2
# MXFP8 forward and backward against the oracle's MXFP8 forward and backward
# (the same quantized operands: weights, x and h, and in the backward dO, dA|dB
# and h, each quantized from the same bf16 values on both sides).
REL_FRO_MXFP8 = 2e-2


def to_dev_bf16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def from_dev_bf16(t):
    import torch
    return bf16_to_f32(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)).astype(np.float64)


def f64(bits):
    return bf16_to_f32(bits).astype(np.float64)


class ExpertsF64:
    """experts[e] -> (Wg, Wu, Wd) as float64, converted on demand."""

    def __init__(self, wg, wu, wd):
        self.wg, self.wu, self.wd = wg, wu, wd

    def __len__(self):
        return self.wg.shape[0]

    def __getitem__(self, e):
        return f64(self.wg[e]), f64(self.wu[e]), f64(self.wd[e])


class ExpertsSliceI:
    """experts[e] restricted to the intermediate channels [i0, i1): rows of Wg
    and Wu, columns of Wd. Every quantity the MXFP8 weight gradients are made
    of is channel-local: a and b (x and the Wg, Wu rows blocked along H), dh
    (dO and the Wd columns blocked along H), dA, dB and h elementwise, and
    their token-blocked copies blocked per channel along the rows; nothing
    in that path is blocked along I. So the backward's dWg, dWu rows and dWd
    columns of the range come out as with all channels (not dX, whose
    operand dA|dB is blocked along 2I, nor d topk_w, which takes the forward
    output)."""

    def __init__(self, experts, i0, i1):
        assert 0 <= i0 < i1
        self.ex, self.i0, self.i1 = experts, i0, i1

    def __len__(self):
        return len(self.ex)

    def __getitem__(self, e):
        wg, wu, wd = self.ex[e]
        return wg[self.i0:self.i1], wu[self.i0:self.i1], wd[:, self.i0:self.i1]


def rel_fro(got, ref):
    n = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (n if n > 0 else 1.0)


def assert_close_bf16(got, ref, what="", rel=REL_FRO_BF16, frac=MAX_ABS_FRAC_BF16):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    r = rel_fro(got, ref)
    m = np.max(np.abs(got - ref)) if ref.size else 0.0
    lim = frac * (np.max(np.abs(ref)) if ref.size else 0.0)
    assert r <= rel, f"{what}: relative Frobenius error {r:.3e} > {rel}"
    assert m <= lim + 1e-30, f"{what}: max |err| {m:.3e} > {lim:.3e}"
    return r, m
