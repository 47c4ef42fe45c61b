"""Seeded synthetic workloads for a top-k routed SwiGLU mixture-of-experts layer.

Recipe (one NumPy PCG64 stream per tensor, so that any expert's weights can be
drawn on their own and in any order):

    SeedSequence(seed).spawn(4 + E):
        child 0      -> x      [T][H]  N(0, 1)
        child 1      -> Wr     [H][E]  N(0, 1/sqrt(H))   (router, fp32)
        child 2      -> rank permutation of the experts (load skew)
        child 3      -> dY     [T][H]  N(0, 1)
        child 4 + e  -> expert e: Wg [I][H] and Wu [I][H] with std 1/sqrt(H),
                        then Wd [H][I] with std 1/sqrt(I), drawn in that order

Every normal is drawn in float32, multiplied by its std in float32 and rounded
to bfloat16 (round to nearest even); bf16 tensors are returned as uint16 bit
patterns.

Routing (the router sits in front of the layer; the layer consumes its output):
    logits = x . Wr in float64 (x widened from bf16, Wr from fp32);
    score  = logits + bias_e, bias_e = -s * ln(rank_e) for a skewed workload
             (rank_e in 1..E from child 2; exp(bias) then follows Zipf(s)),
             and bias_e = -inf for the E/den lowest-ranked experts when the
             workload asks for empty experts;
    top-k  = the k largest scores, in descending order, ties to the lower
             expert id; slot j of token t is the j-th pick;
    topk_w = softmax over the k selected *unbiased* logits, stored as fp32.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np


@dataclasses.dataclass(frozen=True)
class Problem:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    seed: int = 0
    zipf_s: float = 0.0      # 0: no load-skew bias
    empty_den: int = 0       # >0: the E // empty_den lowest-ranked experts never chosen
    dtype: str = "bf16"      # "bf16" or "mxfp8"
    backward: bool = False

    @property
    def R(self) -> int:
        return self.T * self.k

    def fwd_flops(self) -> float:
        return 6.0 * self.R * self.H * self.I

    def bwd_flops(self) -> float:
        return 12.0 * self.R * self.H * self.I


# The five reference workloads.
CONFIGS = {
    0: Problem("bf16-fwd T256 H256 E8 k2 I512", 256, 256, 8, 2, 512, seed=0),
    1: Problem("bf16-fwd T4096 H2048 E64 k8 I768 uniform", 4096, 2048, 64, 8, 768, seed=1),
    2: Problem("bf16-fwd T16384 H4096 E128 k8 I1536 zipf1.2", 16384, 4096, 128, 8, 1536,
               seed=2, zipf_s=1.2, empty_den=16),
    3: Problem("mxfp8-fwd T16384 H4096 E128 k8 I1536 zipf1.2", 16384, 4096, 128, 8, 1536,
               seed=2, zipf_s=1.2, empty_den=16, dtype="mxfp8"),
    4: Problem("bf16-fwdbwd T16384 H7168 E32 k4 I2048 zipf0.8", 16384, 7168, 32, 4, 2048,
               seed=4, zipf_s=0.8, backward=True),
}


def problem(T, H, I, E, k, seed=0, zipf_s=0.0, empty_den=0, dtype="bf16", backward=False,
            name=None) -> Problem:
    """A workload of T tokens, hidden H, expert size I, E experts, top-k."""
    return Problem(name or f"T{T} H{H} E{E} k{k} I{I}", T, H, E, k, I, seed=seed,
                   zipf_s=zipf_s, empty_den=empty_den, dtype=dtype, backward=backward)


# ----------------------------------------------------------------------------- formats

def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a) -> np.ndarray:
    """Round float32 values to bf16 precision, returned as float32."""
    return bf16_to_f32(f32_to_bf16_bits(a))


# ----------------------------------------------------------------------------- streams

def _children(p: Problem):
    return np.random.SeedSequence(p.seed).spawn(4 + p.E)


def _normal_bf16(rng, shape, std: float) -> np.ndarray:
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


def make_x(p: Problem) -> np.ndarray:
    """x [T][H] bf16 bits, N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(_children(p)[0]))
    return _normal_bf16(rng, (p.T, p.H), 1.0)


def make_dy(p: Problem) -> np.ndarray:
    """Upstream gradient dY [T][H] bf16 bits, N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(_children(p)[3]))
    return _normal_bf16(rng, (p.T, p.H), 1.0)


def make_expert(p: Problem, e: int):
    """(Wg [I][H], Wu [I][H], Wd [H][I]) bf16 bits for expert e."""
    rng = np.random.Generator(np.random.PCG64(_children(p)[4 + e]))
    sh, si = 1.0 / math.sqrt(p.H), 1.0 / math.sqrt(p.I)
    wg = _normal_bf16(rng, (p.I, p.H), sh)
    wu = _normal_bf16(rng, (p.I, p.H), sh)
    wd = _normal_bf16(rng, (p.H, p.I), si)
    return wg, wu, wd


def make_all_experts(p: Problem, threads: int = 8):
    """Stacked weights Wg, Wu [E][I][H] and Wd [E][H][I] as bf16 bits."""
    wg = np.empty((p.E, p.I, p.H), np.uint16)
    wu = np.empty((p.E, p.I, p.H), np.uint16)
    wd = np.empty((p.E, p.H, p.I), np.uint16)

    def one(e):
        wg[e], wu[e], wd[e] = make_expert(p, e)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(p.E)))
    return wg, wu, wd


def expert_bias(p: Problem) -> np.ndarray:
    """Per-expert routing bias (float64 [E]) that shapes the load."""
    bias = np.zeros(p.E, np.float64)
    if p.zipf_s == 0.0 and p.empty_den == 0:
        return bias
    rng = np.random.Generator(np.random.PCG64(_children(p)[2]))
    rank = rng.permutation(p.E) + 1                       # rank_e in 1..E
    if p.zipf_s:
        bias = -p.zipf_s * np.log(rank.astype(np.float64))
    if p.empty_den:
        n_empty = p.E // p.empty_den
        bias[rank > p.E - n_empty] = -np.inf
    return bias


def router_weights(p: Problem):
    """(Wr [H][E] float32, selection bias [E] float64) of the seeded router."""
    rng = np.random.Generator(np.random.PCG64(_children(p)[1]))
    wr = rng.standard_normal((p.H, p.E), dtype=np.float32)
    wr *= np.float32(1.0 / math.sqrt(p.H))
    return wr, expert_bias(p)


def make_routing(p: Problem, x_bits: np.ndarray, chunk: int = 2048):
    """(topk_ids int32 [T][k], topk_w float32 [T][k]) from the seeded router."""
    wr, bias = router_weights(p)
    wr64 = wr.astype(np.float64)
    ids = np.empty((p.T, p.k), np.int32)
    w = np.empty((p.T, p.k), np.float32)
    for t0 in range(0, p.T, chunk):
        xs = bf16_to_f32(x_bits[t0:t0 + chunk]).astype(np.float64)
        logits = xs @ wr64
        score = logits + bias[None, :]
        order = np.argsort(-score, axis=1, kind="stable")[:, :p.k]
        sel = np.take_along_axis(logits, order, axis=1)
        sel = np.exp(sel - sel.max(axis=1, keepdims=True))
        ids[t0:t0 + chunk] = order
        w[t0:t0 + chunk] = (sel / sel.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w
