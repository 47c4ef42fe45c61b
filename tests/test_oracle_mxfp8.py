"""Pins for the oracle's MXFP8 quantizer and MXFP8 forward (CPU only).

The block format is OCP MX v1.0 (E4M3 elements, one E8M0 scale per 32). The
spec's E4M3 values sit in tests/golden/e4m3_spec_values.json; torch's
float8_e4m3fn is an independent library encoder/decoder for in-range values.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from test_oracle_forward import rand_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spec_values.json")


def torch_e4m3_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_spec_values():
    g = json.load(open(GOLDEN))
    for code, val in g["e4m3"]:
        v = oracle.e4m3_decode(int(code, 16))
        assert v == val and np.signbit(v) == np.signbit(val), (code, v, val)
    for code in g["e4m3_nan"]:
        assert np.isnan(oracle.e4m3_decode(int(code, 16)))


def test_decode_all_codes_match_torch():
    ours = oracle.e4m3_decode(np.arange(256))
    ref = torch_e4m3_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_encode_every_code_round_trips():
    vals = oracle.e4m3_decode(np.arange(256))
    ok = ~np.isnan(vals)
    codes = oracle.e4m3_encode(vals[ok])
    assert np.array_equal(codes, np.arange(256)[ok].astype(np.uint8))


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000) * 30,
        rng.standard_normal(20000) * 0.01,
        rng.uniform(-448, 448, 20000),
    ])
    # all midpoints between neighbouring finite codes (ties to even)
    pos = np.sort(oracle.e4m3_decode(np.arange(0, 0x7F)))
    mids = (pos[:-1] + pos[1:]) / 2
    v = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v), ref)


def test_ties_to_even_and_saturation():
    enc = lambda v: int(oracle.e4m3_encode(np.array(v)))  # noqa: E731
    assert enc(1.0625) == 0x38      # halfway 1.0 / 1.125 -> even mantissa (1.0)
    assert enc(1.1875) == 0x3A      # halfway 1.125 / 1.25 -> 1.25
    assert enc(2.0 ** -10) == 0x00  # halfway 0 / 2^-9 -> 0
    assert enc(3 * 2.0 ** -10) == 0x02
    assert enc(464.0) == 0x7E       # above 448 saturates
    assert enc(1e9) == 0x7E and enc(-1e9) == 0xFE
    assert enc(-0.0) == 0x80 and enc(-2.0 ** -12) == 0x80


def test_worked_block_values():
    # amax 1.0 -> scale byte 127 + 0 - 8 = 119; 1.0 / 2^-8 = 256 -> 0x78
    blk = np.zeros(32)
    blk[0] = 1.0
    blk[5] = -0.5
    q, s = oracle.mxfp8_quantize(blk)
    assert s.tolist() == [119]
    assert q[0] == 0x78 and q[5] == 0xF0 and q[1] == 0
    # amax bf16(1.9) = 1.8984375 -> scale 119, 1.8984375 * 256 = 486 -> saturates to 0x7E
    blk[0] = 1.8984375
    q, s = oracle.mxfp8_quantize(blk)
    assert s.tolist() == [119] and q[0] == 0x7E
    assert oracle.mxfp8_dequantize(q, s)[0] == 1.75
    # all-zero block -> scale 0, codes 0
    q, s = oracle.mxfp8_quantize(np.zeros(64))
    assert s.tolist() == [0, 0] and not q.any()
    # scale byte follows floor(log2 amax): tiny and huge blocks
    for e in (-130, -120, -5, 0, 3, 60, 127):
        blk = np.zeros(32)
        blk[7] = 2.0 ** e * 1.5
        _, s = oracle.mxfp8_quantize(blk)
        assert s[0] == max(0, min(254, e - 8 + 127))


def test_round_trip_of_representable_blocks():
    rng = np.random.default_rng(1)
    for e in (-20, -3, 0, 7):
        codes = rng.integers(0, 0x7F, size=32)
        codes[rng.integers(32)] = 0x7E          # pin the amax to 448 * 2^e
        signs = rng.integers(0, 2, size=32) * 0x80
        c = (codes | signs).astype(np.uint8)
        v = oracle.e4m3_decode(c) * 2.0 ** e
        q, s = oracle.mxfp8_quantize(v)
        assert s[0] == e + 127
        ok = oracle.e4m3_decode(c) != 0
        assert np.array_equal(q[ok], c[ok])
        np.testing.assert_array_equal(oracle.mxfp8_dequantize(q, s), v)


def test_quantize_is_row_local():
    rng = np.random.default_rng(2)
    m = rng.standard_normal((6, 64))
    q, s = oracle.mxfp8_quantize(m)
    for r in range(6):
        qr, sr = oracle.mxfp8_quantize(m[r])
        assert np.array_equal(qr, q[r]) and np.array_equal(sr, s[r])


def test_mxfp8_forward_equals_exact_forward_on_representable_inputs():
    # Operands already in MXFP8 (E4M3 codes times one power of two per block):
    # quantizing them again is the identity, so the MXFP8 forward must equal
    # a per-token loop that only rounds h.
    x, ids, w, ex = rand_case(T=8, H=64, I=32, E=3, k=2, seed=3)
    xr = oracle.mxfp8_roundtrip(x)
    np.testing.assert_array_equal(oracle.mxfp8_roundtrip(xr), xr)
    exr = [tuple(oracle.mxfp8_roundtrip(m) for m in t) for t in ex]
    y_mx, _ = oracle.forward_mxfp8(xr, ids, w, exr)
    # reference: exact forward with the h quantization applied explicitly
    T, k = ids.shape
    y = np.zeros((T, 64))
    for t in range(T):
        for j in range(k):
            Wg, Wu, Wd = exr[ids[t, j]]
            a, b = Wg @ xr[t], Wu @ xr[t]
            h = oracle.mxfp8_roundtrip((a / (1 + np.exp(-a)) * b)[None, :])[0]
            y[t] += w[t, j] * (Wd @ h)
    np.testing.assert_allclose(y_mx, y, rtol=1e-12, atol=1e-12)


def test_mxfp8_forward_close_to_exact_forward():
    x, ids, w, ex = rand_case(T=32, H=128, I=64, E=4, k=2, seed=4)
    y, _ = oracle.forward(x, ids, w, ex)
    ymx, _ = oracle.forward_mxfp8(x, ids, w, ex)
    rel = np.linalg.norm(ymx - y) / np.linalg.norm(y)
    assert 1e-3 < rel < 0.08
    ys, _ = oracle.forward_mxfp8_tokens(x[[0, 5]], ids[[0, 5]], w[[0, 5]], ex)
    np.testing.assert_allclose(ys, ymx[[0, 5]], rtol=1e-12, atol=1e-12)
