"""Pins for the oracle's FP8 (E4M3FN) per-channel weight quantisation."""
import numpy as np
import pytest
import torch

import oracle


def test_e4m3_table_matches_library():
    # every code, against torch's float8_e4m3fn (an independent library decoder)
    pats = torch.arange(256, dtype=torch.uint8)
    ref = pats.view(torch.float8_e4m3fn).double().numpy()
    got = oracle.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(ref[~np.isnan(ref)], got[~np.isnan(got)])
    assert np.nanmax(got) == 448.0 and oracle.e4m3_decode([0x7E])[0] == 448.0


def test_e4m3_encode_matches_library_rounding():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * 30, rng.uniform(-448, 448, 50000),
                        rng.standard_normal(20000) * 1e-3, [0.0, -0.0, 448.0, -448.0, 1e-9]]
                       ).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x)
    assert np.array_equal(ref, got)


def test_e4m3_encode_ties_go_to_even():
    # midpoints between neighbouring codes round to the even mantissa
    for lo_code in (0x38, 0x39, 0x40, 0x01, 0x77):
        lo = oracle.e4m3_decode([lo_code])[0]
        hi = oracle.e4m3_decode([lo_code + 1])[0]
        mid = np.float32((lo + hi) / 2)
        if float(mid) != (lo + hi) / 2:
            continue
        want = lo_code if lo_code % 2 == 0 else lo_code + 1
        assert oracle.e4m3_encode(np.array([mid]))[0] == want


def test_per_channel_scales_and_roundtrip():
    rng = np.random.default_rng(1)
    w = (0.02 * rng.standard_normal((3, 64, 96))).astype(np.float32)
    w[1, 5] = 0.0
    q, s = oracle.quantize_fp8_per_channel(w)
    assert q.shape == w.shape and q.dtype == np.uint8 and s.shape == (3, 64)
    # the largest element of each nonzero row maps to exactly +-448
    d = oracle.e4m3_decode(q)
    rows = np.abs(w).max(-1) > 0
    assert np.all(np.abs(d).max(-1)[rows] == 448.0)
    assert s[1, 5] == 1.0 and np.all(q[1, 5] == 0)
    # dequantised weights within the E4M3 half-step (2^-4 relative) of the input
    deq = oracle.dequantize_fp8(q, s)
    err = np.abs(deq - w)
    tol = np.maximum(np.abs(w) * 2.0 ** -4, s[..., None] * 2.0 ** -9 / 2 * 1.0001)
    assert np.all(err <= tol)


def test_representable_weights_roundtrip_exactly():
    # weights that are scale * (an E4M3 value) with the row maximum 448 * scale
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 0x7E, size=(8, 32)).astype(np.uint8)
    codes[:, 0] = 0x7E                                   # +448 sets the scale
    sign = rng.integers(0, 2, size=codes.shape).astype(np.uint8) << 7
    codes[:, 1:] |= sign[:, 1:]
    scale = np.float32(2.0 ** -12)
    w = (oracle.e4m3_decode(codes) * float(scale)).astype(np.float32)
    q, s = oracle.quantize_fp8_per_channel(w)
    assert np.all(s == scale)
    assert np.array_equal(oracle.e4m3_decode(q), oracle.e4m3_decode(codes))
