"""Pins for the oracle's number formats against independent sources:
torch's CPU float8_e4m3fn / bfloat16 casts (a separate library implementation),
hand-derived cases from the OCP FP8 format definition (tests/golden), and
closed-form tie constructions."""

import os

import numpy as np
import torch

from oracle.codec import (e4m3_decode, e4m3_encode, e4m3_round, bf16_round,
                          bf16_bits, bf16_decode)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_cases.txt")


def _torch_e4m3_codes(v32):
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_encode_all_bf16_patterns_match_torch_after_saturation():
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    finite = np.isfinite(v)
    sat = np.clip(v[finite], -448.0, 448.0)
    ours = e4m3_encode(v[finite].astype(np.float64))
    ref = _torch_e4m3_codes(sat)
    assert np.array_equal(ours, ref)
    # NaN inputs encode to a NaN code
    nan_in = np.isnan(v)
    assert np.all(np.isnan(e4m3_decode(e4m3_encode(v[nan_in].astype(np.float64)))))


def test_encode_random_fp32_match_torch():
    g = np.random.default_rng(123)
    v = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * 100,
        g.uniform(-2 ** -5, 2 ** -5, 200000).astype(np.float32),
        (g.standard_normal(50000) * 1e-3).astype(np.float32),
    ])
    ours = e4m3_encode(v.astype(np.float64))
    ref = _torch_e4m3_codes(np.clip(v, -448, 448))
    assert np.array_equal(ours, ref)


def test_encode_golden_cases():
    n = 0
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        expr, code = line.split()[:2]
        val = float(eval(expr, {"__builtins__": {}}))
        got = int(e4m3_encode(np.array([val]))[0])
        assert got == int(code, 16), (expr, hex(got), code)
        n += 1
    assert n >= 15


def test_round_is_idempotent_and_monotone():
    g = np.random.default_rng(5)
    v = np.sort(g.standard_normal(100000) * 50)
    r = e4m3_round(v)
    assert np.all(np.diff(r) >= 0)
    assert np.array_equal(e4m3_round(r), r)
    # every rounded value decodes from its code
    assert np.array_equal(e4m3_decode(e4m3_encode(v)), r)


def test_bf16_round_matches_torch_on_fp32():
    g = np.random.default_rng(7)
    v = np.concatenate([
        g.standard_normal(300000).astype(np.float32),
        (g.standard_normal(100000) * 1e30).astype(np.float32),
        (g.standard_normal(100000) * 1e-38).astype(np.float32),   # subnormal range
        np.array([3.3895314e38, 3.4e38, -3.4e38, 0.0, -0.0], dtype=np.float32),
    ])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = bf16_bits(v.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_round_fp64_ties_and_near_ties():
    # values exactly halfway between consecutive bf16 numbers go to the even one;
    # a hair above halfway goes up (a double-rounding path through fp32 would
    # get the second case wrong)
    lo = 1.0 + 2 ** -7          # odd mantissa (1 ulp above 1.0)
    assert bf16_round(np.array([1.0 + 2 ** -8]))[0] == 1.0              # tie -> even (1.0)
    assert bf16_round(np.array([lo + 2 ** -8]))[0] == 1.0 + 2 ** -6      # tie -> even (up)
    assert bf16_round(np.array([1.0 + 2 ** -8 + 2 ** -40]))[0] == lo     # above tie -> up
    assert bf16_round(np.array([1.0 + 2 ** -8 - 2 ** -40]))[0] == 1.0    # below tie -> down
    assert np.isinf(bf16_round(np.array([2.0 ** 128 * (1 - 2 ** -9)]))[0])
    assert bf16_round(np.array([-2.5]))[0] == -2.5


def test_bf16_decode_roundtrip():
    bits = np.arange(65536, dtype=np.uint16)
    v = bf16_decode(bits)
    finite = np.isfinite(v)
    assert np.array_equal(bf16_bits(v[finite]), bits[finite])
