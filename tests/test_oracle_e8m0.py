"""Pins of the power-of-two ("packed") scale oracle (oracle/e8m0.py) against
closed forms, brute force and the independently pinned fp32-scale mode."""

import numpy as np

from oracle import e8m0, moe
from oracle.codec import e4m3_decode


def test_scale_exponent_closed_forms():
    # amax = 448 * 2^k  ->  amax / 448 is exactly 2^k  ->  e = k
    k = np.arange(-100, 100)
    amax = (np.float32(448.0) * np.ldexp(np.float32(1.0), k)).astype(np.float32)
    assert np.array_equal(e8m0.scale_exponents(amax), k)
    # one fp32 ulp above: the quotient rounds to 2^k (1 + 2^-23) -> e = k + 1
    up = np.nextafter(amax, np.float32(np.inf)).astype(np.float32)
    assert np.array_equal(e8m0.scale_exponents(up), k + 1)
    # one ulp below: the quotient rounds to 2^k (1 - 2^-24) -> e = k
    dn = np.nextafter(amax, np.float32(0)).astype(np.float32)
    assert np.array_equal(e8m0.scale_exponents(dn), k)
    # zero block -> scale 1; tiny and huge blocks stay inside E8M0
    assert e8m0.scale_exponents(np.float32(0.0)) == 0
    assert e8m0.scale_exponents(np.float32(1e-44)) == -127
    assert e8m0.scale_exponents(np.float32(3e38)) == 120


def test_scale_brackets_block_maximum():
    g = np.random.default_rng(1)
    amax = np.abs(g.standard_normal(20000) * np.exp(g.uniform(-60, 60, 20000))).astype(np.float32)
    e = e8m0.scale_exponents(amax)
    sf = (amax / np.float32(448)).astype(np.float64)
    assert np.all(np.ldexp(1.0, e) >= sf)
    assert np.all(np.ldexp(1.0, e - 1) < sf)


def test_codes_bounded_and_block_max_in_top_binade():
    g = np.random.default_rng(2)
    x = g.standard_normal((64, 1024)) * np.exp(g.uniform(-8, 8, (64, 1)))
    q, e = e8m0.quantize_blocks(x, 1)
    d = np.abs(e4m3_decode(q)).reshape(64, 8, 128)
    assert d.max() <= 448.0
    # amax / s lies in (224, 448]; E4M3 RNE keeps the block maximum >= 224
    assert np.all(d.max(axis=2) >= 224.0)


def test_equals_fp32_mode_when_amax_is_448_times_power_of_two():
    g = np.random.default_rng(3)
    R, C = 256, 512
    x = g.uniform(-1, 1, (R, C))
    k = g.integers(-20, 20, (R // 128, C // 128))
    blk = x.reshape(R // 128, 128, C // 128, 128)
    blk /= np.abs(blk).max(axis=(1, 3), keepdims=True)
    blk *= 448.0 * np.ldexp(1.0, k)[:, None, :, None]   # amax = 448 * 2^k exactly
    x = blk.reshape(R, C).astype(np.float32)
    q, e = e8m0.quantize_blocks(x, 128)
    q32, s32 = moe.quantize_blocks(x, 128)
    assert np.array_equal(e, k)
    assert np.array_equal(s32, e8m0.scales(e))
    assert np.array_equal(q, q32)


def test_codes_are_nearest_e4m3_brute_force():
    g = np.random.default_rng(4)
    x = (g.standard_normal((8, 256)) * np.exp(g.uniform(-5, 5, (8, 1)))).astype(np.float32)
    q, e = e8m0.quantize_blocks(x, 1)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = e4m3_decode(codes)
    for r in range(8):
        for c in range(256):
            t = np.ldexp(np.float64(x[r, c]), -int(e[r, c // 128]))
            dist = np.abs(vals - t)
            best = dist.min()
            cand = codes[dist == best]
            if len(cand) > 1:            # a tie: the even mantissa wins
                cand = cand[(cand & 1) == 0]
            vq = e4m3_decode(np.array([q[r, c]]))[0]
            assert vq in e4m3_decode(cand), (r, c, t, vq)


def test_pack_layout_fixture():
    # biased bytes 127, 128, 126, 132 | 254, 0, pad 127, pad 127 (little-endian)
    w = e8m0.pack(np.array([[0, 1, -1, 5, 127, -127]]))
    assert w.dtype == np.uint32
    assert [int(v) for v in w[0]] == [0x847E807F, 0x7F7F00FE]


def test_pack_roundtrip():
    g = np.random.default_rng(5)
    for nb in (1, 2, 4, 7, 56):
        e = g.integers(-127, 128, (3, 5, nb))
        w = e8m0.pack(e)
        assert w.shape == (3, 5, (nb + 3) // 4)
        assert np.array_equal(e8m0.unpack(w, nb), e)


def test_layer_requant_hook_uses_power_of_two_scales():
    """The chained oracle layer with the e8m0 quantiser: every S6 scale is a
    power of two and S6 codes decode to the values the scales produce."""
    g = np.random.default_rng(6)
    T, K, E, H, I = 24, 2, 3, 256, 128
    idx = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = np.full((T, K), 0.5, np.float32)
    x, xe = e8m0.quantize_blocks(g.standard_normal((T, H)), 1)
    w13, e13 = e8m0.quantize_blocks(g.standard_normal((E * 2 * I, H)) * 0.05, 128)
    w2, e2 = e8m0.quantize_blocks(g.standard_normal((E * H, I)) * 0.05, 128)
    res = moe.layer(x, e8m0.scales(xe), idx, w, w13.reshape(E, 2 * I, H),
                    e8m0.scales(e13).reshape(E, 2 * I // 128, H // 128), w2.reshape(E, H, I),
                    e8m0.scales(e2).reshape(E, H // 128, I // 128), moe.LAYOUT_CONTIGUOUS,
                    align_m=1, rows=T * K, requant=e8m0.act_requant)
    s = res["q2_scale"].astype(np.float64)
    m, _ = np.frexp(s)
    assert np.all(m == 0.5)
    q_ref, e_ref = e8m0.quantize_blocks(moe.silu_mul(res["h"]), 1)
    assert np.array_equal(res["q2"], q_ref)
