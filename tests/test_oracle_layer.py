"""Pins for the oracle's layer stages: brute force on tiny inputs, closed forms,
exact-integer GEMM cases and invariants.  Each check is written so that a
plausible mistake in oracle.moe (a dropped term, a wrong index, a transposed
operand or scale) fails at least one of them."""

import math

import numpy as np
import pytest

from oracle import moe, dense
from oracle.codec import e4m3_decode, e4m3_encode, bf16_round
from workloads import CONFIGS, routing, activations, weights, bf16_to_f32

C, M = moe.LAYOUT_CONTIGUOUS, moe.LAYOUT_MASKED


# ------------------------------------------------------------------ layout
def brute_layout(topk_idx, E, layout, align_m=128, rows=None, capacity=None):
    """Python-loop layout: walk entries in flat order, hand out slots."""
    T, K = topk_idx.shape
    status = 0
    counts = [0] * E
    for t in range(T):
        for k in range(K):
            e = int(topk_idx[t, k])
            if e == -1:
                continue
            if e < 0 or e >= E:
                status |= 1
                continue
            counts[e] += 1
    offsets = [0]
    for e in range(E):
        if layout == C:
            offsets.append(offsets[-1] + ((counts[e] + align_m - 1) // align_m) * align_m)
        else:
            offsets.append((e + 1) * capacity)
    rows_total = rows if layout == C else E * capacity
    nxt = [0] * E
    slot_of = [[-1] * K for _ in range(T)]
    row_src = [-1] * rows_total
    row_exp = [-1] * rows_total
    for t in range(T):
        for k in range(K):
            e = int(topk_idx[t, k])
            if e < 0 or e >= E:
                continue
            r = nxt[e]
            nxt[e] += 1
            s = offsets[e] + r
            if (layout == C and s >= rows_total) or (layout == M and r >= capacity):
                status |= 2
                continue
            slot_of[t][k] = s
            row_src[s] = t
            row_exp[s] = e
    return counts, offsets, slot_of, row_src, row_exp, status


def _check_layout_vs_brute(idx, E, layout, **kw):
    L = moe.dispatch_layout(idx, E, layout, **kw)
    counts, offsets, slot_of, row_src, row_exp, status = brute_layout(idx, E, layout, **kw)
    assert list(L["counts"]) == counts
    assert list(L["offsets"]) == offsets
    assert L["slot_of"].tolist() == slot_of
    assert list(L["row_src"]) == row_src
    assert list(L["row_expert"]) == row_exp
    assert L["status"] == status
    return L


@pytest.mark.parametrize("align_m", [1, 16, 128])
def test_layout_tiny_vs_brute(align_m):
    cfg = CONFIGS[1]
    idx, _ = routing(cfg)
    _check_layout_vs_brute(idx, cfg.E, C, align_m=align_m, rows=cfg.T * cfg.K + cfg.E * align_m)


def test_layout_config2_slice_vs_brute():
    cfg = CONFIGS[2]
    idx, _ = routing(cfg)
    idx = idx[:300]
    _check_layout_vs_brute(idx, cfg.E, C, align_m=128, rows=300 * 4 + 4 * 128)
    _check_layout_vs_brute(idx, cfg.E, M, capacity=64)   # forces drops


def test_layout_bad_ids_and_overflow_vs_brute():
    g = np.random.default_rng(3)
    idx = g.integers(-3, 7, size=(50, 4)).astype(np.int32)
    L = _check_layout_vs_brute(idx, 5, C, align_m=4, rows=40)
    assert L["status"] == 3
    _check_layout_vs_brute(idx, 5, M, capacity=8)


def test_layout_invariants_config5():
    cfg = CONFIGS[5]
    idx, w = routing(cfg)
    L = moe.dispatch_layout(idx, cfg.E, M, capacity=cfg.capacity)
    so = L["slot_of"]
    valid = so >= 0
    assert L["status"] == 0
    assert L["counts"].sum() == (idx >= 0).sum() == valid.sum()
    s = so[valid]
    assert len(np.unique(s)) == len(s)                                      # injective
    assert np.array_equal(L["row_expert"][s], idx[valid])
    assert np.array_equal(L["row_src"][s], np.nonzero(valid)[0])
    # in-expert order increasing in flat index
    f = np.nonzero(valid.reshape(-1))[0]
    for e in range(cfg.E):
        fe = f[idx.reshape(-1)[f] == e]
        assert np.all(np.diff(so.reshape(-1)[fe]) == 1)
    # combine weights sum to each token's routed mass (1 for local picks)
    assert np.allclose(np.where(valid, w, 0).sum(1), 1.0, atol=1e-6)


# ------------------------------------------------------------------ quantise
def test_quantize_blocks_invariants():
    g = np.random.default_rng(11)
    v = g.standard_normal((8, 512)) * np.array([1e-3, 1.0, 30.0, 0.0])[:, None].repeat(2, 0)
    q, s = moe.quantize_blocks(v, 1)
    assert s.dtype == np.float32 and s.shape == (8, 4)
    dq = moe.dequantize_blocks(q, s, 1)
    for r in range(8):
        for b in range(4):
            blk = v[r, b * 128:(b + 1) * 128]
            codes = q[r, b * 128:(b + 1) * 128]
            if np.all(blk == 0):
                assert s[r, b] == 1.0 and np.all(e4m3_decode(codes) == 0)
                continue
            assert np.any((codes & 0x7F) == 0x7E)            # amax hits 448
            assert abs(float(s[r, b]) / (np.abs(blk).max() / 448.0) - 1) < 2 ** -23
            # error at most half a spacing of the code's binade times s
            err = np.abs(dq[r, b * 128:(b + 1) * 128] - blk)
            a = np.abs(blk / float(s[r, b]))
            _, ex = np.frexp(np.minimum(a, 448.0))
            half = np.ldexp(1.0, np.maximum(ex, -5) - 5) * float(s[r, b])
            # plus the fp32 rounding of v and of v / s (relative 2^-24 each)
            assert np.all(err <= half + np.abs(blk) * 2 ** -22)
    # 128x128 weight blocks: one scale per block
    w = g.standard_normal((256, 256)) * 0.02
    q, s = moe.quantize_blocks(w, 128)
    assert s.shape == (2, 2)
    for i in range(2):
        for j in range(2):
            blk = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert abs(float(s[i, j]) / (np.abs(blk).max() / 448.0) - 1) < 2 ** -23


# ------------------------------------------------------------------ GEMM
def _int_codes(g, shape, lim=4):
    """E4M3 codes of small integers |v| <= lim (exact in E4M3)."""
    vals = g.integers(-lim, lim + 1, size=shape).astype(np.float64)
    return e4m3_encode(vals), vals.astype(np.int64)


def test_gemm_exact_integers_vs_int64():
    g = np.random.default_rng(1)
    a, ai = _int_codes(g, (37, 384))
    w, wi = _int_codes(g, (256, 384))
    h = moe.gemm_rows(a, np.ones((37, 3), np.float32), w, np.ones((2, 3), np.float32))
    exact = (ai @ wi.T).astype(np.float64)      # exact integer sums; only the bf16 store rounds
    assert np.array_equal(h, bf16_round(exact))
    # sums that fit in 8 significant bits are reproduced exactly
    small = np.abs(exact) < 256
    assert np.array_equal(h[small], exact[small])


def test_gemm_power_of_two_block_scales():
    """Distinct power-of-two scales per (row, k-block) and (n-block, k-block):
    everything stays exact, so the result must equal the explicit per-block
    integer sum; a transposed or mis-indexed scale fails."""
    g = np.random.default_rng(2)
    Mr, N, K = 20, 256, 512
    a, ai = _int_codes(g, (Mr, K), 3)
    w, wi = _int_codes(g, (N, K), 3)
    sa = np.ldexp(1.0, g.integers(-4, 5, size=(Mr, K // 128))).astype(np.float32)
    sw = np.ldexp(1.0, g.integers(-4, 5, size=(N // 128, K // 128))).astype(np.float32)
    h = moe.gemm_rows(a, sa, w, sw)
    for m in range(Mr):
        for n in range(0, N, 7):
            tot = 0.0
            for kb in range(K // 128):
                blk = int(np.dot(ai[m, kb * 128:(kb + 1) * 128], wi[n, kb * 128:(kb + 1) * 128]))
                tot += blk * float(sa[m, kb]) * float(sw[n // 128, kb])
            assert h[m, n] == bf16_round(np.array([tot]))[0]


# ------------------------------------------------------------------ act
def test_silu_closed_forms():
    h = np.array([[0.0, 1.0, 50.0, -50.0, 2.0, 3.0, -1.5, 0.5]])
    v = moe.silu_mul(h)
    assert v[0, 0] == 0.0                                     # silu(0) = 0
    assert abs(v[0, 1] - 0.7310585786300049 * 3.0) < 1e-15    # sigmoid(1) = 0.7310585786...
    assert abs(v[0, 2] - 50.0 * (-1.5)) < 1e-12               # silu(g) -> g, g >> 0
    assert abs(v[0, 3]) < 1e-18                               # silu(g) -> 0, g << 0


def test_act_requant_block_structure():
    g = np.random.default_rng(4)
    h = bf16_round(g.standard_normal((5, 512)))
    q, s = moe.act_requant(h)
    assert q.shape == (5, 256) and s.shape == (5, 2)
    v = moe.silu_mul(h)
    q2, s2 = moe.quantize_blocks(v, 1)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # swapping gate and up changes the result (catches a gate/up mix-up)
    hs = np.concatenate([h[:, 256:], h[:, :256]], axis=1)
    assert not np.array_equal(moe.act_requant(hs)[0], q)


# ------------------------------------------------------------------ combine
def test_combine_closed_forms():
    cfg = CONFIGS[2]
    idx, w = routing(cfg)
    L = moe.dispatch_layout(idx, cfg.E, C, align_m=128, rows=4096)
    H = 16
    ones = {s: np.ones(H) for s in range(L["rows_total"])}
    toks = np.arange(200)
    out = moe.combine_rows(ones, L["slot_of"], w, toks)
    mass = [sum(float(w[t, k]) for k in range(cfg.K) if idx[t, k] >= 0) for t in toks]
    assert np.array_equal(out[:, 0], bf16_round(np.array(mass)))
    # single-row tokens recover their slot exactly from integer-coded y rows
    ident = {s: np.full(H, float(s)) for s in range(L["rows_total"])}
    unit_w = np.where(idx >= 0, 1.0, 0.0).astype(np.float32)
    one = [t for t in toks if (idx[t] >= 0).sum() == 1]
    out = moe.combine_rows(ident, L["slot_of"], unit_w, one)
    for i, t in enumerate(one):
        s = L["slot_of"][t][L["slot_of"][t] >= 0][0]
        assert out[i, 0] == bf16_round(np.array([float(s)]))[0]
    # a token with no valid row is zero
    so = L["slot_of"].copy()
    so[0] = -1
    assert np.all(moe.combine_rows(ones, so, w, [0]) == 0)


# ------------------------------------------------------------------ whole layer
def _tiny_inputs():
    cfg = CONFIGS[1]
    idx, w = routing(cfg)
    x, xs = moe.quantize_blocks(bf16_to_f32(activations(cfg)), 1)
    w13b, w2b = weights(cfg)
    w13 = np.empty(w13b.shape, np.uint8)
    s13 = np.empty((cfg.E, 2 * cfg.I // 128, cfg.H // 128), np.float32)
    w2 = np.empty(w2b.shape, np.uint8)
    s2 = np.empty((cfg.E, cfg.H // 128, cfg.I // 128), np.float32)
    for e in range(cfg.E):
        w13[e], s13[e] = moe.quantize_blocks(bf16_to_f32(w13b[e]), 128)
        w2[e], s2[e] = moe.quantize_blocks(bf16_to_f32(w2b[e]), 128)
    return cfg, idx, w, x, xs, w13, s13, w2, s2


def test_layer_tiny_vs_brute_force_dense():
    cfg, idx, w, x, xs, w13, s13, w2, s2 = _tiny_inputs()
    res = moe.layer(x, xs, idx, w, w13, s13, w2, s2, C, align_m=128, rows=1024)
    w13d = [dense.dequant_weight(w13[e], s13[e]) for e in range(cfg.E)]
    w2d = [dense.dequant_weight(w2[e], s2[e]) for e in range(cfg.E)]
    for t in range(cfg.T):
        ref = dense.token_forward(x[t], xs[t], list(idx[t]), list(w[t]), w13d, w2d)
        assert np.array_equal(res["out"][t], ref), t
    # the tiny layer is not degenerate
    assert np.abs(res["out"]).max() > 0


def test_layer_masked_equals_contiguous_rows():
    cfg, idx, w, x, xs, w13, s13, w2, s2 = _tiny_inputs()
    rc = moe.layer(x, xs, idx, w, w13, s13, w2, s2, C, align_m=16, rows=256)
    rm = moe.layer(x, xs, idx, w, w13, s13, w2, s2, M, capacity=64)
    assert np.array_equal(rc["out"], rm["out"])


def test_layer_token_subset_matches_full():
    cfg, idx, w, x, xs, w13, s13, w2, s2 = _tiny_inputs()
    full = moe.layer(x, xs, idx, w, w13, s13, w2, s2, C, align_m=128, rows=1024)
    toks = np.array([3, 17, 40, 63])
    sub = moe.layer(x, xs, idx, w, w13, s13, w2, s2, C, align_m=128, rows=1024, tokens=toks)
    assert np.array_equal(sub["out"], full["out"][toks])
