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


# ------------------------------------------------------------------ R4 against torch
def _torch_fp32_quantiser(v, block_rows):
    """An independent fp32 block quantiser built from torch CPU primitives:
    amax and amax / 448 in fp32, unit scale for an all-zero block, then
    (v / s) saturated to +-448 and cast by torch's float8_e4m3fn conversion
    (round to nearest even).  Shares nothing with oracle.codec."""
    import torch
    x = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    R, Cn = x.shape
    blk = x.reshape(R // block_rows, block_rows, Cn // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    s = amax / torch.tensor(448.0, dtype=torch.float32)
    s = torch.where(amax == 0, torch.ones_like(s), s)
    quot = blk / s[:, None, :, None]
    q = quot.clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(R, Cn).numpy(), s.numpy()


def _tie_heavy_bf16(g, rows):
    """bf16 rows whose block scale is an exact power of two (each block holds
    +-448 * 2^k) and whose other values sit exactly on E4M3 rounding
    midpoints (5 significant bits, so bf16-exact), or one bf16 ulp beside
    them: every code is decided by the tie rule or by one ulp."""
    from oracle.codec import e4m3_decode as dec
    vals = np.unique(np.abs(dec(np.arange(0x7F))))
    mids = (vals[:-1] + vals[1:]) / 2.0
    out = np.empty((rows, 256), np.float32)
    for r in range(rows):
        for b in range(2):
            k = int(g.integers(-20, 20))
            m = g.choice(mids, size=128) * np.where(g.random(128) < 0.5, -1.0, 1.0)
            m = m.astype(np.float32)
            nudge = g.integers(-1, 2, size=128).astype(np.int32)   # -1, 0, +1 ulp
            bits = m.view(np.uint32).astype(np.int64) + (nudge << 16)
            m = (bits.astype(np.uint32)).view(np.float32)
            m[int(g.integers(0, 128))] = 448.0 * (1 if g.random() < 0.5 else -1)
            out[r, b * 128:(b + 1) * 128] = np.ldexp(m, k)
    return out


@pytest.mark.parametrize("block_rows", [1, 128])
def test_quantize_blocks_r4_matches_torch_fp32_quantiser(block_rows):
    """R4 (codes decided from the correctly rounded fp32 quotient v / s) is
    the conventional fp32 quantiser; torch's CPU ops compute the same thing
    independently.  Random bf16 blocks over a wide dynamic range, tie-heavy
    blocks, zero blocks and subnormal-range blocks: codes and scales bit-exact."""
    g = np.random.default_rng(20 + block_rows)
    R = 256 if block_rows == 1 else 384
    v = (g.standard_normal((R, 512)) *
         np.exp(g.uniform(-30, 30, (R // block_rows, 1))).repeat(block_rows, 0))
    v = bf16_to_f32(_bf16_bits(v))
    v[:block_rows, :128] = 0.0                                     # zero block
    v[block_rows:2 * block_rows, 128:256] *= 2.0 ** -120           # tiny scales
    q, s = moe.quantize_blocks(v, block_rows)
    tq, ts = _torch_fp32_quantiser(v, block_rows)
    assert np.array_equal(s, ts)
    assert np.array_equal(q, tq)
    if block_rows == 1:
        t = _tie_heavy_bf16(g, 64)
        q, s = moe.quantize_blocks(t, 1)
        tq, ts = _torch_fp32_quantiser(t, 1)
        assert np.array_equal(s, ts) and np.array_equal(q, tq)
        # the blocks really are tie-heavy: about a third of the quotients
        # lie exactly on a rounding midpoint
        from oracle.codec import e4m3_decode as dec
        vals = np.unique(np.abs(dec(np.arange(0x7F))))
        mids = set(((vals[:-1] + vals[1:]) / 2.0).tolist())
        quot = np.abs(t / np.repeat(s, 128, axis=1)).astype(np.float64).ravel()
        assert np.mean([x in mids for x in quot]) > 0.25


def _bf16_bits(a):
    import torch
    return (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------------ permute / segments
def _distinct_rows(g, T, H):
    """Source rows that differ from each other in every 16-byte piece (the
    token id is written into each piece), so any row or piece moved to the
    wrong slot is caught."""
    x = g.integers(0, 256, size=(T, H), dtype=np.uint8)
    for p in range(0, H, 16):
        x[:, p] = np.arange(T) & 0xFF
        x[:, p + 1] = (np.arange(T) >> 8) & 0xFF
    xs = g.standard_normal((T, H // 128)).astype(np.float32)
    xs[:, 0] = np.arange(T, dtype=np.float32)
    return x, xs


@pytest.mark.parametrize("case", ["contig", "contig_overflow", "masked_drops", "bad_ids"])
def test_permute_vs_brute(case):
    """moe.permute against a walk over (t, k) in the Python-loop layout:
    every routed, kept entry's slot holds its token's row and scales byte for
    byte; every other slot is zero and reported unfilled."""
    g = np.random.default_rng(7)
    T, K, E, H = 90, 4, 5, 384
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        n = int(g.integers(0, K + 1))
        idx[t, g.permutation(K)[:n]] = g.permutation(E)[:n]
    kw = dict(align_m=8, rows=T * K + E * 8)
    layout = C
    if case == "contig_overflow":
        kw = dict(align_m=8, rows=100)
    elif case == "masked_drops":
        layout, kw = M, dict(capacity=12)
    elif case == "bad_ids":
        idx[g.random((T, K)) < 0.1] = 9
        idx[g.random((T, K)) < 0.05] = -4
    x, xs = _distinct_rows(g, T, H)
    L = moe.dispatch_layout(idx, E, layout, **kw)
    a, sa, filled = moe.permute(x, xs, L)
    _, _, slot_of, _, _, _ = brute_layout(idx, E, layout, **kw)
    rows_total = L["rows_total"]
    want_a = np.zeros((rows_total, H), np.uint8)
    want_s = np.zeros((rows_total, H // 128), np.float32)
    want_f = np.zeros(rows_total, bool)
    for t in range(T):
        for k in range(K):
            s = slot_of[t][k]
            if s >= 0:
                assert not want_f[s]            # a slot is filled once
                want_a[s], want_s[s], want_f[s] = x[t], xs[t], True
    assert np.array_equal(filled, want_f)
    assert np.array_equal(a, want_a)
    assert np.array_equal(sa, want_s)
    assert want_f.sum() == sum(s >= 0 for row in slot_of for s in row)


@pytest.mark.parametrize("case", ["contig", "contig_overflow", "masked_drops", "empty_experts"])
def test_expert_segments_vs_brute(case):
    """moe.expert_segments against the slots the Python-loop layout actually
    filled for each expert: a segment is exactly [first, last + 1) of the
    expert's filled slots, it starts at the expert's offset (clipped to the
    buffer), and an expert with no kept row has an empty segment there."""
    g = np.random.default_rng(8)
    T, K, E = 120, 3, 6
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        n = int(g.integers(1, K + 1))
        idx[t, g.permutation(K)[:n]] = g.permutation(E)[:n]
    layout, kw = C, dict(align_m=16, rows=T * K + E * 16)
    if case == "contig_overflow":
        kw = dict(align_m=16, rows=150)
    elif case == "masked_drops":
        layout, kw = M, dict(capacity=20)
    elif case == "empty_experts":
        idx[(idx == 1) | (idx == 4)] = -1
    L = moe.dispatch_layout(idx, E, layout, **kw)
    counts, offsets, slot_of, row_src, row_exp, _ = brute_layout(idx, E, layout, **kw)
    rows_total = kw["rows"] if layout == C else E * kw["capacity"]
    segs = moe.expert_segments(L)
    assert len(segs) == E
    for e in range(E):
        mine = [s for s in range(rows_total) if row_exp[s] == e]
        s0, s1 = segs[e]
        if mine:
            assert (s0, s1) == (min(mine), max(mine) + 1)
            assert mine == list(range(s0, s1))      # contiguous, no gaps
            assert s0 == offsets[e]
        else:
            assert s0 == s1 == min(offsets[e], rows_total)
    if case == "empty_experts":
        assert segs[1][0] == segs[1][1] and segs[4][0] == segs[4][1]
