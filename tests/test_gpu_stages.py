"""Stage-isolated GPU parity: each C-ABI call on inputs produced by the CPU
oracle (or drawn by the generator), compared with the oracle's stage.

Acceptance: integer / byte work bit-exact; FP8 codes >= 99.9% agreement
(decoded values); bf16 outputs relative L2 <= 2e-3 and max |err| <= 0.02 *
max|ref|.  The full-size configurations run in the same launch configuration
as the benchmark and are checked on sampled rows / tokens.
"""

import numpy as np
import pytest
import torch

import fp8_routed_expert_amd as fre
from oracle import moe
from oracle.codec import e4m3_encode, e4m3_decode, bf16_decode
from tests.gpu_util import (dev, host, bf16_vals, check_close, code_agreement, log)
from tests.inputs import layer_inputs, rows_for
from workloads import CONFIGS

pytestmark = pytest.mark.gpu

ALL = [1, 2, 3, 4, 5]


def _layer_for(cfg, rows):
    # gather=False: the dispatch also copies the rows (the permute under test)
    return fre.MoELayer(cfg.E, cfg.H, cfg.I, cfg.T, cfg.K, cfg.layout, rows,
                        align_m=cfg.align_m, gather=False)


def _oracle_layout(cfg, idx, rows):
    if cfg.layout == moe.LAYOUT_MASKED:
        return moe.dispatch_layout(idx, cfg.E, cfg.layout, capacity=rows)
    return moe.dispatch_layout(idx, cfg.E, cfg.layout, align_m=cfg.align_m, rows=rows)


# --------------------------------------------------------------- quantiser
def _blocks_with_unit_scale(vals):
    """Rows of 128 whose first element is 448 so every block scale is 1."""
    per = 127
    n = -(-len(vals) // per)
    pad = np.zeros(n * per, dtype=vals.dtype)
    pad[:len(vals)] = vals
    blk = np.concatenate([np.full((n, 1), 448.0, dtype=vals.dtype), pad.reshape(n, per)], 1)
    return blk


def _assert_codes_equal(got, ref, x):
    bad = np.nonzero(got != ref)
    if len(bad[0]):
        ex = [(float(x[i, j]), hex(int(got[i, j])), hex(int(ref[i, j])))
              for i, j in list(zip(*bad))[:24]]
        raise AssertionError(f"{len(bad[0])} codes differ (value, device, oracle): {ex}")


def test_quantize_codec_all_bf16_in_range(gpu):
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    x = _blocks_with_unit_scale(v)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)      # exact: all values are bf16
    q = torch.empty(x.shape, dtype=torch.uint8, device=gpu)
    s = torch.empty(x.shape[0], 1, dtype=torch.float32, device=gpu)
    fre.moe_quantize_fp8(dev(xb), 1, q, s)
    torch.cuda.synchronize()
    assert np.all(host(s) == 1.0)
    ref = e4m3_encode(x.astype(np.float64))
    got = host(q)
    _assert_codes_equal(got, ref, x)


def test_quantize_codec_fp32_ties(gpu):
    # every E4M3 value, the midpoints between neighbours (ties), and values
    # one fp32 ulp either side of each midpoint
    pos = np.unique(np.abs(e4m3_decode(np.arange(256, dtype=np.uint8))))
    pos = pos[np.isfinite(pos)]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    g = np.random.default_rng(0)
    rnd = (g.standard_normal(100000) * 60).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 448]
    v = np.concatenate([pos, mids, up, dn, -pos, -mids, -up, -dn, rnd]).astype(np.float32)
    x = _blocks_with_unit_scale(v)
    q = torch.empty(x.shape, dtype=torch.uint8, device=gpu)
    s = torch.empty(x.shape[0], 1, dtype=torch.float32, device=gpu)
    fre.moe_quantize_fp8(dev(x), 1, q, s)
    torch.cuda.synchronize()
    ref = e4m3_encode(x.astype(np.float64))
    _assert_codes_equal(host(q), ref, x)


@pytest.mark.parametrize("block_rows", [1, 128])
def test_quantize_blocks_vs_oracle(gpu, block_rows):
    g = np.random.default_rng(block_rows)
    x = (g.standard_normal((512, 1024)) * np.exp(g.uniform(-6, 6, (512, 1)))).astype(np.float32)
    x[3, :128] = 0.0                                   # an all-zero block -> scale 1
    xb = torch.from_numpy(x).to(torch.bfloat16)
    xf = xb.to(torch.float64).numpy()
    q = torch.empty(x.shape, dtype=torch.uint8, device=gpu)
    s = torch.empty(512 // block_rows, 8, dtype=torch.float32, device=gpu)
    fre.moe_quantize_fp8(xb.cuda(), block_rows, q, s)
    torch.cuda.synchronize()
    rq, rs = moe.quantize_blocks(xf, block_rows)
    assert np.array_equal(host(s), rs)                 # amax/448 of bf16: exact
    code_agreement(host(q), rq, f"quantize {block_rows}x128", minimum=0.9999)


# --------------------------------------------------------------- layout
def _check_layout(cfg, idx, x, xs, rows, layer=None, align_m=None):
    layer = layer or _layer_for(cfg, rows)
    if align_m is not None:
        layer.align_m = align_m
    layer.status.zero_()
    layer.dispatch(dev(idx), dev(x), dev(xs))
    torch.cuda.synchronize()
    am = align_m if align_m is not None else cfg.align_m
    if cfg.layout == moe.LAYOUT_MASKED:
        L = moe.dispatch_layout(idx, cfg.E, cfg.layout, capacity=rows)
    else:
        L = moe.dispatch_layout(idx, cfg.E, cfg.layout, align_m=am, rows=rows)
    assert np.array_equal(host(layer.counts), L["counts"])
    assert np.array_equal(host(layer.offsets), L["offsets"])
    assert np.array_equal(host(layer.slot_of), L["slot_of"])
    assert np.array_equal(host(layer.row_src), L["row_src"])
    assert np.array_equal(host(layer.row_expert), L["row_expert"])
    assert int(host(layer.status)[0]) == L["status"]
    a_ref, sa_ref, filled = moe.permute(x, xs, L)
    a = host(layer.a)
    assert np.array_equal(a[filled], a_ref[filled])
    sa = host(layer.a_scale).T
    assert np.array_equal(sa[filled], sa_ref[filled])
    return L


@pytest.mark.parametrize("cid", ALL)
def test_layout_parity(gpu, cid):
    inp = layer_inputs(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    log(f"layout config {cid}: T={cfg.T} K={cfg.K} E={cfg.E} rows={rows}")
    _check_layout(cfg, inp["idx"], inp["x"], inp["xs"], rows)


@pytest.mark.parametrize("align_m", [1, 16, 64])
def test_layout_alignment_variants(gpu, align_m):
    inp = layer_inputs(1)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"]) + cfg.E * align_m
    _check_layout(cfg, inp["idx"], inp["x"], inp["xs"], rows, align_m=align_m)


def test_layout_overflow_and_bad_ids(gpu):
    inp = layer_inputs(1)
    cfg = inp["cfg"]
    idx = inp["idx"].copy()
    idx[5, 0] = 9          # bad id -> skipped, bit 0
    idx[7, 1] = -3         # bad id
    idx[9, 0] = -1         # not routed: fine
    # contiguous buffer too small: tail rows dropped in stable order, bit 1
    L = _check_layout(cfg, idx, inp["x"], inp["xs"], 150)
    assert L["status"] == 3
    # masked with a small capacity
    from dataclasses import replace
    mcfg = replace(cfg, layout=moe.LAYOUT_MASKED, capacity=20)
    L = _check_layout(mcfg, idx, inp["x"], inp["xs"], 20)
    assert L["status"] == 3


def test_layout_large_expert_count(gpu):
    """E = 300 experts (key needs 9 ballot bits), T*K spans several chunks."""
    from dataclasses import replace
    g = np.random.default_rng(9)
    T, K, E = 3000, 8, 300
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        n = g.integers(1, K + 1)
        idx[t, g.permutation(K)[:n]] = g.choice(E, size=n, replace=False)
    cfg = replace(CONFIGS[1], E=E, T=T, K=K)
    x = g.integers(0, 256, (T, cfg.H), dtype=np.uint8)
    x[(x & 0x7F) == 0x7F] = 0
    xs = g.uniform(0.5, 2, (T, cfg.H // 128)).astype(np.float32)
    rows = int((idx >= 0).sum()) + E * 127
    _check_layout(cfg, idx, x, xs, rows)


def _random_routing(g, T, K, E, fill=1.0):
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        if g.uniform() > fill:
            continue
        n = int(g.integers(1, min(K, E) + 1))
        idx[t, g.permutation(K)[:n]] = g.choice(E, size=n, replace=False)
    return idx


# (T, K, E, H, layout, rows or capacity): empty input into a non-empty
# buffer, a single expert, the maximum expert count (one scan lane per
# expert, the masked end offset), rows whose 16-byte chunks split unevenly
# into permute pieces (H = 4224: 264 chunks, two pieces of 132), and a
# masked capacity that overflows.
EDGE_LAYOUTS = [
    (0, 8, 9, 256, moe.LAYOUT_CONTIGUOUS, 300),
    (0, 8, 9, 256, moe.LAYOUT_MASKED, 4),
    (50, 4, 1, 128, moe.LAYOUT_CONTIGUOUS, 50 * 4 + 127),
    (700, 8, 1024, 4224, moe.LAYOUT_MASKED, 4),
    (700, 8, 1024, 4224, moe.LAYOUT_CONTIGUOUS, None),
    (2500, 3, 7, 4224, moe.LAYOUT_CONTIGUOUS, None),
    (2500, 6, 33, 384, moe.LAYOUT_MASKED, 200),
]


@pytest.mark.parametrize("case", EDGE_LAYOUTS, ids=lambda c: f"T{c[0]}K{c[1]}E{c[2]}H{c[3]}L{c[4]}")
def test_layout_edge_shapes(gpu, case):
    from dataclasses import replace
    T, K, E, H, layout, rows = case
    g = np.random.default_rng(T * 131 + E)
    idx = _random_routing(g, T, K, E, fill=0.9)
    if rows is None:
        rows = int((idx >= 0).sum()) + E * 127
    cfg = replace(CONFIGS[1], E=E, H=H, T=T, K=K, layout=layout,
                  capacity=rows if layout == moe.LAYOUT_MASKED else 0)
    x = g.integers(0, 256, (T, H), dtype=np.uint8)
    x[(x & 0x7F) == 0x7F] = 0
    xs = g.uniform(0.5, 2, (T, H // 128)).astype(np.float32)
    log(f"layout edge: T={T} K={K} E={E} H={H} layout={layout} rows={rows}")
    _check_layout(cfg, idx, x, xs, rows)


# --------------------------------------------------------------- GEMM
def _run_gemm(a, sa_rows, w, sw, offsets, counts, rows_total):
    """Upload, run moe_grouped_gemm_fp8, return bf16 bits [rows_total, N]."""
    E, N, K = w.shape
    c = torch.zeros(rows_total, N, dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    fre.moe_grouped_gemm_fp8(dev(a), dev(np.ascontiguousarray(sa_rows.T)), dev(w), dev(sw),
                             dev(offsets.astype(np.int32)), dev(counts.astype(np.int32)),
                             c, st)
    torch.cuda.synchronize()
    return host(c)


@pytest.mark.parametrize("tile_rows,tail", [(64, 3), (128, 240)])
def test_gemm_exact_integers_pow2_scales(gpu, tile_rows, tail):
    """Small-integer codes and power-of-two scales keep every sum exact, so
    the device result must equal the oracle's bit for bit: with codes in
    [-4, 4] and scales 2^[-2, 2] every partial sum is a multiple of 2^-4
    below 2^17, exact in fp32 in any summation order.  Segments are
    unaligned, one expert is empty, and tiles straddle segment ends.  The
    rows after the last segment decide the tile height (at most 128 buffer
    rows per expert: 64-row tiles; more: 128)."""
    g = np.random.default_rng(21)
    E, N, K = 4, 384, 512
    counts = np.array([37, 0, 200, 129])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    rows_total = int(offsets[-1]) + tail
    assert fre.moe_gemm_tile_rows(rows_total, N, K, E) == tile_rows
    a = e4m3_encode(g.integers(-4, 5, (rows_total, K)).astype(np.float64))
    w = e4m3_encode(g.integers(-4, 5, (E, N, K)).astype(np.float64))
    sa = np.ldexp(1.0, g.integers(-2, 3, (rows_total, K // 128))).astype(np.float32)
    sw = np.ldexp(1.0, g.integers(-2, 3, (E, N // 128, K // 128))).astype(np.float32)
    got = _run_gemm(a, sa, w, sw, offsets, counts, rows_total)
    for e in range(E):
        s, en = offsets[e], offsets[e] + counts[e]
        if en > s:
            ref = moe.gemm_rows(a[s:en], sa[s:en], w[e], sw[e])
            assert np.array_equal(bf16_decode(got[s:en]), ref), e


CORRUPT_TABLES = [
    ("decreasing", [0, 100, 90, 220], [100, 50, 70]),      # expert 2 starts inside expert 1
    ("negative_count", [0, 100, 150, 220], [100, -5, 70]),
    ("negative_start", [-64, 100, 150, 220], [100, 50, 70]),
]


@pytest.mark.parametrize("name,offs,cnts", CORRUPT_TABLES, ids=[c[0] for c in CORRUPT_TABLES])
def test_corrupt_segment_table_flagged(gpu, name, offs, cnts):
    """A segment table that does not describe segments sets
    MOE_ERR_BAD_INDEX in the gate/up GEMM, the activation and the fused
    call; rows of segments the table still describes correctly come out
    exactly as with the good table, and nothing outside the buffer is
    touched (every row index is clipped)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    E, I, H, rows = 3, 128, 256, 256
    good_o = np.array([0, 100, 150, 220], np.int32)
    good_c = np.array([100, 50, 70], np.int32)
    a = torch.randint(0, 0x7E, (rows, H), dtype=torch.uint8, device="cuda", generator=g)
    sa = torch.rand(H // 128, rows, device="cuda", generator=g) + 0.5
    w = torch.randint(0, 0x7E, (E, 2 * I, H), dtype=torch.uint8, device="cuda", generator=g)
    sw = torch.rand(E, 2 * I // 128, H // 128, device="cuda", generator=g) * 1e-3

    def run(o, c):
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        od, cd = dev(np.array(o, np.int32)), dev(np.array(c, np.int32))
        h = torch.zeros(rows, 2 * I, dtype=torch.bfloat16, device="cuda")
        q = torch.zeros(rows, I, dtype=torch.uint8, device="cuda")
        qs = torch.zeros(I // 128, rows, dtype=torch.float32, device="cuda")
        qf, qfs = q.clone(), qs.clone()
        fre.moe_grouped_gemm_fp8(a, sa, w, sw, od, cd, h, st)
        torch.cuda.synchronize()
        st_gemm = int(host(st)[0])
        st.zero_()
        fre.moe_act_requant(h, od, cd, q, qs, st)
        torch.cuda.synchronize()
        st_act = int(host(st)[0])
        st.zero_()
        fre.moe_gate_up_act_fp8(a, sa, w, sw, od, cd, qf, qfs, st)
        torch.cuda.synchronize()
        st_fused = int(host(st)[0])
        return (st_gemm, st_act, st_fused), host(h), host(q), host(qs), host(qf), host(qfs)

    sg, h0, q0, qs0, qf0, qfs0 = run(good_o, good_c)
    assert sg == (0, 0, 0)
    sb, h1, q1, qs1, qf1, qfs1 = run(offs, cnts)
    assert all(v == fre.ERR_BAD_INDEX for v in sb), sb
    # rows described identically by both tables and written by no other
    # segment: expert 0's (in "decreasing", expert 2's segment [90, 160)
    # overlaps its last ten rows), or expert 1's when expert 0's start is bad
    keep = {"decreasing": slice(0, 90), "negative_count": slice(0, 100),
            "negative_start": slice(100, 150)}[name]
    assert np.array_equal(h1[keep], h0[keep])
    assert np.array_equal(q1[keep], q0[keep]) and np.array_equal(qs1[:, keep], qs0[:, keep])
    assert np.array_equal(qf1[keep], qf0[keep]) and np.array_equal(qfs1[:, keep], qfs0[:, keep])


def test_gemm_exact_many_experts(gpu):
    """More experts than one wave has lanes (the tile lookup then takes
    several passes of 64 experts): 150 experts, a third of them empty, the
    rest with 1..40 rows in unaligned segments; exact small-integer data as
    above, so every valid row must equal the oracle bit for bit."""
    g = np.random.default_rng(23)
    E, N, K = 150, 256, 256
    counts = g.integers(1, 41, E)
    counts[g.choice(E, E // 3, replace=False)] = 0
    offsets = np.concatenate([[0], np.cumsum(counts)])
    rows_total = int(offsets[-1]) + 2
    a = e4m3_encode(g.integers(-4, 5, (rows_total, K)).astype(np.float64))
    w = e4m3_encode(g.integers(-4, 5, (E, N, K)).astype(np.float64))
    sa = np.ldexp(1.0, g.integers(-2, 3, (rows_total, K // 128))).astype(np.float32)
    sw = np.ldexp(1.0, g.integers(-2, 3, (E, N // 128, K // 128))).astype(np.float32)
    got = _run_gemm(a, sa, w, sw, offsets, counts, rows_total)
    for e in range(E):
        s, en = offsets[e], offsets[e] + counts[e]
        if en > s:
            ref = moe.gemm_rows(a[s:en], sa[s:en], w[e], sw[e])
            assert np.array_equal(bf16_decode(got[s:en]), ref), e


def _sample_rows(L, n_per_expert=6, seed=0):
    g = np.random.default_rng(seed)
    rows = []
    for s, en in moe.expert_segments(L):
        if en <= s:
            continue
        cand = {s, en - 1, min(s + 127, en - 1), min(s + 128, en - 1)}
        cand |= set(g.integers(s, en, size=n_per_expert).tolist())
        rows += sorted(cand)
    return np.array(sorted(set(rows)))


@pytest.mark.parametrize("cid", ALL)
def test_gemm1_parity(gpu, cid):
    inp = layer_inputs(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    L = _oracle_layout(cfg, inp["idx"], rows)
    a, sa, filled = moe.permute(inp["x"], inp["xs"], L)
    got = _run_gemm(a, sa, inp["w13"], inp["s13"], L["offsets"], L["counts"], L["rows_total"])
    rs = _sample_rows(L)
    ex = L["row_expert"][rs]
    ref = np.zeros((len(rs), 2 * cfg.I))
    for e in np.unique(ex):
        sel = ex == e
        ref[sel] = moe.gemm_rows(a[rs[sel]], sa[rs[sel]], inp["w13"][e], inp["s13"][e])
    g = bf16_decode(got[rs])
    check_close(g, ref, f"gemm1 config {cid} ({len(rs)} rows)")
    log(f"gemm1 config {cid}: exact bf16 fraction {(g == ref).mean():.5f}")


@pytest.mark.parametrize("cid", ALL)
def test_gemm2_parity(gpu, cid):
    inp = layer_inputs(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    L = _oracle_layout(cfg, inp["idx"], rows)
    R = L["rows_total"]
    rs = _sample_rows(L, seed=1)
    # synthetic down-projection input: oracle-quantised N(0, 1) rows on the
    # sampled rows, zero codes elsewhere
    g = np.random.default_rng(cid)
    q2 = np.zeros((R, cfg.I), np.uint8)
    q2s = np.ones((R, cfg.I // 128), np.float32)
    vals = g.standard_normal((len(rs), cfg.I)) * np.exp(g.uniform(-3, 3, (len(rs), 1)))
    q2[rs], q2s[rs] = moe.quantize_blocks(vals, 1)
    got = _run_gemm(q2, q2s, inp["w2"], inp["s2"], L["offsets"], L["counts"], R)
    ex = L["row_expert"][rs]
    ref = np.zeros((len(rs), cfg.H))
    for e in np.unique(ex):
        sel = ex == e
        ref[sel] = moe.gemm_rows(q2[rs[sel]], q2s[rs[sel]], inp["w2"][e], inp["s2"][e])
    check_close(bf16_decode(got[rs]), ref, f"gemm2 config {cid} ({len(rs)} rows)")


# --------------------------------------------------------------- act
@pytest.mark.parametrize("cid", ALL)
def test_act_requant_parity(gpu, cid):
    inp = layer_inputs(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    L = _oracle_layout(cfg, inp["idx"], rows)
    R = L["rows_total"]
    rs = _sample_rows(L, n_per_expert=40, seed=2)
    g = np.random.default_rng(100 + cid)
    h = np.zeros((R, 2 * cfg.I), np.uint16)
    vals = (g.standard_normal((len(rs), 2 * cfg.I)) * 2.0).astype(np.float32)
    vals[0, :128] = 0.0                                 # zero gate block -> scale 1
    hb = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    h[rs] = hb
    q = torch.zeros(R, cfg.I, dtype=torch.uint8, device=gpu)
    qs = torch.zeros(cfg.I // 128, R, dtype=torch.float32, device=gpu)
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    fre.moe_act_requant(dev(h), dev(L["offsets"].astype(np.int32)),
                        dev(L["counts"].astype(np.int32)), q, qs, st)
    torch.cuda.synchronize()
    rq, rqs = moe.act_requant(bf16_decode(hb))
    code_agreement(host(q)[rs], rq, f"act codes config {cid}")
    gs = host(qs).T[rs]
    rel = np.abs(gs.astype(np.float64) / rqs - 1.0)
    log(f"act scales config {cid}: max rel diff {rel.max():.3e}")
    assert rel.max() <= 1e-5


# --------------------------------------------------------------- combine
@pytest.mark.parametrize("cid", ALL)
def test_combine_parity(gpu, cid):
    inp = layer_inputs(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    L = _oracle_layout(cfg, inp["idx"], rows)
    R = L["rows_total"]
    g = np.random.default_rng(200 + cid)
    n_tok = min(cfg.T, 256)
    toks = np.sort(g.choice(cfg.T, size=n_tok, replace=False))
    so = L["slot_of"]
    slots = np.unique(so[toks][so[toks] >= 0])
    vals = (g.standard_normal((len(slots), cfg.H))).astype(np.float32)
    yb = torch.from_numpy(vals).to(torch.bfloat16)
    y = torch.zeros(R, cfg.H, dtype=torch.bfloat16, device=gpu)
    y[torch.from_numpy(slots).cuda()] = yb.cuda()
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=gpu)
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    fre.moe_combine(y, dev(so.astype(np.int32)), dev(inp["w"]), out, st)
    torch.cuda.synchronize()
    ydec = bf16_decode(yb.view(torch.int16).numpy().view(np.uint16))
    y_of_slot = {int(s): ydec[i] for i, s in enumerate(slots)}
    ref = moe.combine_rows(y_of_slot, so, inp["w"], toks)
    got = bf16_vals(out)
    check_close(got[toks], ref, f"combine config {cid} ({n_tok} tokens)")
    log(f"combine config {cid}: exact bf16 fraction {(got[toks] == ref).mean():.5f}")
    # tokens whose rows all read zero rows give zero
    others = np.setdiff1d(np.arange(cfg.T), toks)
    touched = np.isin(so[others], slots).any(axis=1)
    assert np.all(got[others[~touched]] == 0)
    assert int(host(st)[0]) == 0


def test_combine_bad_slot_flagged(gpu):
    y = torch.ones(4, 128, dtype=torch.bfloat16, device=gpu)
    so = torch.tensor([[0, 7], [1, -1]], dtype=torch.int32, device=gpu)
    w = torch.tensor([[0.5, 0.5], [1.0, 0.0]], dtype=torch.float32, device=gpu)
    out = torch.empty(2, 128, dtype=torch.bfloat16, device=gpu)
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    fre.moe_combine(y, so, w, out, st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == fre.ERR_BAD_INDEX
    assert np.all(bf16_vals(out)[0] == 0.5) and np.all(bf16_vals(out)[1] == 1.0)
