"""GPU parity of the packed power-of-two scale path (the *_e8m0 calls)
against the oracle's reading of scale quantisation and packing
(oracle/e8m0.py; "Deploying DeepSeek on GB200 NVL72 with PD and Large Scale
EP (Part I)", section 方法实现细节)."""

import numpy as np
import pytest
import torch

import fp8_routed_expert_amd as fre
from oracle import moe, e8m0
from oracle.codec import e4m3_encode, bf16_decode
from tests import chained
from tests.gpu_util import dev, host, check_close, code_agreement, log
from tests.inputs import layer_inputs_e8m0, rows_for, as_words
from workloads import bf16_to_f32

pytestmark = pytest.mark.gpu

def _bf16(g, shape, scale_spread=6.0):
    x = g.standard_normal(shape) * np.exp(g.uniform(-scale_spread, scale_spread, (shape[0], 1)))
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("block_rows,shape", [(1, (256, 384)), (1, (130, 2048)),
                                              (128, (256, 1152)), (128, (128, 512))])
def test_quantize_e8m0_bit_exact(gpu, block_rows, shape):
    """Codes and packed words (including the padding bytes past a row's last
    block) equal the oracle's bit for bit: the exponent is decided from the
    same fp32 quotient and the scaling is exact."""
    g = np.random.default_rng(shape[1] + block_rows)
    xb = _bf16(g, shape)
    R, C = shape
    q = torch.empty(R, C, dtype=torch.uint8, device="cuda")
    nw = (C // 128 + 3) // 4
    s = torch.full((R // block_rows, nw), -1, dtype=torch.int32, device="cuda")
    fre.moe_quantize_fp8_e8m0(xb.cuda(), block_rows, q, s)
    torch.cuda.synchronize()
    rq, re = e8m0.quantize_blocks(bf16_to_f32(xb.view(torch.int16).numpy().view(np.uint16)),
                                  block_rows)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s), as_words(e8m0.pack(re)))


def test_dispatch_e8m0_moves_packed_words(gpu):
    inp = layer_inputs_e8m0(1)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    layer = fre.MoELayer(cfg.E, cfg.H, cfg.I, cfg.T, cfg.K, cfg.layout, rows,
                         align_m=cfg.align_m, scale_fmt="e8m0", gather=False)
    layer.dispatch(dev(inp["idx"]), dev(inp["x"]), dev(inp["xp"]))
    torch.cuda.synchronize()
    L = moe.dispatch_layout(inp["idx"], cfg.E, cfg.layout, align_m=cfg.align_m, rows=rows)
    a_ref, e_ref, filled = moe.permute(inp["x"], inp["xe"], L)
    assert np.array_equal(host(layer.a)[filled], a_ref[filled])
    words = host(layer.a_scale).T
    assert np.array_equal(words[filled], as_words(e8m0.pack(e_ref.astype(np.int32)))[filled])


def _run_gemm_e8m0(a, ea, w, ew, offsets, counts):
    E, N, K = w.shape
    R = a.shape[0]
    c = torch.zeros(R, N, dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    fre.moe_grouped_gemm_fp8_e8m0(dev(a), dev(np.ascontiguousarray(as_words(e8m0.pack(ea)).T)),
                                  dev(w), dev(as_words(e8m0.pack(ew))),
                                  dev(offsets.astype(np.int32)), dev(counts.astype(np.int32)),
                                  c, st)
    torch.cuda.synchronize()
    return host(c)


def test_gemm_e8m0_exact_integers(gpu):
    """Small-integer codes and power-of-two scales keep every sum exact: the
    hardware-scaled product must equal the oracle bit for bit.  With codes
    in [-4, 4] and exponents in [-2, 2] every partial sum is a multiple of
    2^-4 below 2^18, so it is exact in fp32 in any summation order.  K = 640
    has five scale blocks (two words, the second padded); segments are
    unaligned, one expert is empty, tiles straddle segment ends."""
    g = np.random.default_rng(31)
    E, N, K = 4, 384, 640
    counts = np.array([37, 0, 200, 129])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    R = int(offsets[-1]) + 3
    a = e4m3_encode(g.integers(-4, 5, (R, K)).astype(np.float64))
    w = e4m3_encode(g.integers(-4, 5, (E, N, K)).astype(np.float64))
    ea = g.integers(-2, 3, (R, K // 128)).astype(np.int32)
    ew = g.integers(-2, 3, (E, N // 128, K // 128)).astype(np.int32)
    got = _run_gemm_e8m0(a, ea, w, ew, offsets, counts)
    for e in range(E):
        s, en = offsets[e], offsets[e] + counts[e]
        if en > s:
            ref = moe.gemm_rows(a[s:en], e8m0.scales(ea[s:en]), w[e], e8m0.scales(ew[e]))
            assert np.array_equal(bf16_decode(got[s:en]), ref), e


def _run_gemm_fp32(a, sa_rows, w, sw, offsets, counts):
    E, N, K = w.shape
    c = torch.zeros(a.shape[0], N, dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    fre.moe_grouped_gemm_fp8(dev(a), dev(np.ascontiguousarray(sa_rows.T)), dev(w), dev(sw),
                             dev(offsets.astype(np.int32)), dev(counts.astype(np.int32)), c, st)
    torch.cuda.synchronize()
    return host(c)


@pytest.mark.parametrize("packed", [False, True], ids=["fp32", "e8m0"])
def test_gemm_exact_integers_192_row_tiles(gpu, packed):
    """The 192 x 256 tiles (taken when the large tiles fit one round on the
    CUs either way) on exact small-integer data with power-of-two scales, in
    both scale formats: a 5-row expert, an empty one and a long one whose
    last tile straddles its end (4700 = 24 x 192 + 92).  Sampled rows (segment
    ends, every tile boundary, random rows) equal the oracle bit for bit and
    rows outside the segments are never written."""
    g = np.random.default_rng(53 + packed)
    E, N, K = 3, 2048, 384
    counts = np.array([5, 0, 4700])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    R = int(offsets[-1]) + 7
    assert fre.moe_gemm_tile_rows(R, N, K, E, packed) == 192
    a = e4m3_encode(g.integers(-4, 5, (R, K)).astype(np.float64))
    w = e4m3_encode(g.integers(-4, 5, (E, N, K)).astype(np.float64))
    ea = g.integers(-2, 3, (R, K // 128)).astype(np.int32)
    ew = g.integers(-2, 3, (E, N // 128, K // 128)).astype(np.int32)
    log(f"192-row tiles: R={R} N={N} K={K} E={E} packed={packed}")
    if packed:
        got = _run_gemm_e8m0(a, ea, w, ew, offsets, counts)
    else:
        got = _run_gemm_fp32(a, np.ldexp(1.0, ea).astype(np.float32), w,
                             np.ldexp(1.0, ew).astype(np.float32), offsets, counts)
    inside = np.zeros(R, bool)
    for e in range(E):
        s, en = int(offsets[e]), int(offsets[e] + counts[e])
        if en <= s:
            continue
        inside[s:en] = True
        rows = {s, en - 1}
        rows |= {r for t in range(1, (en - s) // 192 + 1) for r in (s + 192 * t - 1, s + 192 * t)
                 if r < en}
        rows |= set(g.integers(s, en, 24).tolist())
        rows = np.array(sorted(rows))
        ref = moe.gemm_rows(a[rows], e8m0.scales(ea[rows]), w[e], e8m0.scales(ew[e]))
        assert np.array_equal(bf16_decode(got[rows]), ref), e
    assert not got[~inside].any()


@pytest.mark.parametrize("K", [128, 384, 640])
def test_gemm_e8m0_exact_integers_320_row_tiles(gpu, K):
    """The 320 x 256 tiles of the packed path (two A stages) on exact
    small-integer data: one, three and five k-blocks, a 5-row expert, an
    empty one and a long ragged one whose tiles straddle its end.  Sampled
    rows (segment ends, every tile boundary, random rows) equal the oracle
    bit for bit; rows outside the segments are never written; and the fused
    gate/up + activation call on the same tiles equals the GEMM followed by
    the activation call bit for bit."""
    g = np.random.default_rng(37 + K)
    E, N = 3, 2048
    counts = np.array([5, 0, 13123])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    R = int(offsets[-1]) + 7
    assert fre.moe_gemm_tile_rows(R, N, K, E, True) == 320
    a = e4m3_encode(g.integers(-4, 5, (R, K)).astype(np.float64))
    w = e4m3_encode(g.integers(-4, 5, (E, N, K)).astype(np.float64))
    ea = g.integers(-2, 3, (R, K // 128)).astype(np.int32)
    ew = g.integers(-2, 3, (E, N // 128, K // 128)).astype(np.int32)
    log(f"320-row tiles: R={R} N={N} K={K} E={E}")
    got = _run_gemm_e8m0(a, ea, w, ew, offsets, counts)
    inside = np.zeros(R, bool)
    for e in range(E):
        s, en = int(offsets[e]), int(offsets[e] + counts[e])
        if en <= s:
            continue
        inside[s:en] = True
        rows = {s, en - 1}
        rows |= {r for t in range(1, (en - s) // 320 + 1) for r in (s + 320 * t - 1, s + 320 * t)
                 if r < en}
        rows |= set(g.integers(s, en, 24).tolist())
        rows = np.array(sorted(rows))
        ref = moe.gemm_rows(a[rows], e8m0.scales(ea[rows]), w[e], e8m0.scales(ew[e]))
        assert np.array_equal(bf16_decode(got[rows]), ref), (e, K)
    assert not got[~inside].any()
    # fused against GEMM + activation on the same 320-row tiles (N = 2I)
    I = N // 2
    od, cd = dev(offsets.astype(np.int32)), dev(counts.astype(np.int32))
    ad, sad = dev(a), dev(np.ascontiguousarray(as_words(e8m0.pack(ea)).T))
    wd, swd = dev(w), dev(as_words(e8m0.pack(ew)))
    nw = (I // 128 + 3) // 4
    h = torch.zeros(R, N, dtype=torch.bfloat16, device="cuda")
    q, qs = (torch.zeros(R, I, dtype=torch.uint8, device="cuda"),
             torch.zeros(nw, R, dtype=torch.int32, device="cuda"))
    qf, qfs = q.clone(), qs.clone()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    fre.moe_grouped_gemm_fp8_e8m0(ad, sad, wd, swd, od, cd, h, st)
    fre.moe_act_requant_e8m0(h, od, cd, q, qs, st)
    fre.moe_gate_up_act_fp8_e8m0(ad, sad, wd, swd, od, cd, qf, qfs, st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    assert np.array_equal(host(qf), host(q)) and np.array_equal(host(qfs), host(qs))


ALL = [1, 2, 3, 4, 5]


@pytest.mark.parametrize("cid", ALL)
def test_gemm1_e8m0_parity(gpu, cid):
    inp = layer_inputs_e8m0(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    kw = dict(capacity=rows) if cfg.layout == moe.LAYOUT_MASKED else \
        dict(align_m=cfg.align_m, rows=rows)
    L = moe.dispatch_layout(inp["idx"], cfg.E, cfg.layout, **kw)
    a, ea, filled = moe.permute(inp["x"], inp["xe"], L)
    ea = ea.astype(np.int32)
    got = _run_gemm_e8m0(a, ea, inp["w13"], inp["e13"], L["offsets"], L["counts"])
    g = np.random.default_rng(cid)
    rs = np.nonzero(filled)[0]
    rs = rs if len(rs) <= 256 else np.sort(g.choice(rs, 256, replace=False))
    ex = L["row_expert"][rs]
    ref = np.zeros((len(rs), 2 * cfg.I))
    for e in np.unique(ex):
        sel = ex == e
        ref[sel] = moe.gemm_rows(a[rs[sel]], e8m0.scales(ea[rs[sel]]), inp["w13"][e],
                                 inp["s13"][e])
    check_close(bf16_decode(got[rs]), ref, f"gemm1 e8m0 config {cid} ({len(rs)} rows)")


@pytest.mark.parametrize("cid", ALL)
def test_gemm2_e8m0_parity(gpu, cid):
    """Stage-isolated down projection with packed power-of-two scales:
    oracle-quantised (R18-R19) rows on sampled slots of every expert,
    including each segment's first and last row, against oracle.moe.gemm_rows
    fed the scales 2^e."""
    inp = layer_inputs_e8m0(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    kw = dict(capacity=rows) if cfg.layout == moe.LAYOUT_MASKED else \
        dict(align_m=cfg.align_m, rows=rows)
    L = moe.dispatch_layout(inp["idx"], cfg.E, cfg.layout, **kw)
    R = L["rows_total"]
    g = np.random.default_rng(100 + cid)
    rs = set()
    for s, en in moe.expert_segments(L):
        if en > s:
            rs |= {s, en - 1}
            rs |= set(g.choice(np.arange(s, en), size=min(6, en - s), replace=False).tolist())
    rs = np.array(sorted(rs))
    q2 = np.zeros((R, cfg.I), np.uint8)
    eq = np.zeros((R, cfg.I // 128), np.int32)
    vals = g.standard_normal((len(rs), cfg.I)) * np.exp(g.uniform(-3, 3, (len(rs), 1)))
    q2[rs], eq[rs] = e8m0.quantize_blocks(vals, 1)
    got = _run_gemm_e8m0(q2, eq, inp["w2"], inp["e2"], L["offsets"], L["counts"])
    ex = L["row_expert"][rs]
    ref = np.zeros((len(rs), cfg.H))
    for e in np.unique(ex):
        sel = ex == e
        ref[sel] = moe.gemm_rows(q2[rs[sel]], e8m0.scales(eq[rs[sel]]), inp["w2"][e],
                                 inp["s2"][e])
    check_close(bf16_decode(got[rs]), ref, f"gemm2 e8m0 config {cid} ({len(rs)} rows)")


def test_act_e8m0_vs_oracle(gpu):
    """From the same bf16 h: codes and exponents agree with the oracle in
    >= 99.9% of places (SiLU is evaluated with the hardware exp2 and
    reciprocal, the oracle in fp64), and the padding bytes are exact."""
    g = np.random.default_rng(8)
    E, I, rows = 3, 640, 300          # five blocks per row: two words, padded
    counts = np.array([100, 0, 190])
    offsets = np.array([0, 100, 100, 290], np.int32)
    hv = g.standard_normal((rows, 2 * I)) * np.exp(g.uniform(-2, 2, (rows, 1)))
    hb = torch.from_numpy(hv.astype(np.float32)).to(torch.bfloat16)
    q = torch.zeros(rows, I, dtype=torch.uint8, device="cuda")
    qs = torch.zeros((I // 128 + 3) // 4, rows, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    fre.moe_act_requant_e8m0(hb.cuda(), dev(offsets), dev(counts.astype(np.int32)), q, qs, st)
    torch.cuda.synchronize()
    valid = np.r_[0:100, 100:290]
    h = bf16_to_f32(hb.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    rq, re = e8m0.quantize_blocks(moe.silu_mul(h[valid]), 1)
    code_agreement(host(q)[valid], rq, "act e8m0 codes")
    words = host(qs).T[valid].view(np.uint32)
    ge = e8m0.unpack(words, I // 128)
    agree = float(np.mean(ge == re))
    log(f"act e8m0 exponent agreement {agree:.5f}")
    assert agree >= 0.999
    pad = (words[:, -1] >> 8) & 0xFFFFFF          # bytes 1..3 of the last word
    assert np.all(pad == 0x7F7F7F)


def _acceptance_params(cids):
    ps = []
    for cid in cids:
        for fuse in (True, False):
            reason = chained.known_miss_reason("e8m0", cid)
            marks = [pytest.mark.xfail(strict=True, reason=reason)] if reason else []
            ps.append(pytest.param(cid, fuse, marks=marks,
                                   id=f"{cid}-{'fused' if fuse else 'unfused'}"))
    return ps


@pytest.mark.parametrize("cid,fuse", _acceptance_params(ALL))
def test_layer_e8m0_chained(gpu, cid, fuse):
    """The packed-scale layer against the oracle's packed-scale chain at the
    workload's acceptance bars; recorded misses are strict expected failures
    carrying their measured numbers (tests/chained.py)."""
    res = chained.chained("e8m0", cid, fuse)
    chained.check_hard(res)
    chained.check_acceptance(res)


@pytest.mark.parametrize("fuse", [True, False], ids=["fused", "unfused"])
@pytest.mark.parametrize("cid", ALL)
def test_layer_e8m0_chained_no_regression(gpu, cid, fuse):
    """Regression guard, not the acceptance bar (see the fp32-scale one)."""
    res = chained.chained("e8m0", cid, fuse)
    chained.check_hard(res)
    chained.check_regression("e8m0", cid, res)
