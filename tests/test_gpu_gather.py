"""GPU tests of the gathered gate/up calls (moe_grouped_gemm_fp8_gather,
moe_gate_up_act_fp8_gather and their packed-scale forms) and of the dispatch
without the row copy (a = NULL).  The gathered calls read buffer row r from
x[row_src[r]] in their tile loads instead of reading a permuted buffer; they
must give, bit for bit, what the plain calls give on the permuted buffer --
on the layer workloads and on edge shapes -- and a row whose source is
missing or out of range reads as zero.  Their parity with the oracle is the
chained layer test's, whose default layer runs them (tests/test_gpu_layer.py)."""

import numpy as np
import pytest
import torch

import fp8_routed_expert_amd as fre
from oracle.codec import e4m3_encode
from tests.gpu_util import dev, host, log
from tests.inputs import layer_inputs, layer_inputs_e8m0, rows_for

pytestmark = pytest.mark.gpu

SENTINEL_CODE = 0x5A
SENTINEL_SCALE = -7
CASES = [(c, fmt) for fmt in ("fp32", "e8m0") for c in (1, 2, 3, 4, 5)]


def _dispatch(inp, packed, copy_rows):
    cfg = inp["cfg"]
    idx, x = dev(inp["idx"]), dev(inp["x"])
    xs = dev(inp["xp"] if packed else inp["xs"])
    rows = rows_for(cfg, inp["idx"])
    R = cfg.E * rows if cfg.layout == fre.LAYOUT_MASKED else rows
    T, K, E, H = cfg.T, cfg.K, cfg.E, cfg.H
    i32 = dict(dtype=torch.int32, device="cuda")
    out = dict(counts=torch.zeros(E, **i32), offsets=torch.zeros(E + 1, **i32),
               slot_of=torch.zeros(T, K, **i32), row_src=torch.zeros(R, **i32),
               row_expert=torch.zeros(R, **i32))
    nw = (H // 128 + 3) // 4
    out["a_scale"] = (torch.full((nw, R), SENTINEL_SCALE, **i32) if packed else
                      torch.full((H // 128, R), float(SENTINEL_SCALE), device="cuda"))
    out["a"] = torch.zeros(R, H, dtype=torch.uint8, device="cuda") if copy_rows else None
    ws = torch.zeros(max(1, fre.moe_layout_workspace_bytes(T, K, E)), dtype=torch.uint8,
                     device="cuda")
    st = torch.zeros(1, **i32)
    f = fre.moe_dispatch_layout_e8m0 if packed else fre.moe_dispatch_layout
    f(idx, x, xs, E, cfg.layout, cfg.align_m, rows, out["counts"], out["offsets"],
      out["slot_of"], out["row_src"], out["row_expert"], out["a"], out["a_scale"], ws, st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    return x, out


@pytest.mark.parametrize("cid,fmt", CASES, ids=[f"{c}-{f}" for c, f in CASES])
def test_gather_equals_permuted(gpu, cid, fmt):
    """Dispatch without the row copy writes the same indices and permuted
    scales; the gathered gate/up GEMM and the gathered fused call equal the
    plain calls on the permuted buffer bit for bit, on every row."""
    packed = fmt == "e8m0"
    inp = layer_inputs_e8m0(cid) if packed else layer_inputs(cid)
    cfg = inp["cfg"]
    log(f"gather: config {cid} {fmt}")
    x, full = _dispatch(inp, packed, True)
    _, bare = _dispatch(inp, packed, False)
    for k in ("counts", "offsets", "slot_of", "row_src", "row_expert", "a_scale"):
        assert torch.equal(full[k], bare[k]), k
    w13 = dev(inp["w13"])
    s13 = dev(inp["p13"] if packed else inp["s13"])
    R, I = full["row_src"].numel(), cfg.I
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    h0 = torch.zeros(R, 2 * I, dtype=torch.bfloat16, device="cuda")
    h1 = torch.zeros_like(h0)
    sdt = torch.int32 if packed else torch.float32
    nw = (I // 128 + 3) // 4 if packed else I // 128
    q0 = torch.full((R, I), SENTINEL_CODE, dtype=torch.uint8, device="cuda")
    s0 = torch.full((nw, R), SENTINEL_SCALE, dtype=sdt, device="cuda")
    q1, s1 = q0.clone(), s0.clone()
    o, c, rs, asc = full["offsets"], full["counts"], full["row_src"], full["a_scale"]
    if packed:
        fre.moe_grouped_gemm_fp8_e8m0(full["a"], asc, w13, s13, o, c, h0, st)
        fre.moe_grouped_gemm_fp8_gather_e8m0(x, rs, asc, w13, s13, o, c, h1, st)
        fre.moe_gate_up_act_fp8_e8m0(full["a"], asc, w13, s13, o, c, q0, s0, st)
        fre.moe_gate_up_act_fp8_gather_e8m0(x, rs, asc, w13, s13, o, c, q1, s1, st)
    else:
        fre.moe_grouped_gemm_fp8(full["a"], asc, w13, s13, o, c, h0, st)
        fre.moe_grouped_gemm_fp8_gather(x, rs, asc, w13, s13, o, c, h1, st)
        fre.moe_gate_up_act_fp8(full["a"], asc, w13, s13, o, c, q0, s0, st)
        fre.moe_gate_up_act_fp8_gather(x, rs, asc, w13, s13, o, c, q1, s1, st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(q0, q1) and torch.equal(s0.view(torch.int32), s1.view(torch.int32))
    valid = host(full["row_expert"]) >= 0
    s1h = host(s1)
    assert np.all(s1h[:, valid] != SENTINEL_SCALE)   # every valid row was written
    log(f"gather: config {cid} {fmt}: {int(valid.sum())} rows bit-identical (GEMM and fused)")


@pytest.mark.parametrize("packed", [False, True], ids=["fp32", "e8m0"])
@pytest.mark.parametrize("shape", ["small", "rows320", "rows192"])
def test_gather_edge_rows(gpu, packed, shape):
    """Unaligned segments, an empty expert, and rows whose source is -1 or
    past the last source row inside a segment: the gathered GEMM equals the
    plain GEMM on a buffer built on the host (a[r] = x[row_src[r]], zero
    for a missing source), so a missing source reads zero; the gathered fused
    call equals the plain fused call on that buffer.  "rows320" is a shape
    where the packed-scale GEMM runs its 320-row tiles, "rows192" one where
    both formats run 192-row tiles."""
    g = np.random.default_rng(41 + packed)
    if shape == "small":
        E, I, H, T = 3, 256, 640, 300
        counts = np.array([37, 0, 200])
    elif shape == "rows320":
        E, I, H, T = 3, 1024, 384, 9000
        counts = np.array([5, 0, 13123])
    else:
        E, I, H, T = 3, 1024, 384, 3000
        counts = np.array([5, 0, 4700])
    N = 2 * I
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1]) + 7
    if packed and shape == "rows320":
        assert fre.moe_gemm_tile_rows(R, N, H, E, True) == 320
    if shape == "rows192":
        assert fre.moe_gemm_tile_rows(R, N, H, E, packed) == 192
    x = e4m3_encode(g.standard_normal((T, H)))
    row_src = np.full(R, -1, np.int32)
    row_src[: offsets[-1]] = g.integers(0, T, int(offsets[-1]))
    bad = g.choice(int(offsets[-1]), 6, replace=False)
    row_src[bad[:3]] = -1
    row_src[bad[3:]] = T + np.arange(3)                  # past the source rows
    a = np.zeros((R, H), np.uint8)
    ok = (row_src >= 0) & (row_src < T)
    a[ok] = x[row_src[ok]]
    w13 = e4m3_encode(g.standard_normal((E, N, H)) * 0.05)
    if packed:
        asc = g.integers(0, 2**31 - 1, ((H // 128 + 3) // 4, R)).astype(np.int32)
        asc = (asc & 0x03030303) + 0x7C7C7C7C            # exponents 124..127, four per word
        s13 = ((g.integers(0, 2**31 - 1, (E, N // 128, (H // 128 + 3) // 4)) & 0x03030303)
               + 0x7C7C7C7C).astype(np.int32)
    else:
        asc = g.uniform(0.5, 2.0, (H // 128, R)).astype(np.float32)
        s13 = g.uniform(1e-3, 2e-3, (E, N // 128, H // 128)).astype(np.float32)
    xd, ad, rsd, ascd, wd, swd = dev(x), dev(a), dev(row_src), dev(asc), dev(w13), dev(s13)
    od, cd = dev(offsets), dev(counts.astype(np.int32))
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    h0 = torch.zeros(R, N, dtype=torch.bfloat16, device="cuda")
    h1 = torch.zeros_like(h0)
    sdt = torch.int32 if packed else torch.float32
    nw = (I // 128 + 3) // 4 if packed else I // 128
    q0 = torch.full((R, I), SENTINEL_CODE, dtype=torch.uint8, device="cuda")
    s0 = torch.full((nw, R), SENTINEL_SCALE, dtype=sdt, device="cuda")
    q1, s1 = q0.clone(), s0.clone()
    log(f"gather edge rows: {shape} packed={packed} R={R} N={N} H={H} T={T}")
    if packed:
        fre.moe_grouped_gemm_fp8_e8m0(ad, ascd, wd, swd, od, cd, h0, st)
        fre.moe_grouped_gemm_fp8_gather_e8m0(xd, rsd, ascd, wd, swd, od, cd, h1, st)
        fre.moe_gate_up_act_fp8_e8m0(ad, ascd, wd, swd, od, cd, q0, s0, st)
        fre.moe_gate_up_act_fp8_gather_e8m0(xd, rsd, ascd, wd, swd, od, cd, q1, s1, st)
    else:
        fre.moe_grouped_gemm_fp8(ad, ascd, wd, swd, od, cd, h0, st)
        fre.moe_grouped_gemm_fp8_gather(xd, rsd, ascd, wd, swd, od, cd, h1, st)
        fre.moe_gate_up_act_fp8(ad, ascd, wd, swd, od, cd, q0, s0, st)
        fre.moe_gate_up_act_fp8_gather(xd, rsd, ascd, wd, swd, od, cd, q1, s1, st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    hb0, hb1 = host(h0.view(torch.int16)), host(h1.view(torch.int16))
    assert np.array_equal(hb0, hb1)
    assert not hb1[bad[:3]].any() and not hb1[bad[3:]].any()   # missing sources: zeros
    assert torch.equal(q0, q1) and torch.equal(s0.view(torch.int32), s1.view(torch.int32))
