"""GPU tests of the fused gate/up + activation call (moe_gate_up_act_fp8 and
its packed-scale form).  It must give, bit for bit, what the gate/up grouped
GEMM followed by the activation call gives -- codes and scales of every
valid row, and no write to any other row -- on the layer workloads (both
tile configurations, both layouts) and on edge shapes.  Its parity with the
oracle is the chained layer test's, whose default layer runs the fused call
(tests/test_gpu_layer.py)."""

import numpy as np
import pytest
import torch

import fp8_routed_expert_amd as fre
from oracle import moe
from tests.gpu_util import dev, host, log
from tests.inputs import layer_inputs, layer_inputs_e8m0, rows_for

pytestmark = pytest.mark.gpu

SENTINEL_CODE = 0x5A
SENTINEL_SCALE = -7


def _both(a, a_s, w13, s13, offsets, counts, I, packed):
    """(unfused codes, unfused scales, fused codes, fused scales) on host;
    outputs start as sentinels so that rows nobody may write are compared
    too."""
    rows = a.shape[0]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    nb = I // 128
    sdt = torch.int32 if packed else torch.float32
    sw = (nb + 3) // 4 if packed else nb
    h = torch.zeros(rows, 2 * I, dtype=torch.bfloat16, device="cuda")
    qu = torch.full((rows, I), SENTINEL_CODE, dtype=torch.uint8, device="cuda")
    su = torch.full((sw, rows), SENTINEL_SCALE, dtype=sdt, device="cuda")
    qf, sf = qu.clone(), su.clone()
    if packed:
        fre.moe_grouped_gemm_fp8_e8m0(a, a_s, w13, s13, offsets, counts, h, st)
        fre.moe_act_requant_e8m0(h, offsets, counts, qu, su, st)
        fre.moe_gate_up_act_fp8_e8m0(a, a_s, w13, s13, offsets, counts, qf, sf, st)
    else:
        fre.moe_grouped_gemm_fp8(a, a_s, w13, s13, offsets, counts, h, st)
        fre.moe_act_requant(h, offsets, counts, qu, su, st)
        fre.moe_gate_up_act_fp8(a, a_s, w13, s13, offsets, counts, qf, sf, st)
    torch.cuda.synchronize()
    return host(qu), host(su), host(qf), host(sf)


def _assert_same(qu, su, qf, sf, valid, what):
    assert valid.any(), what
    # the unfused pair wrote every valid row (sentinel scales are gone) ...
    assert np.all(su[:, valid] != SENTINEL_SCALE), what
    # ... and the fused call wrote exactly the same bytes everywhere
    assert np.array_equal(qu, qf), what
    assert np.array_equal(su.view(np.uint8), sf.view(np.uint8)), what
    log(f"{what}: {int(valid.sum())} valid rows bit-identical")


CASES = [(c, fmt) for fmt in ("fp32", "e8m0") for c in (1, 2, 3, 4, 5)]


@pytest.mark.parametrize("cid,fmt", CASES, ids=lambda v: str(v))
def test_fused_equals_gemm_then_act(gpu, cid, fmt):
    packed = fmt == "e8m0"
    inp = (layer_inputs_e8m0 if packed else layer_inputs)(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    layer = fre.MoELayer(cfg.E, cfg.H, cfg.I, cfg.T, cfg.K, cfg.layout, rows,
                         align_m=cfg.align_m, scale_fmt=fmt, gather=False)
    layer.dispatch(dev(inp["idx"]), dev(inp["x"]), dev(inp["xp"] if packed else inp["xs"]))
    w13 = dev(inp["w13"])
    s13 = dev(inp["p13"] if packed else inp["s13"])
    qu, su, qf, sf = _both(layer.a, layer.a_scale, w13, s13, layer.offsets, layer.counts,
                           cfg.I, packed)
    kw = dict(capacity=rows) if cfg.layout == moe.LAYOUT_MASKED else \
        dict(align_m=cfg.align_m, rows=rows)
    L = moe.dispatch_layout(inp["idx"], cfg.E, cfg.layout, **kw)
    valid = L["row_expert"] >= 0
    _assert_same(qu, su, qf, sf, valid, f"config {cid} {fmt}")


def _codes(g, shape):
    t = torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=g)
    t[(t & 0x7F) == 0x7F] = 0x38          # no NaN codes
    return t


# (counts per expert, I, H): unaligned segments with an empty expert and
# tiles straddling segment ends; I = 640 gives five scale blocks (the packed
# form's last word padded) and H = 384 an odd number of K steps; I = H = 128
# a single tile column and a single K step; 150 experts take several passes
# of the wave-parallel tile lookup
EDGE = [((37, 0, 200, 129), 640, 384), ((5, 300), 128, 128), ((1,), 256, 1024),
        (tuple([3, 0, 17, 40, 0, 1] * 25), 256, 256)]   # 150 experts: several lookup passes


@pytest.mark.parametrize("packed", [False, True], ids=["fp32", "e8m0"])
@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"I{c[1]}_H{c[2]}")
def test_fused_edge_shapes(gpu, case, packed):
    counts_l, I, H = case
    E = len(counts_l)
    g = torch.Generator(device="cuda")
    g.manual_seed(I + H + E)
    counts = np.array(counts_l, np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1]) + 5                       # rows past the last segment
    a = _codes(g, (rows, H))
    w13 = _codes(g, (E, 2 * I, H))
    if packed:
        def words(*shape):
            b = torch.randint(120, 135, shape + (4,), dtype=torch.uint8, device="cuda",
                              generator=g)
            return b.view(torch.int32).reshape(shape)
        a_s = words((H // 128 + 3) // 4, rows)
        s13 = words(E, 2 * I // 128, (H // 128 + 3) // 4)
    else:
        a_s = torch.rand(H // 128, rows, device="cuda", generator=g) + 0.5
        s13 = torch.rand(E, 2 * I // 128, H // 128, device="cuda", generator=g) * 1e-3
    qu, su, qf, sf = _both(a, a_s, w13, s13, dev(offsets), dev(counts), I, packed)
    valid = np.zeros(rows, bool)
    for e in range(E):
        valid[offsets[e]:offsets[e] + counts[e]] = True
    _assert_same(qu, su, qf, sf, valid, f"edge {case} {'e8m0' if packed else 'fp32'}")
