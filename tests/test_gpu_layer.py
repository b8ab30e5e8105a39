"""Chained GPU layer vs the chained CPU oracle on all five configurations,
plus hipGraph replay, layout equivalence and run-to-run determinism."""

import numpy as np
import pytest
import torch

import fp8_routed_expert_amd as fre
from oracle import moe
from tests import chained
from tests.gpu_util import dev, host, log
from tests.inputs import layer_inputs, rows_for
from workloads import CONFIGS, routing

pytestmark = pytest.mark.gpu

ALL = [1, 2, 3, 4, 5]


class DeviceInputs:
    def __init__(self, inp):
        self.idx = dev(inp["idx"])
        self.w = dev(inp["w"])
        self.x = dev(inp["x"])
        self.xs = dev(inp["xs"])
        self.w13 = dev(inp["w13"])
        self.s13 = dev(inp["s13"])
        self.w2 = dev(inp["w2"])
        self.s2 = dev(inp["s2"])

    def run(self, layer, stream=None):
        return layer.forward(self.idx, self.x, self.xs, self.w, self.w13, self.s13,
                             self.w2, self.s2, stream)


def _layer(cfg, rows, layout=None, fuse_act=True):
    return fre.MoELayer(cfg.E, cfg.H, cfg.I, cfg.T, cfg.K,
                        cfg.layout if layout is None else layout, rows, align_m=cfg.align_m,
                        fuse_act=fuse_act)


def _acceptance_params(fmt, cids):
    ps = []
    for cid in cids:
        for fuse in (True, False):
            reason = chained.known_miss_reason(fmt, cid)
            marks = [pytest.mark.xfail(strict=True, reason=reason)] if reason else []
            ps.append(pytest.param(cid, fuse, marks=marks,
                                   id=f"{cid}-{'fused' if fuse else 'unfused'}"))
    return ps


@pytest.mark.parametrize("cid,fuse", _acceptance_params("fp32", ALL))
def test_layer_chained_parity(gpu, cid, fuse):
    """The whole layer against the oracle at the workload's acceptance bars
    (q2 codes >= 99.9%, y and out rel L2 <= 2e-3, per-element bound).
    fused: gate/up GEMM and activation in one call (the default layer at
    large sizes); unfused: two calls through the bf16 buffer h.  A
    configuration recorded as missing a bar is a strict expected failure
    whose reason carries the measured numbers (tests/chained.py)."""
    res = chained.chained("fp32", cid, fuse)
    chained.check_hard(res)
    chained.check_acceptance(res)


@pytest.mark.parametrize("fuse", [True, False], ids=["fused", "unfused"])
@pytest.mark.parametrize("cid", ALL)
def test_layer_chained_no_regression(gpu, cid, fuse):
    """Regression guard, not the acceptance bar: layout bit-exact, status
    clear, per-element bounds, h within the stage bar, and chained metrics
    no worse than the MI355X record."""
    res = chained.chained("fp32", cid, fuse)
    chained.check_hard(res)
    chained.check_regression("fp32", cid, res)


@pytest.mark.parametrize("fuse", [True, False], ids=["fused", "unfused"])
def test_masked_layer_hipgraph_replay(gpu, fuse):
    """Config 5 (masked, decode): the layer's launches captured in one graph;
    every replay equals the eager result bit for bit."""
    inp = layer_inputs(5, experts_needed_only=True)
    cfg = inp["cfg"]
    layer = _layer(cfg, cfg.capacity, fuse_act=fuse)
    d = DeviceInputs(inp)
    d.run(layer)
    torch.cuda.synchronize()
    eager = host(layer.out).copy()
    eager_y = host(layer.y).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.run(layer)                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.run(layer)
    for rep in range(4):
        layer.out.zero_()
        layer.y.zero_()
        layer.status.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(layer.out), eager), rep
        assert np.array_equal(host(layer.y), eager_y), rep
        assert int(host(layer.status)[0]) == 0
        # eager work between replays
        x2 = layer.out.float().sum()
        assert torch.isfinite(x2)


def test_contiguous_equals_masked(gpu):
    """The same routing through both layouts gives bit-identical expert rows
    and outputs (each row's result depends only on its own data)."""
    inp = layer_inputs(5, experts_needed_only=True)
    cfg = inp["cfg"]
    d = DeviceInputs(inp)
    lm = _layer(cfg, cfg.capacity)
    d.run(lm)
    lc = _layer(cfg, rows_for(cfg, inp["idx"]) if cfg.layout != moe.LAYOUT_MASKED
                else int((inp["idx"] >= 0).sum()) + cfg.E * 127, layout=fre.LAYOUT_CONTIGUOUS)
    d.run(lc)
    torch.cuda.synchronize()
    assert np.array_equal(host(lm.out), host(lc.out))
    som, soc = host(lm.slot_of), host(lc.slot_of)
    v = som >= 0
    assert np.array_equal(v, soc >= 0)
    assert np.array_equal(host(lm.y)[som[v]], host(lc.y)[soc[v]])


def _device_quantised_inputs(cfg, fmt, seed):
    """Routing from the workload; activations and weights drawn on the
    device and quantised there (inputs only need to be the same from run to
    run here, not known to the oracle)."""
    idx, w = routing(cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    E, H, I, T = cfg.E, cfg.H, cfg.I, cfg.T
    pk = fmt == "e8m0"
    q = fre.moe_quantize_fp8_e8m0 if pk else fre.moe_quantize_fp8
    hw, iw = ((H // 128 + 3) // 4, (I // 128 + 3) // 4) if pk else (H // 128, I // 128)
    sdt = torch.int32 if pk else torch.float32
    x = torch.empty(T, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(T, hw, dtype=sdt, device="cuda")
    w13 = torch.empty(E, 2 * I, H, dtype=torch.uint8, device="cuda")
    s13 = torch.empty(E, 2 * I // 128, hw, dtype=sdt, device="cuda")
    w2 = torch.empty(E, H, I, dtype=torch.uint8, device="cuda")
    s2 = torch.empty(E, H // 128, iw, dtype=sdt, device="cuda")
    q(torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16), 1, x, xs)
    q((torch.randn(E * 2 * I, H, generator=g, device="cuda") * 0.02).to(torch.bfloat16), 128,
      w13.view(E * 2 * I, H), s13.view(E * 2 * I // 128, -1))
    q((torch.randn(E * H, I, generator=g, device="cuda") * 0.02).to(torch.bfloat16), 128,
      w2.view(E * H, I), s2.view(E * H // 128, -1))
    return dev(idx), dev(w), x, xs, w13, s13, w2, s2


DETERMINISM = [(2, "fp32"), (2, "e8m0"), (3, "fp32"), (3, "e8m0"), (5, "fp32"), (5, "e8m0"),
               (4, "e8m0")]


@pytest.mark.parametrize("cid,fmt", DETERMINISM, ids=[f"{c}-{f}" for c, f in DETERMINISM])
def test_run_to_run_determinism(gpu, cid, fmt):
    """Three passes of the default layer over the same inputs give the same
    bits in y, q2 and out.  The cases span the tile shapes the host rule
    picks: 192-row fused gate/up tiles (EP72), 256-row tiles (EP48),
    64-row gate/up and 128-row down tiles (masked), 320-row down tiles
    (prefill, packed scales), in both scale formats.  A tile stage read
    before it was loaded showed up exactly as run-to-run differences."""
    cfg = CONFIGS[cid]
    args = _device_quantised_inputs(cfg, fmt, 4000 + cid)
    R = int((args[0] >= 0).sum().item())
    rows = cfg.capacity if cfg.layout == fre.LAYOUT_MASKED else fre.contiguous_rows(
        R, cfg.E, cfg.align_m)
    layer = fre.MoELayer(cfg.E, cfg.H, cfg.I, cfg.T, cfg.K, cfg.layout, rows,
                         align_m=cfg.align_m, scale_fmt=fmt)
    idx, w, x, xs, w13, s13, w2, s2 = args
    log(f"determinism: config {cid} {fmt} rows={rows} fused={layer.fuse_act}")
    snaps = []
    for _ in range(3):
        layer.y.zero_()
        layer.q2.zero_()
        layer.out.zero_()
        layer.forward(idx, x, xs, w, w13, s13, w2, s2)
        torch.cuda.synchronize()
        valid = layer.row_expert >= 0
        snaps.append((layer.y[valid].view(torch.int16).cpu().numpy(),
                      layer.q2[valid].cpu().numpy(), host(layer.out).copy()))
    assert int(layer.status.item()) == 0
    for later in snaps[1:]:
        for a, b in zip(snaps[0], later):
            assert np.array_equal(a, b)
