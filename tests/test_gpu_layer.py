"""Chained GPU layer vs the chained CPU oracle on all five configurations,
plus hipGraph replay, layout equivalence and run-to-run determinism."""

import numpy as np
import pytest
import torch

import fp8_routed_expert_amd as fre
from oracle import moe
from tests import chained
from tests.gpu_util import dev, host
from tests.inputs import layer_inputs, rows_for

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


def test_run_to_run_determinism(gpu):
    inp = layer_inputs(3, experts_needed_only=True)
    cfg = inp["cfg"]
    layer = _layer(cfg, rows_for(cfg, inp["idx"]))
    d = DeviceInputs(inp)
    d.run(layer)
    torch.cuda.synchronize()
    first = host(layer.out).copy()
    for _ in range(2):
        layer.out.zero_()
        d.run(layer)
        torch.cuda.synchronize()
        assert np.array_equal(host(layer.out), first)
