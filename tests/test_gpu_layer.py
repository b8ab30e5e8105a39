"""Chained GPU layer vs the chained CPU oracle on all five configurations,
plus hipGraph replay, layout equivalence and run-to-run determinism."""

import numpy as np
import pytest
import torch

import fp8_routed_expert_amd as fre
from oracle import moe
from tests.gpu_util import dev, host, bf16_vals, check_close, code_agreement, log
from tests.inputs import layer_inputs, rows_for

pytestmark = pytest.mark.gpu

ALL = [1, 2, 3, 4, 5]
CHAINED_REL_L2 = 3e-3


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


def _sample_tokens(inp, L, n=24, seed=0):
    """Tokens with the most rows, tokens owning segment boundary rows, and
    random tokens (all tokens for the tiny configuration)."""
    T = inp["idx"].shape[0]
    if T <= 64:
        return np.arange(T)
    g = np.random.default_rng(seed)
    nrows = (inp["idx"] >= 0).sum(1)
    picks = set(np.argsort(-nrows, kind="stable")[:4].tolist())
    for s, en in moe.expert_segments(L):
        if en > s:
            picks.add(int(L["row_src"][s]))
            picks.add(int(L["row_src"][en - 1]))
    picks |= set(g.choice(T, size=n, replace=False).tolist())
    picks.add(int(np.argmin(nrows)))
    return np.array(sorted(picks))


@pytest.mark.parametrize("fuse", [True, False], ids=["fused", "unfused"])
@pytest.mark.parametrize("cid", ALL)
def test_layer_chained_parity(gpu, cid, fuse):
    """The whole layer against the oracle; fused: gate/up GEMM and
    activation in one call (the default layer), unfused: two calls through
    the bf16 buffer h, which is then checked too."""
    inp = layer_inputs(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    layer = _layer(cfg, rows, fuse_act=fuse)
    d = DeviceInputs(inp)
    layer.status.zero_()
    d.run(layer)
    torch.cuda.synchronize()
    assert int(host(layer.status)[0]) == 0
    kw = dict(capacity=rows) if cfg.layout == moe.LAYOUT_MASKED else \
        dict(align_m=cfg.align_m, rows=rows)
    L = moe.dispatch_layout(inp["idx"], cfg.E, cfg.layout, **kw)
    toks = _sample_tokens(inp, L)
    log(f"config {cid}: oracle on {len(toks)} tokens")
    ref = moe.layer(inp["x"], inp["xs"], inp["idx"], inp["w"], inp["w13"], inp["s13"],
                    inp["w2"], inp["s2"], cfg.layout, tokens=toks, **kw)
    slots = ref["slots"]
    assert np.array_equal(host(layer.slot_of), ref["layout"]["slot_of"])
    if not fuse:
        check_close(bf16_vals(layer.h)[slots], ref["h"], f"config {cid} h")
    # q2 codes here are decided from the device's own h, which differs from
    # the oracle's correctly rounded bf16 h by one ulp in ~1.2% of elements
    # (the FP8 matrix-core sum of 128 products carries an error of ~1e-6 of
    # the sum of |products|); a one-ulp change of a block's amax moves the
    # whole block's scale, so chained codes are held to 99.5% while the
    # 99.9% bar applies where both sides decide from the same h (stage test).
    code_agreement(host(layer.q2)[slots], ref["q2"], f"config {cid} q2", minimum=0.995)
    # The same one-ulp h differences move some blocks' q2 scales by ~0.4%,
    # which shifts every dequantised value of such a block; chained y and out
    # therefore carry ~1.5-2.2e-3 relative L2 against the exact oracle
    # (measured on all five workloads) and are held to 3e-3 here, while every
    # stage-isolated output (tests/test_gpu_stages.py) is held to 2e-3.  The
    # per-element bound (0.02 * max|ref|) is unchanged.
    check_close(bf16_vals(layer.y)[slots], ref["y"], f"config {cid} y", rel_l2_tol=CHAINED_REL_L2)
    out = bf16_vals(layer.out)
    check_close(out[toks], ref["out"], f"config {cid} out", rel_l2_tol=CHAINED_REL_L2)
    # every token with no routed row is exactly zero
    empty = (inp["idx"] < 0).all(axis=1)
    assert np.all(out[empty] == 0)


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
