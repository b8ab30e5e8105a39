"""Canary-padded buffers around every argument of every layer call: each
device tensor a call reads or writes sits inside a larger allocation with
4 KiB of guard bytes on both sides, and after each call the guard bytes must
be unchanged (no write outside an output) and every input must equal its
copy from before the call (no write into an input).  Run on the three tile
and layout shapes of the layer (the tiny workload, the EP72 decode share with
the large tiles, the masked layout with the small tiles), for both scale
formats and for the copying and the gathering paths."""

import numpy as np
import pytest
import torch

import fp8_routed_expert_amd as fre
from tests.gpu_util import dev, log
from tests.inputs import layer_inputs, layer_inputs_e8m0, rows_for

pytestmark = pytest.mark.gpu

PAD = 4096
GUARD = 0xA5


class Guarded:
    """Device tensors carved out of guarded allocations."""

    def __init__(self):
        self.bufs = []

    def new(self, shape, dtype, fill=0):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        raw = torch.full((n + 2 * PAD,), GUARD, dtype=torch.uint8, device="cuda")
        t = raw[PAD:PAD + n].view(dtype).view(shape)
        if fill is not None:
            t.fill_(fill)
        self.bufs.append(raw)
        return t

    def like(self, a):
        t = self.new(tuple(a.shape), a.dtype, fill=None)
        t.copy_(a)
        return t

    def check(self, what):
        torch.cuda.synchronize()
        for raw in self.bufs:
            assert int((raw[:PAD] != GUARD).sum()) == 0, f"{what}: write before a buffer"
            assert int((raw[-PAD:] != GUARD).sum()) == 0, f"{what}: write after a buffer"


def _unchanged(inputs, copies, what):
    torch.cuda.synchronize()
    for name, (t, c) in zip(inputs, copies):
        assert torch.equal(t.view(torch.uint8), c.view(torch.uint8)), f"{what}: input {name} written"


CASES = [(c, fmt, gather) for c in (1, 2, 5) for fmt in ("fp32", "e8m0")
         for gather in (False, True)]


@pytest.mark.parametrize("cid,fmt,gather", CASES,
                         ids=[f"{c}-{f}-{'gather' if g else 'copy'}" for c, f, g in CASES])
def test_calls_stay_inside_their_buffers(gpu, cid, fmt, gather):
    packed = fmt == "e8m0"
    inp = (layer_inputs_e8m0 if packed else layer_inputs)(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    E, H, I, T, K = cfg.E, cfg.H, cfg.I, cfg.T, cfg.K
    rows = rows_for(cfg, inp["idx"])
    R = E * rows if cfg.layout == fre.LAYOUT_MASKED else rows
    g = Guarded()
    i32, u8, bf = torch.int32, torch.uint8, torch.bfloat16
    sdt = i32 if packed else torch.float32
    hw = (H // 128 + 3) // 4 if packed else H // 128
    iw = (I // 128 + 3) // 4 if packed else I // 128
    # inputs
    idx, x = g.like(dev(inp["idx"])), g.like(dev(inp["x"]))
    xs = g.like(dev(inp["xp"] if packed else inp["xs"]))
    w = g.like(dev(inp["w"]))
    w13, w2 = g.like(dev(inp["w13"])), g.like(dev(inp["w2"]))
    s13 = g.like(dev(inp["p13"] if packed else inp["s13"]))
    s2 = g.like(dev(inp["p2"] if packed else inp["s2"]))
    ins = ["topk_idx", "x", "x_scale", "topk_w", "w13", "s13", "w2", "s2"]
    tens = [idx, x, xs, w, w13, s13, w2, s2]
    copies = [t.clone() for t in tens]
    # outputs
    counts, offsets = g.new((E,), i32), g.new((E + 1,), i32)
    slot_of, row_src, row_expert = g.new((T, K), i32), g.new((R,), i32), g.new((R,), i32)
    a = None if gather else g.new((R, H), u8)
    a_scale = g.new((hw, R), sdt)
    ws = g.new((max(1, fre.moe_layout_workspace_bytes(T, K, E)),), u8)
    st = g.new((1,), i32)
    h = g.new((R, 2 * I), bf)
    q2, q2s = g.new((R, I), u8), g.new((iw, R), sdt)
    q2f, q2fs = g.new((R, I), u8), g.new((iw, R), sdt)
    y, out = g.new((R, H), bf), g.new((T, H), bf)
    log(f"canary: config {cid} {fmt} {'gather' if gather else 'copy'} R={R}")

    def step(what, f, *args):
        f(*args)
        g.check(what)
        _unchanged(ins, list(zip(tens, copies)), what)

    disp = fre.moe_dispatch_layout_e8m0 if packed else fre.moe_dispatch_layout
    step("dispatch", disp, idx, x, xs, E, cfg.layout, cfg.align_m, rows, counts, offsets,
         slot_of, row_src, row_expert, a, a_scale, ws, st)
    if gather:
        gemm = fre.moe_grouped_gemm_fp8_gather_e8m0 if packed else fre.moe_grouped_gemm_fp8_gather
        fused = fre.moe_gate_up_act_fp8_gather_e8m0 if packed else fre.moe_gate_up_act_fp8_gather
        step("gate/up GEMM", gemm, x, row_src, a_scale, w13, s13, offsets, counts, h, st)
        step("gate/up + act", fused, x, row_src, a_scale, w13, s13, offsets, counts, q2f, q2fs,
             st)
    else:
        gemm = fre.moe_grouped_gemm_fp8_e8m0 if packed else fre.moe_grouped_gemm_fp8
        fused = fre.moe_gate_up_act_fp8_e8m0 if packed else fre.moe_gate_up_act_fp8
        step("gate/up GEMM", gemm, a, a_scale, w13, s13, offsets, counts, h, st)
        step("gate/up + act", fused, a, a_scale, w13, s13, offsets, counts, q2f, q2fs, st)
    act = fre.moe_act_requant_e8m0 if packed else fre.moe_act_requant
    step("act", act, h, offsets, counts, q2, q2s, st)
    down = fre.moe_grouped_gemm_fp8_e8m0 if packed else fre.moe_grouped_gemm_fp8
    step("down GEMM", down, q2, q2s, w2, s2, offsets, counts, y, st)
    step("combine", fre.moe_combine, y, slot_of, w, out, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
