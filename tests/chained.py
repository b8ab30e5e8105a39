"""The chained layer on the GPU against the chained oracle, shared by the
acceptance tests (tests/test_gpu_layer.py, tests/test_gpu_e8m0.py).

Acceptance, per the workload definition: FP8 codes of the intermediate q2
agree on >= 99.9% of elements, and y and out have relative L2 error <= 2e-3
and per-element |err| <= 0.02 * max|ref|, all against the exact (fp64-sum)
oracle fed the same inputs.

The chained q2 misses the 99.9% bar on every workload, and y / out miss
2e-3 on some.  The cause is measured, not assumed: the FP8 matrix cores
return a 128-product block sum with an error of about 1e-6 of the sum of
|products| (not the correctly rounded fp32 value), which puts about 1% of
GEMM1's bf16 h one ulp away from the exactly rounded value; where that ulp
falls on a block's amax it moves the whole block's q2 scale, and every
dequantised value of the block with it.  Stage by stage, where both sides
start from the same inputs, every bar is met (tests/test_gpu_stages.py).
The misses are therefore reported as strict expected failures carrying
their measured numbers (MEASURED below), never as passes at a looser bar.
"""

import functools

import numpy as np
import torch

import fp8_routed_expert_amd as fre
from oracle import moe, e8m0
from tests.gpu_util import (dev, host, bf16_vals, log, REL_L2_TOL, CODE_AGREE_MIN,
                            MAX_ERR_FRAC)
from tests.inputs import layer_inputs, layer_inputs_e8m0, rows_for

# Chained metrics measured on an MI355X with the current kernels (the fused
# and unfused gate/up paths give bit-identical q2, y and out, so one record
# serves both).  q2: fraction of codes equal; y, out: relative L2.
MEASURED = {
    ("fp32", 1): dict(q2=0.9968872, y=1.781e-3, out=1.554e-3),
    ("fp32", 2): dict(q2=0.9977158, y=1.838e-3, out=1.950e-3),
    ("fp32", 3): dict(q2=0.9981884, y=2.004e-3, out=2.277e-3),
    ("fp32", 4): dict(q2=0.9981883, y=2.215e-3, out=2.057e-3),
    ("fp32", 5): dict(q2=0.9982773, y=1.763e-3, out=1.684e-3),
    ("e8m0", 1): dict(q2=0.9984741, y=1.061e-3, out=1.405e-3),
    ("e8m0", 2): dict(q2=0.9985430, y=1.559e-3, out=1.393e-3),
    ("e8m0", 3): dict(q2=0.9985000, y=2.026e-3, out=2.631e-3),
    ("e8m0", 4): dict(q2=0.9984030, y=1.707e-3, out=2.467e-3),
    ("e8m0", 5): dict(q2=0.9983270, y=1.264e-3, out=1.284e-3),
}


def misses(m):
    """The metrics of `m` that miss the acceptance bar."""
    out = []
    if m["q2"] < CODE_AGREE_MIN:
        out.append(f"q2 code agreement {100 * m['q2']:.3f}% < {100 * CODE_AGREE_MIN:.1f}%")
    for k in ("y", "out"):
        if m[k] > REL_L2_TOL:
            out.append(f"{k} rel_l2 {m[k]:.3e} > {REL_L2_TOL:.0e}")
    return out


def known_miss_reason(fmt, cid):
    """Reason text for a configuration recorded as missing the bar, or None
    if its record meets it."""
    m = MEASURED[(fmt, cid)]
    miss = misses(m)
    if not miss:
        return None
    return (f"{fmt} scales, config {cid}, measured on MI355X: " + "; ".join(miss) +
            " (h from the FP8 matrix cores is ~1% one bf16 ulp off the exact sum)")


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


def _stats(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    nref = np.linalg.norm(ref)
    rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    maxerr = float(np.abs(d).max()) if d.size else 0.0
    bound = MAX_ERR_FRAC * (float(np.abs(ref).max()) if ref.size else 0.0)
    return rel, maxerr, bound


@functools.lru_cache(maxsize=32)
def chained(fmt, cid, fuse):
    """Run the layer once on the GPU and the oracle on sampled tokens;
    return host-side results and metrics (cached: the acceptance test and
    the regression guard share one run)."""
    pk = fmt == "e8m0"
    inp = (layer_inputs_e8m0 if pk else layer_inputs)(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    rows = rows_for(cfg, inp["idx"])
    layer = fre.MoELayer(cfg.E, cfg.H, cfg.I, cfg.T, cfg.K, cfg.layout, rows,
                         align_m=cfg.align_m, scale_fmt=fmt, fuse_act=fuse)
    layer.status.zero_()
    layer.forward(dev(inp["idx"]), dev(inp["x"]), dev(inp["xp" if pk else "xs"]), dev(inp["w"]),
                  dev(inp["w13"]), dev(inp["p13" if pk else "s13"]), dev(inp["w2"]),
                  dev(inp["p2" if pk else "s2"]))
    torch.cuda.synchronize()
    kw = dict(capacity=rows) if cfg.layout == moe.LAYOUT_MASKED else \
        dict(align_m=cfg.align_m, rows=rows)
    L = moe.dispatch_layout(inp["idx"], cfg.E, cfg.layout, **kw)
    toks = _sample_tokens(inp, L)
    log(f"{fmt} config {cid} ({'fused' if fuse else 'unfused'}): oracle on {len(toks)} tokens")
    ref = moe.layer(inp["x"], inp["xs"], inp["idx"], inp["w"], inp["w13"], inp["s13"],
                    inp["w2"], inp["s2"], cfg.layout, tokens=toks,
                    requant=e8m0.act_requant if pk else None, **kw)
    slots = ref["slots"]
    res = dict(status=int(host(layer.status)[0]), slot_of=host(layer.slot_of),
               ref_slot_of=ref["layout"]["slot_of"], empty=(inp["idx"] < 0).all(axis=1))
    out_all = bf16_vals(layer.out)
    res["out_empty"] = out_all[res["empty"]]
    q2 = host(layer.q2)[slots]
    from oracle.codec import e4m3_decode
    res["q2"] = float(np.mean(e4m3_decode(q2) == e4m3_decode(ref["q2"])))
    res["y"], res["y_max"], res["y_bound"] = _stats(bf16_vals(layer.y)[slots], ref["y"])
    res["out"], res["out_max"], res["out_bound"] = _stats(out_all[toks], ref["out"])
    if not fuse:
        h = bf16_vals(layer.h)[slots]
        res["h"], res["h_max"], res["h_bound"] = _stats(h, ref["h"])
        res["h_ulp_off"] = float(np.mean(h != ref["h"]))
    log(f"{fmt} config {cid}: q2 agreement {100 * res['q2']:.4f}%, y rel_l2 {res['y']:.3e} "
        f"(max {res['y_max']:.3e} / {res['y_bound']:.3e}), out rel_l2 {res['out']:.3e} "
        f"(max {res['out_max']:.3e} / {res['out_bound']:.3e})" +
        (f", h rel_l2 {res['h']:.3e}, h elements not equal {100 * res['h_ulp_off']:.3f}%"
         if not fuse else ""))
    del layer
    torch.cuda.empty_cache()
    return res


def check_hard(res):
    """What holds exactly or within its bound on every configuration: status
    clear, slot_of bit-exact, per-element bounds, empty tokens zero, and h
    (unfused) within the stage bar."""
    assert res["status"] == 0
    assert np.array_equal(res["slot_of"], res["ref_slot_of"])
    assert np.all(res["out_empty"] == 0)
    for k in ("y", "out") + (("h",) if "h" in res else ()):
        assert res[f"{k}_max"] <= res[f"{k}_bound"], (k, res[f"{k}_max"], res[f"{k}_bound"])
    if "h" in res:
        assert res["h"] <= REL_L2_TOL


def check_acceptance(res):
    miss = misses(res)
    assert not miss, "; ".join(miss)


def check_regression(fmt, cid, res):
    """Not an acceptance bar: the chained metrics may not get worse than the
    MI355X record by more than measurement-independent slack (the inputs and
    kernels are deterministic; slack covers a changed summation order)."""
    m = MEASURED[(fmt, cid)]
    assert res["q2"] >= m["q2"] - 3e-4, (res["q2"], m["q2"])
    for k in ("y", "out"):
        assert res[k] <= 1.1 * m[k] + 1e-5, (k, res[k], m[k])
