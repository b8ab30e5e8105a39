"""GPU test of moe_dispatch_layout_noalloc, the dispatch for callers that
cannot allocate: through the C ABI it must give exactly what
moe_dispatch_layout (with a caller workspace) gives -- counts, offsets,
slot_of, row_src, row_expert, the permuted rows and scales, and the status
word -- on two calls in a row, the second on a smaller input, both layouts."""

import numpy as np
import pytest
import torch

import fp8_routed_expert_amd as fre
from tests.gpu_util import dev, host, log
from tests.inputs import layer_inputs, rows_for

pytestmark = pytest.mark.gpu


def _outputs(E, T, K, H, rows_total):
    """Output buffers pre-filled with sentinels, so rows a call leaves
    untouched are compared too."""
    i32 = dict(dtype=torch.int32, device="cuda")
    return dict(counts=torch.full((E,), -3, **i32), offsets=torch.full((E + 1,), -3, **i32),
                slot_of=torch.full((T, K), -3, **i32), row_src=torch.full((rows_total,), -3, **i32),
                row_expert=torch.full((rows_total,), -3, **i32),
                a=torch.full((rows_total, H), 0x5A, dtype=torch.uint8, device="cuda"),
                a_scale=torch.full((H // 128, rows_total), -7.0, dtype=torch.float32,
                                   device="cuda"),
                status=torch.zeros(1, **i32))


def _dispatch(idx, x, xs, E, layout, align_m, rows, noalloc):
    T, K = idx.shape
    H = x.shape[1]
    rows_total = E * rows if layout == fre.LAYOUT_MASKED else rows
    o = _outputs(E, T, K, H, rows_total)
    common = (idx, x, xs, E, layout, align_m, rows, o["counts"], o["offsets"], o["slot_of"],
              o["row_src"], o["row_expert"], o["a"], o["a_scale"])
    if noalloc:
        fre.moe_dispatch_layout_noalloc(*common, o["status"])
    else:
        ws = torch.zeros(max(1, fre.moe_layout_workspace_bytes(T, K, E)), dtype=torch.uint8,
                         device="cuda")
        fre.moe_dispatch_layout(*common, ws, o["status"])
    torch.cuda.synchronize()
    return {k: host(v) for k, v in o.items()}


def _case(cid, tokens):
    inp = layer_inputs(cid, experts_needed_only=True)
    cfg = inp["cfg"]
    idx = inp["idx"][:tokens]
    rows = cfg.capacity if cfg.layout == fre.LAYOUT_MASKED else \
        rows_for(cfg, idx)
    return cfg, dev(idx), dev(inp["x"][:tokens]), dev(inp["xs"][:tokens]), rows


@pytest.mark.parametrize("layout_cid", [4, 5], ids=["contiguous", "masked"])
def test_noalloc_dispatch_equals_workspace_dispatch(gpu, layout_cid):
    # a large call, then a smaller one: the second reuses the device scratch
    # holding the first call's histograms
    big = 65536 if layout_cid == 4 else 1024
    for tokens in (big, big // 8 + 3):
        cfg, idx, x, xs, rows = _case(layout_cid, tokens)
        log(f"no-alloc dispatch: config {layout_cid}, {tokens} tokens, rows {rows}")
        want = _dispatch(idx, x, xs, cfg.E, cfg.layout, cfg.align_m, rows, noalloc=False)
        got = _dispatch(idx, x, xs, cfg.E, cfg.layout, cfg.align_m, rows, noalloc=True)
        assert int(want["status"][0]) == 0
        for k in want:
            assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), k


def test_noalloc_dispatch_rejects_problems_beyond_its_scratch(gpu):
    """Past the fixed scratch (1 MiB of per-chunk histograms) the call fails
    with MOE_SCRATCH_LIMIT before launching anything."""
    from fp8_routed_expert_amd import _lib
    lib = _lib.load()
    fake = 4096
    # 2 * ceil(T*K/1024) * E * 4 bytes: T = 2^20, K = 8, E = 64 -> 4 MiB
    st = lib.moe_dispatch_layout_noalloc(fake, fake, fake, 1 << 20, 8, 64, 7168, 0, 128,
                                         1 << 23, fake, fake, fake, fake, fake, fake, fake,
                                         fake, None)
    assert st == 4
    assert b"scratch" in lib.moe_status_string(4)
