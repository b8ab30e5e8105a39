"""A routed-expert MoE layer share that owns its device buffers.

MoELayer allocates every intermediate once (torch device memory) and runs
the library calls of one layer on a stream:

  moe_dispatch_layout -> moe_gate_up_act_fp8 (gate/up GEMM + activation)
  -> moe_grouped_gemm_fp8 (down) -> moe_combine

With fuse_act=False the gate/up GEMM and the activation run as two calls
(moe_grouped_gemm_fp8 -> moe_act_requant) through a bf16 buffer h; both
orders give the same q2 bit for bit.  fuse_act="auto" (the default) fuses
when the library runs the gate/up GEMM with its large 256 x 256 tiles (the
same size rule as the library's); with the small tiles (the masked decode
layout) the two calls measured faster, since the fused kernel then needs
128 x 256 tiles at one workgroup per CU.

All arithmetic happens in the HIP library; this class only holds memory.
The call sequence allocates nothing and reads nothing back, so it can be
captured into a hipGraph (torch.cuda.CUDAGraph) and replayed.

scale_fmt "fp32" keeps fp32 block scales; "e8m0" uses packed power-of-two
scales (int32 words of four biased exponents; the *_e8m0 calls), in which
case x_scale and the weight scales passed in must be packed the same way.

gather=True (the default) skips the copy of the routed rows into a permuted
buffer: the dispatch writes the indices and the permuted scales only, and the
gate/up call reads buffer row r from x[row_src[r]] in its tile loads (the
*_gather calls; bit-identical results).  The x passed to dispatch() must
then stay unchanged until the gate/up call has run.  gather=False copies the
rows into `a` (moe_dispatch_layout's full permute).
"""

import torch

from . import ops


def contiguous_rows(R, E, align_m=128):
    """Buffer rows that hold R routed rows in E segments aligned to align_m."""
    return int(R) + E * (align_m - 1)


def big_gate_up_tiles(rows_total, I, E):
    """Whether the library runs the gate/up GEMM of this buffer with its
    256 x 256 tiles (asked from the library, which owns the rule)."""
    return ops.moe_gemm_large_tiles(rows_total, 2 * int(I), E) == 1


class MoELayer:
    def __init__(self, E, H, I, T, K, layout, rows, align_m=128, device="cuda",
                 scale_fmt="fp32", fuse_act="auto", gather=True):
        """rows: M_cap for the contiguous layout, capacity C for masked."""
        if scale_fmt not in ("fp32", "e8m0"):
            raise ValueError(f"scale_fmt {scale_fmt!r}")
        if fuse_act not in ("auto", True, False):
            raise ValueError(f"fuse_act {fuse_act!r}")
        if gather not in (True, False):
            raise ValueError(f"gather {gather!r}")
        self.gather = gather
        self._x = None
        self.scale_fmt = scale_fmt
        self.E, self.H, self.I, self.T, self.K = E, H, I, T, K
        self.layout, self.rows, self.align_m = layout, rows, align_m
        self.rows_total = E * rows if layout == ops.LAYOUT_MASKED else rows
        R, d = self.rows_total, device
        if fuse_act == "auto":
            fuse_act = big_gate_up_tiles(R, I, E)
        self.fuse_act = bool(fuse_act)
        i32 = dict(dtype=torch.int32, device=d)
        self.counts = torch.zeros(E, **i32)
        self.offsets = torch.zeros(E + 1, **i32)
        self.slot_of = torch.zeros(T, K, **i32)
        self.row_src = torch.zeros(R, **i32)
        self.row_expert = torch.zeros(R, **i32)
        self.a = None if gather else torch.zeros(R, H, dtype=torch.uint8, device=d)
        pk = scale_fmt == "e8m0"
        sdt = torch.int32 if pk else torch.float32
        self.a_scale = torch.zeros((H // 128 + 3) // 4 if pk else H // 128, R, dtype=sdt,
                                   device=d)
        # h exists only on the unfused path
        self.h = None if self.fuse_act else torch.zeros(R, 2 * I, dtype=torch.bfloat16,
                                                        device=d)
        self.q2 = torch.zeros(R, I, dtype=torch.uint8, device=d)
        self.q2_scale = torch.zeros((I // 128 + 3) // 4 if pk else I // 128, R, dtype=sdt,
                                    device=d)
        self.y = torch.zeros(R, H, dtype=torch.bfloat16, device=d)
        self.out = torch.zeros(T, H, dtype=torch.bfloat16, device=d)
        self.workspace = torch.zeros(max(1, ops.moe_layout_workspace_bytes(T, K, E)),
                                     dtype=torch.uint8, device=d)
        self.status = torch.zeros(1, **i32)

    def dispatch(self, topk_idx, x, x_scale, stream=None):
        f = (ops.moe_dispatch_layout_e8m0 if self.scale_fmt == "e8m0"
             else ops.moe_dispatch_layout)
        f(topk_idx, x, x_scale, self.E, self.layout, self.align_m, self.rows, self.counts,
          self.offsets, self.slot_of, self.row_src, self.row_expert, self.a, self.a_scale,
          self.workspace, self.status, stream)
        self._x = x   # the gathered gate/up call reads the rows from here

    def gemm1(self, w13, s13, stream=None):
        """Unfused path: h = gate/up GEMM (needs fuse_act=False)."""
        if self.h is None:
            raise RuntimeError("gemm1/act are the unfused path: build with fuse_act=False")
        if self.gather:
            f = (ops.moe_grouped_gemm_fp8_gather_e8m0 if self.scale_fmt == "e8m0"
                 else ops.moe_grouped_gemm_fp8_gather)
            f(self._source(), self.row_src, self.a_scale, w13, s13, self.offsets, self.counts,
              self.h, self.status, stream)
            return
        self._gemm(self.a, self.a_scale, w13, s13, self.offsets, self.counts, self.h,
                   self.status, stream)

    def _source(self):
        if self._x is None:
            raise RuntimeError("the gathered gate/up call needs dispatch() first")
        return self._x

    def gemm1_act(self, w13, s13, stream=None):
        """Fused path: q2, q2_scale straight from the gate/up GEMM."""
        if self.gather:
            f = (ops.moe_gate_up_act_fp8_gather_e8m0 if self.scale_fmt == "e8m0"
                 else ops.moe_gate_up_act_fp8_gather)
            f(self._source(), self.row_src, self.a_scale, w13, s13, self.offsets, self.counts,
              self.q2, self.q2_scale, self.status, stream)
            return
        f = (ops.moe_gate_up_act_fp8_e8m0 if self.scale_fmt == "e8m0"
             else ops.moe_gate_up_act_fp8)
        f(self.a, self.a_scale, w13, s13, self.offsets, self.counts, self.q2, self.q2_scale,
          self.status, stream)

    def _gemm(self, *args):
        f = (ops.moe_grouped_gemm_fp8_e8m0 if self.scale_fmt == "e8m0"
             else ops.moe_grouped_gemm_fp8)
        f(*args)

    def act(self, stream=None):
        if self.h is None:
            raise RuntimeError("gemm1/act are the unfused path: build with fuse_act=False")
        f = ops.moe_act_requant_e8m0 if self.scale_fmt == "e8m0" else ops.moe_act_requant
        f(self.h, self.offsets, self.counts, self.q2, self.q2_scale, self.status, stream)

    def gemm2(self, w2, s2, stream=None):
        self._gemm(self.q2, self.q2_scale, w2, s2, self.offsets, self.counts, self.y,
                   self.status, stream)

    def combine(self, topk_w, stream=None):
        ops.moe_combine(self.y, self.slot_of, topk_w, self.out, self.status, stream)

    def forward(self, topk_idx, x, x_scale, topk_w, w13, s13, w2, s2, stream=None):
        """One full pass S1-S8; returns self.out (bf16 [T, H])."""
        self.dispatch(topk_idx, x, x_scale, stream)
        if self.fuse_act:
            self.gemm1_act(w13, s13, stream)
        else:
            self.gemm1(w13, s13, stream)
            self.act(stream)
        self.gemm2(w2, s2, stream)
        self.combine(topk_w, stream)
        return self.out
