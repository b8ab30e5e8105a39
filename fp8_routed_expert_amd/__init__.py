"""MI355X (gfx950) FP8 routed-expert MoE layer: one GPU's share under expert
parallelism.  The arithmetic lives in the HIP library libmoe_fp8.so (C ABI in
include/moe_fp8.h); this package is its Python binding."""

from .ops import (moe_layout_workspace_bytes, moe_gemm_large_tiles, moe_gemm_tile_rows,  # noqa: F401
                  moe_dispatch_layout,
                  moe_dispatch_layout_noalloc,
                  moe_grouped_gemm_fp8, moe_gemm_fp8, moe_act_requant, moe_combine,
                  moe_quantize_fp8, moe_quantize_fp8_e8m0, moe_dispatch_layout_e8m0,
                  moe_grouped_gemm_fp8_e8m0, moe_act_requant_e8m0,
                  moe_gate_up_act_fp8, moe_gate_up_act_fp8_e8m0,
                  moe_grouped_gemm_fp8_gather, moe_grouped_gemm_fp8_gather_e8m0,
                  moe_gate_up_act_fp8_gather, moe_gate_up_act_fp8_gather_e8m0,
                  moe_ceiling_copy, moe_ceiling_mfma_fp8,
                  LAYOUT_CONTIGUOUS, LAYOUT_MASKED,
                  ERR_BAD_EXPERT, ERR_OVERFLOW, ERR_BAD_INDEX)
from .layer import MoELayer, contiguous_rows  # noqa: F401
