// Host-side argument handling of every C-ABI entry point, run without a
// GPU: each call below must return its status before any device work.  The
// test that builds this file links it against the library compiled with
// AddressSanitizer on its host code, so a host-side overread, overflow or
// use of freed memory on these paths aborts the run.  Exit status: the
// number of calls whose status differed from the expected one.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "moe_fp8.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  // plausible non-null device pointers that are never dereferenced on the host
  alignas(64) static unsigned char pool[4096];
  void* p = pool;
  void* odd = pool + 1;                     // misaligned
  const int32_t* ip = static_cast<const int32_t*>(p);
  int32_t* wp = static_cast<int32_t*>(p);
  auto u8 = static_cast<uint8_t*>(p);
  auto f32 = static_cast<float*>(p);
  auto u16 = static_cast<uint16_t*>(p);
  auto u32 = static_cast<uint32_t*>(p);

  // helpers
  expect("abi version", moe_abi_version() > 0, 1);
  for (int s = 0; s <= 5; ++s) expect("status string", std::strlen(moe_status_string(s)) > 0, 1);
  expect("status string unknown", std::strcmp(moe_status_string(99), "unknown status"), 0);
  expect("workspace bytes invalid", (int)moe_layout_workspace_bytes(-1, 8, 4), 0);
  expect("workspace bytes", moe_layout_workspace_bytes(2048, 8, 32) > 0, 1);
  expect("large tiles invalid", moe_gemm_large_tiles(0, 4096, 1), -1);
  expect("large tiles prefill", moe_gemm_large_tiles(132183, 4096, 9), 1);
  expect("tile rows packed prefill", moe_gemm_tile_rows(132183, 7168, 2048, 9, 1), 320);
  expect("tile rows masked gate/up", moe_gemm_tile_rows(4096, 4096, 7168, 32, 0), 64);
  expect("tile rows masked down", moe_gemm_tile_rows(4096, 7168, 2048, 32, 0), 128);
  expect("tile rows invalid K", moe_gemm_tile_rows(4096, 7168, 0, 32, 0), -1);

  // dispatch: topk, x, x_scale, T, K, E, H, layout, align_m, rows, counts,
  // offsets, slot_of, row_src, row_expert, a, a_scale, workspace, bytes, status, stream
  const size_t wsb = moe_layout_workspace_bytes(64, 2, 4);
  expect("dispatch T<0", moe_dispatch_layout(ip, u8, f32, -1, 2, 4, 256, 0, 128, 640, wp, wp, wp,
                                             wp, wp, u8, f32, p, wsb, wp, nullptr), MOE_INVALID_ARG);
  expect("dispatch K=0", moe_dispatch_layout(ip, u8, f32, 64, 0, 4, 256, 0, 128, 640, wp, wp, wp,
                                             wp, wp, u8, f32, p, wsb, wp, nullptr), MOE_INVALID_ARG);
  expect("dispatch layout", moe_dispatch_layout(ip, u8, f32, 64, 2, 4, 256, 7, 128, 640, wp, wp,
                                                wp, wp, wp, u8, f32, p, wsb, wp, nullptr),
         MOE_INVALID_ARG);
  expect("dispatch H%128", moe_dispatch_layout(ip, u8, f32, 64, 2, 4, 200, 0, 128, 640, wp, wp,
                                               wp, wp, wp, u8, f32, p, wsb, wp, nullptr),
         MOE_UNSUPPORTED_SHAPE);
  expect("dispatch small workspace", moe_dispatch_layout(ip, u8, f32, 64, 2, 4, 256, 0, 128, 640,
                                                         wp, wp, wp, wp, wp, u8, f32, p, wsb - 4,
                                                         wp, nullptr), MOE_INVALID_ARG);
  expect("dispatch null counts", moe_dispatch_layout(ip, u8, f32, 64, 2, 4, 256, 0, 128, 640,
                                                     nullptr, wp, wp, wp, wp, u8, f32, p, wsb, wp,
                                                     nullptr), MOE_INVALID_ARG);
  expect("dispatch misaligned x", moe_dispatch_layout(ip, static_cast<uint8_t*>(odd), f32, 64, 2,
                                                      4, 256, 0, 128, 640, wp, wp, wp, wp, wp,
                                                      u8, f32, p, wsb, wp, nullptr),
         MOE_UNSUPPORTED_SHAPE);
  expect("dispatch_e8m0 H%128", moe_dispatch_layout_e8m0(ip, u8, u32, 64, 2, 4, 200, 0, 128, 640,
                                                         wp, wp, wp, wp, wp, u8, u32, p, wsb, wp,
                                                         nullptr), MOE_UNSUPPORTED_SHAPE);
  expect("noalloc beyond scratch", moe_dispatch_layout_noalloc(ip, u8, f32, 1 << 24, 8, 32, 256, 0,
                                                               128, 640, wp, wp, wp, wp, wp, u8,
                                                               f32, wp, nullptr),
         MOE_SCRATCH_LIMIT);
  expect("noalloc K too large", moe_dispatch_layout_noalloc(ip, u8, f32, 64, 1000, 4, 256, 0, 128,
                                                            640, wp, wp, wp, wp, wp, u8, f32, wp,
                                                            nullptr), MOE_INVALID_ARG);

  // grouped GEMM: a, a_scale, w, w_scale, offsets, counts, E, rows, N, K, c, status, stream
  expect("gemm E=0", moe_grouped_gemm_fp8(u8, f32, u8, f32, ip, ip, 0, 256, 256, 256, u16, wp,
                                          nullptr), MOE_INVALID_ARG);
  expect("gemm N%128", moe_grouped_gemm_fp8(u8, f32, u8, f32, ip, ip, 4, 256, 200, 256, u16, wp,
                                            nullptr), MOE_UNSUPPORTED_SHAPE);
  expect("gemm K%128", moe_grouped_gemm_fp8(u8, f32, u8, f32, ip, ip, 4, 256, 256, 200, u16, wp,
                                            nullptr), MOE_UNSUPPORTED_SHAPE);
  expect("gemm no rows", moe_grouped_gemm_fp8(u8, f32, u8, f32, ip, ip, 4, 0, 256, 256, u16, wp,
                                              nullptr), MOE_OK);
  expect("gemm null offsets", moe_grouped_gemm_fp8(u8, f32, u8, f32, nullptr, ip, 4, 256, 256,
                                                   256, u16, wp, nullptr), MOE_INVALID_ARG);
  expect("gemm misaligned", moe_grouped_gemm_fp8(static_cast<uint8_t*>(odd), f32, u8, f32, ip,
                                                 ip, 4, 256, 256, 256, u16, wp, nullptr),
         MOE_UNSUPPORTED_SHAPE);
  expect("gemm scale span", moe_grouped_gemm_fp8(u8, f32, u8, f32, ip, ip, 4, 0x7ffff000 / 224 + 1,
                                                 4096, 7168, u16, wp, nullptr),
         MOE_UNSUPPORTED_SHAPE);
  expect("gemm_e8m0 K%128", moe_grouped_gemm_fp8_e8m0(u8, u32, u8, u32, ip, ip, 4, 256, 256, 200,
                                                      u16, wp, nullptr), MOE_UNSUPPORTED_SHAPE);
  expect("gather null row_src", moe_grouped_gemm_fp8_gather(u8, 64, nullptr, f32, u8, f32, ip, ip,
                                                            4, 256, 256, 256, u16, wp, nullptr),
         MOE_INVALID_ARG);
  expect("gather x span", moe_grouped_gemm_fp8_gather(u8, 0x7ffff000 / 7168 + 1, ip, f32, u8, f32,
                                                      ip, ip, 4, 256, 4096, 7168, u16, wp,
                                                      nullptr), MOE_UNSUPPORTED_SHAPE);
  expect("gather_e8m0 T<0", moe_grouped_gemm_fp8_gather_e8m0(u8, -1, ip, u32, u8, u32, ip, ip, 4,
                                                             256, 256, 256, u16, wp, nullptr),
         MOE_INVALID_ARG);

  // gate/up + activation: a, a_scale, w13, w13_scale, offsets, counts, E, rows, I, H, q2, q2s, st
  expect("fused I%128", moe_gate_up_act_fp8(u8, f32, u8, f32, ip, ip, 4, 256, 200, 256, u8, f32,
                                            wp, nullptr), MOE_UNSUPPORTED_SHAPE);
  expect("fused W13 span", moe_gate_up_act_fp8(u8, f32, u8, f32, ip, ip, 4, 256, 1 << 20, 1024, u8,
                                               f32, wp, nullptr), MOE_UNSUPPORTED_SHAPE);
  expect("fused no rows", moe_gate_up_act_fp8(u8, f32, u8, f32, ip, ip, 4, 0, 256, 256, u8, f32,
                                              wp, nullptr), MOE_OK);
  expect("fused_e8m0 null q2", moe_gate_up_act_fp8_e8m0(u8, u32, u8, u32, ip, ip, 4, 256, 256, 256,
                                                        nullptr, u32, wp, nullptr),
         MOE_INVALID_ARG);
  expect("fused gather null x", moe_gate_up_act_fp8_gather(nullptr, 64, ip, f32, u8, f32, ip, ip,
                                                           4, 256, 256, 256, u8, f32, wp, nullptr),
         MOE_INVALID_ARG);
  expect("fused gather_e8m0 x span", moe_gate_up_act_fp8_gather_e8m0(
             u8, 0x7ffff000 / 7168 + 1, ip, u32, u8, u32, ip, ip, 4, 256, 2048, 7168, u8, u32, wp,
             nullptr), MOE_UNSUPPORTED_SHAPE);

  // activation: h, offsets, counts, E, rows, I, q, q_scale, status, stream
  expect("act I%128", moe_act_requant(u16, ip, ip, 4, 256, 200, u8, f32, wp, nullptr),
         MOE_UNSUPPORTED_SHAPE);
  expect("act no rows", moe_act_requant(u16, ip, ip, 4, 0, 256, u8, f32, wp, nullptr), MOE_OK);
  expect("act_e8m0 E=0", moe_act_requant_e8m0(u16, ip, ip, 0, 256, 256, u8, u32, wp, nullptr),
         MOE_INVALID_ARG);

  // combine: y, rows, slot_of, topk_w, T, K, H, out, status, stream
  expect("combine K=0", moe_combine(u16, 256, ip, f32, 64, 0, 256, u16, wp, nullptr),
         MOE_INVALID_ARG);
  expect("combine H%128", moe_combine(u16, 256, ip, f32, 64, 2, 200, u16, wp, nullptr),
         MOE_UNSUPPORTED_SHAPE);
  expect("combine no tokens", moe_combine(u16, 256, ip, f32, 0, 2, 256, u16, wp, nullptr), MOE_OK);

  // quantiser and dense GEMM
  expect("quant block", moe_quantize_fp8(p, 0, 256, 256, 7, u8, f32, nullptr), MOE_INVALID_ARG);
  expect("quant rows", moe_quantize_fp8(p, 0, 200, 256, 128, u8, f32, nullptr),
         MOE_UNSUPPORTED_SHAPE);
  expect("quant empty", moe_quantize_fp8(p, 0, 0, 256, 1, u8, f32, nullptr), MOE_OK);
  expect("quant_e8m0 flag", moe_quantize_fp8_e8m0(p, 2, 256, 256, 1, u8, u32, nullptr),
         MOE_INVALID_ARG);
  expect("dense M<0", moe_gemm_fp8(u8, f32, u8, f32, -1, 256, 256, u16, nullptr), MOE_INVALID_ARG);
  expect("dense empty", moe_gemm_fp8(u8, f32, u8, f32, 0, 256, 256, u16, nullptr), MOE_OK);

  // measurement helpers
  expect("copy misaligned size", moe_ceiling_copy(p, p, 17, nullptr), MOE_INVALID_ARG);
  expect("copy empty", moe_ceiling_copy(p, p, 0, nullptr), MOE_OK);
  double flops = 0;
  expect("mfma chain args", moe_ceiling_mfma_fp8(0, 10, f32, &flops, nullptr), MOE_INVALID_ARG);

  std::printf("host checks: %d failures\n", failures);
  return failures;
}
