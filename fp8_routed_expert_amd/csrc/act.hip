// SiLU(gate) * up with re-quantisation to E4M3 and fresh 1x128 scales,
// between the two grouped GEMMs of the routed-expert FFN.  The pages name
// the FP8 GEMMs and their quantised input scales ("Deploying DeepSeek on
// GB200 NVL72 with PD and Large Scale EP (Part I)", section 方法实现细节) but
// not the activation; SiLU-gated FFN with gate rows first is the reading.
//
// One workgroup per permuted row; each lane holds 8 consecutive columns, so
// 16 lanes hold one 128-wide scale block and the block amax is a 4-step
// butterfly inside the 16-lane group.  Reads 4 bytes and writes 1 byte per
// element: bound by HBM bandwidth.
#include "device_common.hpp"

namespace moe {

constexpr int kActThreads = 256;

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

__global__ __launch_bounds__(kActThreads) void act_requant_kernel(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ counts, int E, int rows_total, int I,
    uint8_t* __restrict__ q, float* __restrict__ q_scale) {
  const int m = blockIdx.x;
  // is m a valid row?  binary search for the last segment start <= m
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= m) lo = mid; else hi = mid - 1;
  }
  int s, en;
  expert_rows(offsets, counts, lo, rows_total, s, en);
  if (m < s || m >= en) return;

  const uint16_t* hrow = h + (size_t)m * 2 * I;
  uint8_t* qrow = q + (size_t)m * I;
  for (int j0 = threadIdx.x * 8; j0 < I; j0 += kActThreads * 8) {
    uint4 gv = *reinterpret_cast<const uint4*>(hrow + j0);
    uint4 uv = *reinterpret_cast<const uint4*>(hrow + I + j0);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = silu_mul(bf16_to_f32(gw[i] & 0xffffu), bf16_to_f32(uw[i] & 0xffffu));
      v[2 * i + 1] = silu_mul(bf16_to_f32(gw[i] >> 16), bf16_to_f32(uw[i] >> 16));
      amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
    }
    amax = group16_max(amax);
    const float sc = block_scale(amax);
    uint2 out;
    out.x = pack2_e4m3(v[0] / sc, v[1] / sc) | (pack2_e4m3(v[2] / sc, v[3] / sc) << 16);
    out.y = pack2_e4m3(v[4] / sc, v[5] / sc) | (pack2_e4m3(v[6] / sc, v[7] / sc) << 16);
    *reinterpret_cast<uint2*>(qrow + j0) = out;
    if ((threadIdx.x & 15) == 0) q_scale[(size_t)(j0 / kBlock) * rows_total + m] = sc;
  }
}

}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_act_requant(const uint16_t* h, const int32_t* offsets,
                                        const int32_t* counts, int E,
                                        int rows_total, int I, uint8_t* q,
                                        float* q_scale, int32_t* status_dev,
                                        void* stream) {
  (void)status_dev;
  if (E <= 0 || E > MOE_MAX_EXPERTS || rows_total < 0 || I <= 0) return MOE_INVALID_ARG;
  if (I % kBlock != 0) return MOE_UNSUPPORTED_SHAPE;
  if (!offsets || !counts) return MOE_INVALID_ARG;
  if (rows_total == 0) return MOE_OK;
  if (!h || !q || !q_scale) return MOE_INVALID_ARG;
  if (((uintptr_t)h | (uintptr_t)q) & 15) return MOE_UNSUPPORTED_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(act_requant_kernel, dim3((unsigned)rows_total), dim3(kActThreads),
                     0, st, h, offsets, counts, E, rows_total, I, q, q_scale);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
