// Combine: every source token gathers its expert output rows and sums them
// with its top-k weights — the return half of DeepEP's token shuffle
// ("Deploying DeepSeek with PD Disaggregation and Large-Scale Expert
// Parallelism on 96 H100 GPUs", section 大规模专家并行 › 基于 DeepEP 的专家并行),
// here on the rows this GPU's experts produced.
//
// One workgroup per token, 128 threads; each thread owns 8-column slices
// (16-byte loads of bf16) spaced 1024 columns apart and sums the token's
// rows into fp32 registers in ascending k, so the result is deterministic
// (pure gather, no atomics).  Reads y once per routed row and writes out
// once per token: bound by HBM bandwidth.
#include "device_common.hpp"

namespace moe {

constexpr int kCombThreads = 128;
constexpr int kCombSlices = 8;   // slices of 8 columns per thread per pass

__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const uint16_t* __restrict__ y, int rows_total,
    const int32_t* __restrict__ slot_of, const float* __restrict__ topk_w,
    int T, int K, int H, uint16_t* __restrict__ out,
    int32_t* __restrict__ status) {
  const long long t = blockIdx.x;
  const int n8 = H >> 3;
  int bad = 0;
  for (int base = 0; base < n8; base += kCombThreads * kCombSlices) {
    float acc[kCombSlices][8];
#pragma unroll
    for (int u = 0; u < kCombSlices; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int s = slot_of[t * K + k];
      if (s < 0) continue;
      if (s >= rows_total) { bad = 1; continue; }
      const float w = topk_w[t * K + k];
      const uint4* row = reinterpret_cast<const uint4*>(y + (size_t)s * H);
      uint4 v[kCombSlices];
#pragma unroll
      for (int u = 0; u < kCombSlices; ++u) {
        int c = base + u * kCombThreads + threadIdx.x;
        if (c < n8) v[u] = row[c];
      }
#pragma unroll
      for (int u = 0; u < kCombSlices; ++u) {
        const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[u][2 * i] = fmaf(w, bf16_to_f32(wd[i] & 0xffffu), acc[u][2 * i]);
          acc[u][2 * i + 1] = fmaf(w, bf16_to_f32(wd[i] >> 16), acc[u][2 * i + 1]);
        }
      }
    }
    uint4* orow = reinterpret_cast<uint4*>(out + t * H);
#pragma unroll
    for (int u = 0; u < kCombSlices; ++u) {
      int c = base + u * kCombThreads + threadIdx.x;
      if (c < n8) {
        uint4 o;
        o.x = f32_to_bf16(acc[u][0]) | ((uint32_t)f32_to_bf16(acc[u][1]) << 16);
        o.y = f32_to_bf16(acc[u][2]) | ((uint32_t)f32_to_bf16(acc[u][3]) << 16);
        o.z = f32_to_bf16(acc[u][4]) | ((uint32_t)f32_to_bf16(acc[u][5]) << 16);
        o.w = f32_to_bf16(acc[u][6]) | ((uint32_t)f32_to_bf16(acc[u][7]) << 16);
        orow[c] = o;
      }
    }
  }
  if (bad && threadIdx.x == 0) atomicOr(status, MOE_ERR_BAD_INDEX);
}

}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_combine(const uint16_t* y, int rows_total,
                                    const int32_t* slot_of, const float* topk_w,
                                    int T, int K, int H, uint16_t* out,
                                    int32_t* status_dev, void* stream) {
  if (T < 0 || K <= 0 || K > MOE_MAX_TOPK || H <= 0 || rows_total < 0)
    return MOE_INVALID_ARG;
  if (H % kBlock != 0) return MOE_UNSUPPORTED_SHAPE;
  if (T == 0) return MOE_OK;
  if (!slot_of || !topk_w || !out || !status_dev) return MOE_INVALID_ARG;
  if (rows_total > 0 && !y) return MOE_INVALID_ARG;
  if (((uintptr_t)y | (uintptr_t)out) & 15) return MOE_UNSUPPORTED_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(kCombThreads), 0, st, y,
                     rows_total, slot_of, topk_w, T, K, H, out, status_dev);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
