// Combine: every source token gathers its expert output rows and sums them
// with its top-k weights — the return half of DeepEP's token shuffle
// ("Deploying DeepSeek with PD Disaggregation and Large-Scale Expert
// Parallelism on 96 H100 GPUs", section 大规模专家并行 › 基于 DeepEP 的专家并行),
// here on the rows this GPU's experts produced.
//
// One workgroup per token, sized so that each thread owns two 8-column
// slices (16-byte loads of bf16) of the row (448 threads for H = 7168).  The
// token's K slots and weights arrive in one vector load; the thread sums the
// valid rows into fp32 registers in ascending k, two rows' loads in flight at
// a time, so the result is deterministic (pure gather, no atomics).  Reads y
// once per routed row and writes out once per token: bound by HBM bandwidth.
#include "device_common.hpp"

namespace moe {

constexpr int kCombMaxThreads = 512;
constexpr int kCombSlices = 2;   // slices of 8 columns per thread per pass

__device__ __forceinline__ void accumulate8(float (&acc)[8], float w, const uint4& v) {
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, bf16_to_f32(wd[i] & 0xffffu), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, bf16_to_f32(wd[i] >> 16), acc[2 * i + 1]);
  }
}

// Loads this thread's 16-byte slices of row `slot` (slice index base +
// u * blockDim + tid; slices past the row re-read slice 0, never stored).
__device__ __forceinline__ void load_slices(const uint16_t* y, int H, int slot, int base,
                                            int n8, uint4 (&v)[kCombSlices]) {
  const uint4* r = reinterpret_cast<const uint4*>(y + (size_t)slot * H);
#pragma unroll
  for (int u = 0; u < kCombSlices; ++u) {
    const int c = base + u * (int)blockDim.x + threadIdx.x;
    v[u] = r[c < n8 ? c : 0];
  }
}

__global__ __launch_bounds__(kCombMaxThreads) void combine_kernel(
    const uint16_t* __restrict__ y, int rows_total,
    const int32_t* __restrict__ slot_of, const float* __restrict__ topk_w,
    int T, int K, int H, uint16_t* __restrict__ out,
    int32_t* __restrict__ status) {
  const long long t = blockIdx.x;
  const int n8 = H >> 3;
  // lane k of every wave holds pick k's slot and weight; the rows to sum are
  // the set bits of `valid`, walked in ascending k with uniform lane reads
  const int lane = threadIdx.x & 63;
  int s = -1;
  float w = 0.f;
  if (lane < K) {
    s = slot_of[t * K + lane];
    w = topk_w[t * K + lane];
  }
  const unsigned long long valid = __ballot(s >= 0 && s < rows_total);
  const bool bad = __ballot(s >= rows_total) != 0;
  for (int base = 0; base < n8; base += (int)blockDim.x * kCombSlices) {
    float acc[kCombSlices][8];
#pragma unroll
    for (int u = 0; u < kCombSlices; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
    unsigned long long m = valid;
    while (m) {
      const int k0 = __ffsll((long long)m) - 1;
      m &= m - 1;
      const int s0 = __builtin_amdgcn_readlane(s, k0);
      const float w0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k0));
      uint4 v0[kCombSlices];
      load_slices(y, H, s0, base, n8, v0);
      if (m) {   // a second row, loaded before either is summed
        const int k1 = __ffsll((long long)m) - 1;
        m &= m - 1;
        const int s1 = __builtin_amdgcn_readlane(s, k1);
        const float w1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k1));
        uint4 v1[kCombSlices];
        load_slices(y, H, s1, base, n8, v1);
#pragma unroll
        for (int u = 0; u < kCombSlices; ++u) accumulate8(acc[u], w0, v0[u]);
#pragma unroll
        for (int u = 0; u < kCombSlices; ++u) accumulate8(acc[u], w1, v1[u]);
      } else {
#pragma unroll
        for (int u = 0; u < kCombSlices; ++u) accumulate8(acc[u], w0, v0[u]);
      }
    }
    uint4* orow = reinterpret_cast<uint4*>(out + t * H);
#pragma unroll
    for (int u = 0; u < kCombSlices; ++u) {
      const int c = base + u * (int)blockDim.x + threadIdx.x;
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
  // one pass over the row when it fits: ceil(H/8 / slices) lanes, whole waves
  const int n8 = H / 8;
  int threads = ((n8 + kCombSlices - 1) / kCombSlices + 63) / 64 * 64;
  if (threads > kCombMaxThreads) threads = kCombMaxThreads;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(threads), 0, st, y,
                     rows_total, slot_of, topk_w, T, K, H, out, status_dev);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
