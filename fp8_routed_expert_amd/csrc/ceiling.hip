// Measured ceilings of the two resources the layer's kernels are bound by,
// so that the benchmark can report each kernel against what this GPU
// actually sustains as well as against the published peaks:
//   * HBM: a plain device-to-device copy, one 16-byte load and one 16-byte
//     store per lane, grid-stride;
//   * FP8 matrix cores: a register-only chain of the E4M3 16x16x128 MFMA
//     the GEMMs use, eight independent accumulators per wave so that the
//     matrix core never waits on a result.
// Neither is part of the layer; both only time the hardware.
#include "device_common.hpp"

namespace moe {

typedef int v8i_c __attribute__((ext_vector_type(8)));
typedef float v4f_c __attribute__((ext_vector_type(4)));

constexpr int kCeilThreads = 256;

__global__ __launch_bounds__(kCeilThreads) void copy_kernel(const uint4* __restrict__ src,
                                                            uint4* __restrict__ dst,
                                                            long long n16) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

__global__ __launch_bounds__(kCeilThreads) void mfma_chain_kernel(int iters, float* __restrict__ sink) {
  // operands from the thread id, so nothing folds at compile time
  v8i_c a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)(threadIdx.x * 0x01010101u + i * 0x11u) & 0x3b3b3b3b;
    b[i] = (int)(blockIdx.x * 0x01010101u + i * 0x07u) & 0x3b3b3b3b;
  }
  v4f_c c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = (v4f_c){0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[j], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  if (s == 1234.5f) sink[blockIdx.x] = s;   // practically never; keeps the chain live
}

}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || (bytes & 15) || (((uintptr_t)src | (uintptr_t)dst) & 15))
    return MOE_INVALID_ARG;
  const long long n16 = (long long)(bytes >> 4);
  if (n16 == 0) return MOE_OK;
  long long blocks = (n16 + kCeilThreads - 1) / kCeilThreads;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCeilThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(src),
                     reinterpret_cast<uint4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}

extern "C" moe_status_t moe_ceiling_mfma_fp8(int workgroups, int iters, float* sink,
                                             double* flops, void* stream) {
  if (workgroups <= 0 || iters <= 0 || !sink) return MOE_INVALID_ARG;
  hipLaunchKernelGGL(mfma_chain_kernel, dim3((unsigned)workgroups), dim3(kCeilThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), iters, sink);
  if (flops) *flops = (double)workgroups * (kCeilThreads / 64) * 8.0 * iters * (2.0 * 16 * 16 * 128);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
