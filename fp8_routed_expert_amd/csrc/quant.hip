// Source-side block quantisation to E4M3 with fp32 scales: the step that
// produces the layer's inputs (activations per 1x128 block before the
// dispatch, weights per 128x128 block offline).  "Deploying DeepSeek on
// GB200 NVL72 with PD and Large Scale EP (Part I)", section 方法实现细节: the
// FP8 GEMM library's API quantises the input scales.
//
//   1x128   : 16 lanes per block, 8 values per lane, butterfly amax.
//   128x128 : one workgroup per block, 64 values per thread, LDS amax.
#include "device_common.hpp"

namespace moe {

template <bool kF32>
__device__ __forceinline__ void load8(const void* x, size_t idx, float v[8]) {
  if (kF32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + idx);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + idx);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
}

__device__ __forceinline__ uint2 quant8(const float v[8], float sc) {
  uint2 o;
  o.x = pack2_e4m3(v[0] / sc, v[1] / sc) | (pack2_e4m3(v[2] / sc, v[3] / sc) << 16);
  o.y = pack2_e4m3(v[4] / sc, v[5] / sc) | (pack2_e4m3(v[6] / sc, v[7] / sc) << 16);
  return o;
}

// grid-stride over 8-element slices; 16 consecutive slices form a block
template <bool kF32>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const void* __restrict__ x,
                                                          long long n_slices, int cols,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ scale) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  // n_slices and the stride are multiples of 16 and a 16-lane group holds 16
  // consecutive slices, so each group is entirely inside or outside the range
  // and its butterfly only reads lanes of its own group.
  for (long long sl = (long long)blockIdx.x * blockDim.x + threadIdx.x; sl < n_slices;
       sl += stride) {
    const bool in = true;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (in) load8<kF32>(x, (size_t)sl * 8, v);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group16_max(amax);
    const float sc = block_scale(amax);
    if (in) {
      *reinterpret_cast<uint2*>(q + (size_t)sl * 8) = quant8(v, sc);
      if ((sl & 15) == 0) scale[sl >> 4] = sc;
    }
  }
}

template <bool kF32>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const void* __restrict__ x,
                                                            int rows, int cols,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  __shared__ float red[4];
  const int cb = cols / kBlock;
  const int rb = blockIdx.x / cb;
  const int kb = blockIdx.x - rb * cb;
  // thread t: column slice (t & 15) * 8, rows (t >> 4) + 16 * i, i < 8
  const int c0 = kb * kBlock + (threadIdx.x & 15) * 8;
  float v[8][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rb * kBlock + (threadIdx.x >> 4) + 16 * i;
    load8<kF32>(x, (size_t)r * cols + c0, v[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
  }
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = block_scale(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rb * kBlock + (threadIdx.x >> 4) + 16 * i;
    *reinterpret_cast<uint2*>(q + (size_t)r * cols + c0) = quant8(v[i], sc);
  }
  if (threadIdx.x == 0) scale[(size_t)rb * cb + kb] = sc;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_quantize_fp8(const void* x, int x_is_f32, int rows, int cols,
                                         int block_rows, uint8_t* q, float* scale,
                                         void* stream) {
  if (rows < 0 || cols <= 0 || (block_rows != 1 && block_rows != kBlock) ||
      (x_is_f32 != 0 && x_is_f32 != 1))
    return MOE_INVALID_ARG;
  if (cols % kBlock != 0 || rows % block_rows != 0) return MOE_UNSUPPORTED_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scale) return MOE_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)q) & 15) return MOE_UNSUPPORTED_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (block_rows == 1) {
    long long n_slices = (long long)rows * cols / 8;
    long long blocks = (n_slices + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (x_is_f32)
      hipLaunchKernelGGL(quant_1x128_kernel<true>, dim3((unsigned)blocks), dim3(256), 0,
                         st, x, n_slices, cols, q, scale);
    else
      hipLaunchKernelGGL(quant_1x128_kernel<false>, dim3((unsigned)blocks), dim3(256), 0,
                         st, x, n_slices, cols, q, scale);
  } else {
    long long blocks = (long long)(rows / kBlock) * (cols / kBlock);
    if (blocks > 0x7fffffffLL) return MOE_UNSUPPORTED_SHAPE;
    if (x_is_f32)
      hipLaunchKernelGGL(quant_128x128_kernel<true>, dim3((unsigned)blocks), dim3(256), 0,
                         st, x, rows, cols, q, scale);
    else
      hipLaunchKernelGGL(quant_128x128_kernel<false>, dim3((unsigned)blocks), dim3(256), 0,
                         st, x, rows, cols, q, scale);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
