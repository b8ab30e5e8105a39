// Source-side block quantisation to E4M3: the step that produces the
// layer's inputs (activations per 1x128 block before the dispatch, weights
// per 128x128 block offline).  "Deploying DeepSeek on GB200 NVL72 with PD
// and Large Scale EP (Part I)", section 方法实现细节: the FP8 GEMM library's
// API quantises and packs the input scales.  Two scale formats: fp32
// s = amax / 448, or a power of two stored as a biased exponent byte
// (E8M0), four 128-wide blocks per 32-bit word along the columns.
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

// Power-of-two scale: v * 2^-e is exact, so a multiply stands in for the
// division.
__device__ __forceinline__ uint2 quant8_pow2(const float v[8], float inv) {
  uint2 o;
  o.x = pack2_e4m3(v[0] * inv, v[1] * inv) | (pack2_e4m3(v[2] * inv, v[3] * inv) << 16);
  o.y = pack2_e4m3(v[4] * inv, v[5] * inv) | (pack2_e4m3(v[6] * inv, v[7] * inv) << 16);
  return o;
}

// Stores the biased exponent byte of block kb of scale row `row` into the
// packed words [.., ceil(nb / 4)] (byte kb % 4 of word kb / 4); the writer
// of a row's last block also sets the bytes past it to 127 (scale 1).
__device__ __forceinline__ void store_e8m0(uint32_t* words, size_t row, int kb, int nb, int e) {
  const int nw = (nb + 3) / 4;
  uint8_t* b = reinterpret_cast<uint8_t*>(words) + row * (size_t)nw * 4;
  b[kb] = (uint8_t)(e + 127);
  if (kb == nb - 1)
    for (int p = nb; p < nw * 4; ++p) b[p] = 127;
}

// grid-stride over 8-element slices; 16 consecutive slices form a block
template <bool kF32, bool kPow2>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const void* __restrict__ x,
                                                          long long n_slices, int cols,
                                                          uint8_t* __restrict__ q,
                                                          void* __restrict__ scale) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  // n_slices and the stride are multiples of 16 and a 16-lane group holds 16
  // consecutive slices, so each group is entirely inside or outside the range
  // and its butterfly only reads lanes of its own group.
  for (long long sl = (long long)blockIdx.x * blockDim.x + threadIdx.x; sl < n_slices;
       sl += stride) {
    float v[8];
    load8<kF32>(x, (size_t)sl * 8, v);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group16_max(amax);
    if (kPow2) {
      const int e = e8m0_exponent(amax);
      *reinterpret_cast<uint2*>(q + (size_t)sl * 8) = quant8_pow2(v, e8m0_inverse(e));
      if ((sl & 15) == 0) {
        const int nb = cols / kBlock;
        const long long blk = sl >> 4;
        store_e8m0(reinterpret_cast<uint32_t*>(scale), (size_t)(blk / nb), (int)(blk % nb), nb, e);
      }
    } else {
      const float sc = block_scale(amax);
      *reinterpret_cast<uint2*>(q + (size_t)sl * 8) = quant8(v, sc);
      if ((sl & 15) == 0) reinterpret_cast<float*>(scale)[sl >> 4] = sc;
    }
  }
}

template <bool kF32, bool kPow2>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const void* __restrict__ x,
                                                            int rows, int cols,
                                                            uint8_t* __restrict__ q,
                                                            void* __restrict__ scale) {
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
  if (kPow2) {
    const int e = e8m0_exponent(amax);
    const float inv = e8m0_inverse(e);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = rb * kBlock + (threadIdx.x >> 4) + 16 * i;
      *reinterpret_cast<uint2*>(q + (size_t)r * cols + c0) = quant8_pow2(v[i], inv);
    }
    if (threadIdx.x == 0) store_e8m0(reinterpret_cast<uint32_t*>(scale), rb, kb, cb, e);
  } else {
    const float sc = block_scale(amax);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = rb * kBlock + (threadIdx.x >> 4) + 16 * i;
      *reinterpret_cast<uint2*>(q + (size_t)r * cols + c0) = quant8(v[i], sc);
    }
    if (threadIdx.x == 0) reinterpret_cast<float*>(scale)[(size_t)rb * cb + kb] = sc;
  }
}

}  // namespace moe

using namespace moe;

template <bool kPow2>
static moe_status_t quantize(const void* x, int x_is_f32, int rows, int cols, int block_rows,
                             uint8_t* q, void* scale, void* stream) {
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
      hipLaunchKernelGGL((quant_1x128_kernel<true, kPow2>), dim3((unsigned)blocks), dim3(256),
                         0, st, x, n_slices, cols, q, scale);
    else
      hipLaunchKernelGGL((quant_1x128_kernel<false, kPow2>), dim3((unsigned)blocks), dim3(256),
                         0, st, x, n_slices, cols, q, scale);
  } else {
    long long blocks = (long long)(rows / kBlock) * (cols / kBlock);
    if (blocks > 0x7fffffffLL) return MOE_UNSUPPORTED_SHAPE;
    if (x_is_f32)
      hipLaunchKernelGGL((quant_128x128_kernel<true, kPow2>), dim3((unsigned)blocks),
                         dim3(256), 0, st, x, rows, cols, q, scale);
    else
      hipLaunchKernelGGL((quant_128x128_kernel<false, kPow2>), dim3((unsigned)blocks),
                         dim3(256), 0, st, x, rows, cols, q, scale);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}

extern "C" moe_status_t moe_quantize_fp8(const void* x, int x_is_f32, int rows, int cols,
                                         int block_rows, uint8_t* q, float* scale,
                                         void* stream) {
  return quantize<false>(x, x_is_f32, rows, cols, block_rows, q, scale, stream);
}

extern "C" moe_status_t moe_quantize_fp8_e8m0(const void* x, int x_is_f32, int rows, int cols,
                                              int block_rows, uint8_t* q, uint32_t* scale,
                                              void* stream) {
  return quantize<true>(x, x_is_f32, rows, cols, block_rows, q, scale, stream);
}
