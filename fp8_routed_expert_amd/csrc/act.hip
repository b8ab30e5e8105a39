// SiLU(gate) * up with re-quantisation to E4M3 and fresh 1x128 scales,
// between the two grouped GEMMs of the routed-expert FFN.  The pages name
// the FP8 GEMMs and their quantised input scales ("Deploying DeepSeek on
// GB200 NVL72 with PD and Large Scale EP (Part I)", section 方法实现细节) but
// not the activation; SiLU-gated FFN with gate rows first is the reading.
//
// A flat grid: workgroup (m, y) holds columns [2048 y, 2048 y + 2048) of
// permuted row m, 8 consecutive columns per lane, so 16 lanes hold one
// 128-wide scale block and the block amax is a 4-step butterfly inside the
// 16-lane group.  The gate and up loads are issued first; the check that m
// is a valid row (a short search over the segment starts) runs while they
// are in flight, and only the stores depend on it.  Reads 4 bytes and writes
// ~1 byte per element: bound by HBM bandwidth.
#include "device_common.hpp"

namespace moe {

constexpr int kActThreads = 256;
constexpr int kActCols = kActThreads * 8;   // columns per workgroup

// Is permuted row m inside an expert segment?  Binary search for the last
// segment start <= m, then check that segment's valid range.
__device__ __forceinline__ bool row_valid(const int32_t* offsets, const int32_t* counts,
                                          int E, int rows_total, int m) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= m) lo = mid; else hi = mid - 1;
  }
  int s, en;
  expert_rows(offsets, counts, lo, rows_total, s, en);
  return m >= s && m < en;
}

// kPow2: power-of-two scales stored as E8M0 bytes, four 128-column blocks
// per 32-bit word, words K-block-major ([ceil(I/512), rows_total]).
template <bool kPow2>
__global__ __launch_bounds__(kActThreads) void act_requant_kernel(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ counts, int E, int rows_total, int I,
    uint8_t* __restrict__ q, void* __restrict__ q_scale, int32_t* __restrict__ status) {
  const int m = blockIdx.x;
  // the first workgroup's first wave checks that offsets / counts describe
  // segments (rows are clipped to the buffer whatever they hold)
  if (m == 0 && blockIdx.y == 0 && threadIdx.x < 64 && status &&
      segments_bad(offsets, counts, E, threadIdx.x) && threadIdx.x == 0)
    atomicOr(status, MOE_ERR_BAD_INDEX);
  const int j0 = blockIdx.y * kActCols + threadIdx.x * 8;
  const bool in_row = j0 < I;
  const uint16_t* hrow = h + (size_t)m * 2 * I;
  uint4 gv = make_uint4(0, 0, 0, 0), uv = gv;
  if (in_row) {
    gv = *reinterpret_cast<const uint4*>(hrow + j0);
    uv = *reinterpret_cast<const uint4*>(hrow + I + j0);
  }
  if (!row_valid(offsets, counts, E, rows_total, m)) return;   // uniform
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
  amax = group16_max(amax);   // all 16 lanes of a block share in_row
  if (!in_row) return;
  uint2 out;
  const uint32_t sc = requant8<kPow2>(v, amax, out);
  *reinterpret_cast<uint2*>(q + (size_t)m * I + j0) = out;
  if ((threadIdx.x & 15) != 0) return;
  if (kPow2) {
    const int jb = j0 / kBlock, ib = I / kBlock;
    uint8_t* w = reinterpret_cast<uint8_t*>(q_scale) + ((size_t)(jb >> 2) * rows_total + m) * 4;
    w[jb & 3] = (uint8_t)sc;
    if (jb == ib - 1)
      for (int p = (jb & 3) + 1; p < 4; ++p) w[p] = 127;   // past the last block
  } else {
    reinterpret_cast<uint32_t*>(q_scale)[(size_t)(j0 / kBlock) * rows_total + m] = sc;
  }
}

}  // namespace moe

using namespace moe;

template <bool kPow2>
static moe_status_t act_requant(const uint16_t* h, const int32_t* offsets,
                                const int32_t* counts, int E, int rows_total, int I,
                                uint8_t* q, void* q_scale, int32_t* status, void* stream) {
  if (E <= 0 || E > MOE_MAX_EXPERTS || rows_total < 0 || I <= 0) return MOE_INVALID_ARG;
  if (I % kBlock != 0) return MOE_UNSUPPORTED_SHAPE;
  if (!offsets || !counts) return MOE_INVALID_ARG;
  if (rows_total == 0) return MOE_OK;
  if (!h || !q || !q_scale) return MOE_INVALID_ARG;
  if (((uintptr_t)h | (uintptr_t)q) & 15) return MOE_UNSUPPORTED_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL((act_requant_kernel<kPow2>),
                     dim3((unsigned)rows_total, (unsigned)((I + kActCols - 1) / kActCols)),
                     dim3(kActThreads), 0, st, h, offsets, counts, E, rows_total, I, q,
                     q_scale, status);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}

extern "C" moe_status_t moe_act_requant(const uint16_t* h, const int32_t* offsets,
                                        const int32_t* counts, int E, int rows_total,
                                        int I, uint8_t* q, float* q_scale,
                                        int32_t* status_dev, void* stream) {
  return act_requant<false>(h, offsets, counts, E, rows_total, I, q, q_scale, status_dev,
                            stream);
}

extern "C" moe_status_t moe_act_requant_e8m0(const uint16_t* h, const int32_t* offsets,
                                             const int32_t* counts, int E, int rows_total,
                                             int I, uint8_t* q, uint32_t* q_scale,
                                             int32_t* status_dev, void* stream) {
  return act_requant<true>(h, offsets, counts, E, rows_total, I, q, q_scale, status_dev,
                           stream);
}
