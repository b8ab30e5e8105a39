// Device-side helpers shared by the gfx950 kernels of libmoe_fp8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_fp8.h"

namespace moe {

constexpr int kBlock = 128;       // scale block width (1x128 / 128x128)
constexpr float kE4M3Max = 448.0f;

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Saturate to the E4M3 range; NaN passes through (comparisons are false).
__device__ __forceinline__ float sat_e4m3(float v) {
  v = v > kE4M3Max ? kE4M3Max : v;
  v = v < -kE4M3Max ? -kE4M3Max : v;
  return v;
}

// Two fp32 values -> two E4M3 codes in the low 16 bits (a in byte 0, b in
// byte 1).  The gfx950 conversion rounds to nearest even in the default
// rounding mode; inputs are saturated first so no out-of-range value
// reaches it.
__device__ __forceinline__ uint32_t pack2_e4m3(float a, float b) {
  return static_cast<uint32_t>(
             __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false)) &
         0xffffu;
}

// Lane permutation inside rows of 16 lanes (DPP control word kCtrl).
template <int kCtrl>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

// Maximum over an aligned group of 16 lanes (one 128-wide block held as 8
// values per lane), left in every lane of the group.  Lanes are swapped in
// pairs, then pairs of pairs (quad permutations 1032 and 2301), then each
// 8-lane half is mirrored onto itself and the 16-lane row onto itself, so
// every lane has met all 16 values.  All 16 lanes must be active.
__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, dpp_row<0xb1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_row<0x4e>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_row<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_row<0x140>(v));   // row_mirror
  return v;
}

// Power-of-two block scale (E8M0): the exponent e of the smallest power of
// two not below fp32(amax / 448), from the bits of that correctly rounded
// quotient: 1.M x 2^(E-127) needs E - 127 when M == 0 and E - 126
// otherwise; a subnormal quotient M x 2^-149 needs -126 above 2^-127 and
// is clamped to the E8M0 minimum -127 at or below it.  An all-zero block
// takes e = 0 (scale 1).
__device__ __forceinline__ int e8m0_exponent(float amax) {
  if (amax == 0.0f) return 0;
  const uint32_t b = __float_as_uint(amax / kE4M3Max);
  const uint32_t E = (b >> 23) & 0xffu, M = b & 0x7fffffu;
  if (E == 0) return M > (1u << 22) ? -126 : -127;
  return (int)E - (M == 0 ? 127 : 126);
}

// 2^-e as an fp32 value (exact for e in [-127, 127]).
__device__ __forceinline__ float e8m0_inverse(int e) {
  return e >= 127 ? __uint_as_float(0x00400000u)          // 2^-127 (subnormal)
                  : __uint_as_float((uint32_t)(127 - e) << 23);
}

// Block scale for a 128-wide block with absolute maximum amax (>= 0).
__device__ __forceinline__ float block_scale(float amax) {
  return amax == 0.0f ? 1.0f : amax / kE4M3Max;
}

// silu(g) * u in fp32: exp(-g) as the hardware base-2 exponential of
// -g log2(e), and the hardware reciprocal (each good to about 1 ulp).
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// v / s correctly rounded, from y = RN(1/s): q0 = RN(v y) is within an ulp,
// the residual v - s q0 is then exact in one fma, and q0 + residual * y
// rounds to the correctly rounded quotient (Markstein's division theorem).
// Exactness of the residual needs its bits above the fp32 underflow range;
// for s >= 2^-90 that holds whenever |v / s| >= 2^-11, and smaller quotients
// encode to zero in E4M3 either way.  Smaller scales take a real division.
__device__ __forceinline__ float div_scale(float v, float s, float y) {
  const float q0 = v * y;
  const float r = fmaf(-s, q0, v);
  return fmaf(r, y, q0);
}

// Eight values of one 1x128 block, whose |max| over the whole block is
// amax, to E4M3 codes (little-endian in out).  Returns the block's scale:
// fp32 s = amax / 448 (bits), or with kPow2 the biased E8M0 exponent byte.
// Shared by the stand-alone activation kernel and the fused gate/up
// epilogue, so both produce the same codes.
template <bool kPow2>
__device__ __forceinline__ uint32_t requant8(const float v[8], float amax, uint2& out) {
  if (kPow2) {
    const int e = e8m0_exponent(amax);
    const float inv = e8m0_inverse(e);
    out.x = pack2_e4m3(v[0] * inv, v[1] * inv) | (pack2_e4m3(v[2] * inv, v[3] * inv) << 16);
    out.y = pack2_e4m3(v[4] * inv, v[5] * inv) | (pack2_e4m3(v[6] * inv, v[7] * inv) << 16);
    return (uint32_t)(e + 127);
  }
  const float sc = block_scale(amax);
  float qv[8];
  if (sc >= 0x1p-90f) {
    const float y = 1.0f / sc;
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = div_scale(v[i], sc, y);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = v[i] / sc;
  }
  out.x = pack2_e4m3(qv[0], qv[1]) | (pack2_e4m3(qv[2], qv[3]) << 16);
  out.y = pack2_e4m3(qv[4], qv[5]) | (pack2_e4m3(qv[6], qv[7]) << 16);
  return __float_as_uint(sc);
}

// Valid row range of expert e: [start, end) inside the segment and buffer.
// Whatever offsets and counts hold, the range is clipped to the buffer, so
// callers never index out of bounds (segments_bad() below detects a table
// that does not describe segments).
__device__ __forceinline__ void expert_rows(const int32_t* offsets,
                                            const int32_t* counts, int e,
                                            int rows_total, int& start,
                                            int& end) {
  int o0 = offsets[e];
  int o1 = offsets[e + 1];
  int c = counts[e];
  long long s = o0 < 0 ? 0 : o0;
  if (s > rows_total) s = rows_total;
  long long lim = (long long)o0 + (c < 0 ? 0 : c);
  if (lim > o1) lim = o1;
  if (lim > rows_total) lim = rows_total;
  if (lim < s) lim = s;
  start = (int)s;
  end = (int)lim;
}

// Does the segment table fail to describe segments?  True when a start is
// negative, the starts decrease, or a count is negative, for any expert
// handled by this wave (expert base + lane, for base = 0, 64, ...).  A
// segment that reaches past the buffer end is not flagged: that is the
// overflow case of the layout, flagged by the dispatch, and is clipped.
// Wave-uniform result.
__device__ __forceinline__ bool segments_bad(const int32_t* offsets, const int32_t* counts,
                                             int E, int lane) {
  bool bad = false;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    if (e < E) {
      const int o0 = offsets[e], o1 = offsets[e + 1], c = counts[e];
      bad |= o0 < 0 || o1 < o0 || c < 0;
    }
  }
  return __ballot(bad) != 0;
}

}  // namespace moe
