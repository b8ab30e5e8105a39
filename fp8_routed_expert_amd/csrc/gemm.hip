// Block-scaled FP8 (E4M3) grouped GEMM over the expert segments of the
// permuted buffer: the MoE grouped GEMMs of "Deploying DeepSeek with PD
// Disaggregation and Large-Scale Expert Parallelism on 96 H100 GPUs"
// (section 大规模专家并行 › DeepGEMM 集成), whose GB200 rewrite ("Deploying
// DeepSeek on GB200 NVL72 with PD and Large Scale EP (Part I)", section
// 方法实现细节) takes quantised input scales.  The Blackwell UMMA/TMA design
// there is prior art; this kernel is written for CDNA4's matrix cores.
//
//   c[m, n] = bf16( sum_kb sa[kb, m] * sw[e, n/128, kb]
//                         * sum_{k in kb} a[m, k] * w[e, n, k] )
//
// Design (gfx950):
//   * one workgroup = 256 threads = 4 waves computes a 128x128 tile of c;
//     each wave owns 64x64 = 4x4 MFMA subtiles of 16x16.
//   * K advances one 128-wide scale block per step.  v_mfma_f32_16x16x128
//     _f8f6f4 consumes exactly one block per subtile, so each block's raw
//     fp32 product comes out of a single MFMA (issued with a zero
//     accumulator) and is promoted into the fp32 accumulator with one FMA by
//     sa * sw — the scale application the pages put in the epilogue,
//     applied per block as the block-scaled format requires.
//   * A and B tiles (128 rows x 128 bytes each) are double-buffered in LDS;
//     the next block's global loads are in flight while the current block is
//     multiplied.  16-byte chunks are XOR-swizzled by (row & 7) so that the
//     fragment reads of 8 consecutive rows hit 8 distinct bank groups.
//   * tiles are assigned from device-side offsets/counts: m-tiles are
//     numbered expert by expert (ceil(valid rows / 128) per expert), so the
//     grid is fixed by the buffer size alone (floor(rows/128) + E m-tiles)
//     and blocks past the last real tile exit at once.  Nothing is read back
//     on the host, so the launch can be captured in a hipGraph.
#include "device_common.hpp"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kThreads = 256;

__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // format 0 = E4M3 for both operands; zero scale operands select the plain
  // (unscaled) instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0,
                                                          0, 0);
}

__device__ __forceinline__ v8i load_frag(const uint8_t* tile, int row, int g) {
  const uint8_t* base = tile + row * kBK;
  const int sw = row & 7;
  uint4 lo = *reinterpret_cast<const uint4*>(base + (((2 * g) ^ sw) << 4));
  uint4 hi = *reinterpret_cast<const uint4*>(base + (((2 * g + 1) ^ sw) << 4));
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__global__ __launch_bounds__(kThreads) void grouped_gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA,
    const uint8_t* __restrict__ W, const float* __restrict__ SW,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ counts,
    int E, int rows_total, int N, int K, uint16_t* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kBN * kBK];
  __shared__ __attribute__((aligned(16))) float sSA[2][kBM];
  __shared__ float sSB[2];

  const int n_tiles = N / kBN;
  const int tile_m = blockIdx.x / n_tiles;
  const int tile_n = blockIdx.x - tile_m * n_tiles;

  // expert and row range of this m-tile
  int e_sel = -1, row0 = 0, row_end = 0;
  {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      int s, en;
      expert_rows(offsets, counts, e, rows_total, s, en);
      int nt = (en - s + kBM - 1) / kBM;
      if (tile_m < acc + nt) {
        e_sel = e;
        row0 = s + (tile_m - acc) * kBM;
        row_end = en;
        break;
      }
      acc += nt;
    }
  }
  if (e_sel < 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int Kb = K / kBK;
  const int nb_w = N / kBlock;

  const uint8_t* Wt = W + ((size_t)e_sel * N + (size_t)tile_n * kBN) * K;
  const float* SWt = SW + ((size_t)e_sel * nb_w + tile_n) * Kb;

  const int ld_row = tid >> 3;
  const int ld_ch = tid & 7;
  // global->LDS staging: thread tid moves 16-byte chunk (tid & 7) of rows
  // (tid >> 3) + 32 i, i < 4, of both tiles (explicit registers, no arrays,
  // so nothing is placed in scratch memory)
#define MOE_ROW_PTRS(i)                                                        \
  const uint8_t* a_src##i;                                                     \
  const uint8_t* b_src##i;                                                     \
  {                                                                            \
    int r = row0 + ld_row + 32 * i;                                            \
    r = r < rows_total ? r : rows_total - 1;                                   \
    a_src##i = A + (size_t)r * K + ld_ch * 16;                                 \
    b_src##i = Wt + (size_t)(ld_row + 32 * i) * K + ld_ch * 16;                \
  }
  MOE_ROW_PTRS(0)
  MOE_ROW_PTRS(1)
  MOE_ROW_PTRS(2)
  MOE_ROW_PTRS(3)
#undef MOE_ROW_PTRS
  int sa_row = row0 + (tid & (kBM - 1));
  sa_row = sa_row < rows_total ? sa_row : rows_total - 1;

  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  float rsa = 0.f, rsb = 0.f;
#define MOE_GLOAD(kb)                                                          \
  do {                                                                         \
    const size_t ko = (size_t)(kb) * kBK;                                      \
    ra0 = *reinterpret_cast<const uint4*>(a_src0 + ko);                        \
    ra1 = *reinterpret_cast<const uint4*>(a_src1 + ko);                        \
    ra2 = *reinterpret_cast<const uint4*>(a_src2 + ko);                        \
    ra3 = *reinterpret_cast<const uint4*>(a_src3 + ko);                        \
    rb0 = *reinterpret_cast<const uint4*>(b_src0 + ko);                        \
    rb1 = *reinterpret_cast<const uint4*>(b_src1 + ko);                        \
    rb2 = *reinterpret_cast<const uint4*>(b_src2 + ko);                        \
    rb3 = *reinterpret_cast<const uint4*>(b_src3 + ko);                        \
    if (tid < kBM) rsa = SA[(size_t)(kb) * rows_total + sa_row];               \
    if (tid == kBM) rsb = SWt[(kb)];                                           \
  } while (0)
#define MOE_ST1(buf, i)                                                        \
  {                                                                            \
    const int row = ld_row + 32 * i;                                           \
    const int off = row * kBK + ((ld_ch ^ (row & 7)) << 4);                    \
    *reinterpret_cast<uint4*>(&sA[(buf)][off]) = ra##i;                        \
    *reinterpret_cast<uint4*>(&sB[(buf)][off]) = rb##i;                        \
  }
#define MOE_SSTORE(buf)                                                        \
  do {                                                                         \
    MOE_ST1(buf, 0) MOE_ST1(buf, 1) MOE_ST1(buf, 2) MOE_ST1(buf, 3)            \
    if (tid < kBM) sSA[(buf)][tid] = rsa;                                      \
    if (tid == kBM) sSB[(buf)] = rsb;                                          \
  } while (0)

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  MOE_GLOAD(0);
  MOE_SSTORE(0);
  __syncthreads();

  const int g = lane >> 4;
  const int r16 = lane & 15;
  for (int kb = 0; kb < Kb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < Kb) MOE_GLOAD(kb + 1);
    v8i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = load_frag(sA[cur], wm * 64 + i * 16 + r16, g);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = load_frag(sB[cur], wn * 64 + j * 16 + r16, g);
    const float sb = sSB[cur];
    float f[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 s4 = *reinterpret_cast<const float4*>(&sSA[cur][wm * 64 + i * 16 + 4 * g]);
      f[i][0] = s4.x * sb;
      f[i][1] = s4.y * sb;
      f[i][2] = s4.z * sb;
      f[i][3] = s4.w * sb;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v4f t = mfma_fp8_16x16x128(af[i], bf[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(t[r], f[i][r], acc[i][j][r]);
      }
    if (kb + 1 < Kb) MOE_SSTORE(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4g..4g+3 of each 16x16 subtile, column r16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int row = row0 + wm * 64 + i * 16 + 4 * g + r;
      if (row < row_end) {
        uint16_t* crow = C + (size_t)row * N + (size_t)tile_n * kBN + wn * 64 + r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) crow[j * 16] = f32_to_bf16(acc[i][j][r]);
      }
    }
#undef MOE_GLOAD
#undef MOE_ST1
#undef MOE_SSTORE
}

}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_grouped_gemm_fp8(
    const uint8_t* a, const float* a_scale, const uint8_t* w,
    const float* w_scale, const int32_t* offsets, const int32_t* counts, int E,
    int rows_total, int N, int K, uint16_t* c, int32_t* status_dev,
    void* stream) {
  (void)status_dev;
  if (E <= 0 || E > MOE_MAX_EXPERTS || rows_total < 0 || N <= 0 || K <= 0)
    return MOE_INVALID_ARG;
  if (N % kBN != 0 || K % kBK != 0) return MOE_UNSUPPORTED_SHAPE;
  if (!offsets || !counts || !w || !w_scale) return MOE_INVALID_ARG;
  if (rows_total == 0) return MOE_OK;
  if (!a || !a_scale || !c) return MOE_INVALID_ARG;
  if (((uintptr_t)a | (uintptr_t)w | (uintptr_t)c) & 15)
    return MOE_UNSUPPORTED_SHAPE;
  long long m_tiles = (long long)rows_total / kBM + E;
  long long blocks = m_tiles * (N / kBN);
  if (blocks > 0x7fffffffLL) return MOE_UNSUPPORTED_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(grouped_gemm_fp8_kernel, dim3((unsigned)blocks),
                     dim3(kThreads), 0, st, a, a_scale, w, w_scale, offsets,
                     counts, E, rows_total, N, K, c);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
