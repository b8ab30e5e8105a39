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
//   * Large problems: a workgroup computes a 256 x 256 tile of c with 8 waves
//     of 128 x 64 (two waves per SIMD, one workgroup per CU, the full 160 KB
//     of LDS); packed scales at prefill sizes 320 x 256, and decode sizes
//     whose tiles fit one round on the CUs 192 x 256.  Small problems:
//     128 x 128 tiles of 4 waves of 64 x 64, two workgroups per CU (64 x 128
//     for the gate/up projection of the masked decode layout, 128 x 256 for
//     the fused gate/up + activation).  The host picks the shape from the
//     sizes alone (rules beside the tile configurations below).  A wave's
//     sub-tile is a grid of 16 x 16 MFMA subtiles.
//   * K advances one 128-wide scale block per step.  v_mfma_f32_16x16x128
//     _f8f6f4 consumes exactly one block per subtile, so each block's raw
//     product comes out of a single MFMA issued with a zero accumulator and
//     is promoted into the fp32 accumulator with one FMA by the combined
//     scale f = sa[kb, m] * sw[e, nb, kb].  The MFMA computes the transposed
//     product (weights as the first operand), so a lane's four outputs of a
//     subtile are four columns of one row: one row scale per lane.  Each
//     MFMA of subtile row i is followed in issue order by the four FMAs that
//     promote the same column of row i - 1 (whose product is complete), so
//     one wave overlaps its own matrix-core and VALU work; the accumulators
//     stay in VGPRs.
//   * A and B tiles (rows x 128 bytes) go from global memory straight into
//     LDS with buffer_load ... lds (no staging registers).  A has three
//     stages (its k-block kb + 2 is loaded while kb is multiplied), B two
//     (kb + 1); at a 256 x 256 tile that is exactly the 160 KB of LDS.  The
//     third A stage took 2-3% off the prefill gate/up GEMM and 7-20% off the
//     decode ones; a third B stage instead measured slower at prefill.  The
//     row scales (K-block-major, so contiguous per block) go straight to
//     registers one step ahead; the weight-block scale of a wave's columns
//     is a scalar load one step ahead.  Each stage is its own LDS object
//     and the K loop is unrolled by 6, so every access names its stage
//     statically.  The tile and scale loads are issued as inline assembly:
//     the compiler then inserts no waits of its own for them (its
//     conservative tracking of LDS-DMA targets otherwise waited for every
//     load before the next fragment read, serialising the pipeline); they
//     are waited for explicitly with vmcnt, which counts vector-memory
//     operations in issue order, and the step barrier orders LDS only.
//     Inside every 16-row group the 16-byte chunks are XOR-permuted by
//     (row & 7) ^ ((row >> 3) & 1) -- chosen through the per-lane global
//     offset, since each load instruction fills 1 KB of LDS contiguously --
//     which measured free of bank conflicts for the fragment reads (4 LDS
//     cycles per 1 KB read); the (row >> 1) & 7 permutation measured a 2-way
//     conflict.
//   * Tiles come from device-side offsets/counts: m-tiles are numbered
//     expert by expert (ceil(valid rows / BM) per expert), so the grid is
//     fixed by the buffer size alone and workgroups past the last real tile
//     exit at once; nothing is read back on the host and the launch can be
//     captured in a hipGraph.  Buffer descriptors bound every tile load, so
//     rows past the end of the buffer read as zero (and are never stored).
//   * Tile order and the 8 XCDs (each with its own L2): workgroup w runs on
//     XCD w mod 8 and takes tile w of a list ordered in groups of GM m-tiles
//     x all n-tiles (m fastest).  With GM = 2 the 32 tiles one XCD runs at
//     a time are 8 m-tiles x 4 n-tiles (12 distinct panels per 64 panel
//     loads in its L2), and all XCDs work in the same few groups, so the
//     current expert's weights are shared through the memory-side cache.
//     This measured a few percent faster than giving each XCD a contiguous
//     share of the list (XCDs then stream different experts' weights).
#include <type_traits>

#include "device_common.hpp"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 128;
constexpr int kXcds = 8;
constexpr int kLdsBytes = 160 * 1024;   // LDS per workgroup (gfx950)

// Workgroup barrier for the tile pipeline.  __syncthreads() (and even an
// LDS-scoped fence, since loads into LDS count as vector-memory operations)
// makes every wave wait for all its outstanding vector loads -- including
// the tile loads meant to stay in flight across the barrier.  Here the wave
// waits for its own LDS reads (lgkmcnt) and meets the others; completion of
// the tile loads is waited for explicitly with wait_loads<n>() before it.
// Both are compiler memory barriers (asm with a memory clobber), so no
// memory access is moved across them.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef int v4i __attribute__((ext_vector_type(4)));
// Raw buffer descriptor: base, stride 0, num_records bytes (offsets at or
// past it read as zero), 32-bit data format.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  v4i r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)((b >> 32) & 0xffffu);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
  return r;
}
// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane
// (one wave instruction fills 1 KB).  M0 holds the LDS address; nothing else
// in these kernels reads M0 (gfx9 LDS instructions do not use it), so the
// clobber is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(v4i rsrc, uint8_t* lds, uint32_t voff) {
  const uint32_t m = (uint32_t)(uintptr_t)(lds_void*)lds;   // LDS byte offset
  v4i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m), "v"(voff), "s"(r) : "memory", "m0");
}
// The same with the offset split into a per-lane part, XOR-ed with a
// wave-uniform 0 or 16 (the chunk permutation of the odd 8-row half of a
// 16-row group), and a wave-uniform part, combined inside the asm: the
// compiler cannot then hoist one offset register per chunk (or per parity)
// out of the K loop (the address is read when the load issues, so the
// temporary is free right after).
__device__ __forceinline__ void dma16_split(v4i rsrc, uint8_t* lds, uint32_t vlane,
                                            uint32_t sxor, uint32_t suni) {
  const uint32_t m = (uint32_t)(uintptr_t)(lds_void*)lds;
  v4i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  uint32_t t;
  asm volatile("v_xor_b32_e32 %0, %1, %2\n\tv_add_u32_e32 %0, %3, %0\n\ts_mov_b32 m0, %4\n\t"
               "buffer_load_dwordx4 %0, %5, 0 offen lds"
               : "=&v"(t) : "s"(sxor), "v"(vlane), "s"(suni), "s"(m), "s"(r) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory operations of this wave are
// outstanding (they complete in issue order), and publish the registers of
// the asynchronous register loads issued before them (see load_scales).
template <int N, int M>
__device__ __forceinline__ void wait_loads(float (&r)[M]) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
#pragma unroll
  for (int i = 0; i < M; ++i) asm volatile("" : "+v"(r[i]));
}

// Lane l holds the value of row l of a 64-row block; out[k] receives, in
// every lane, the value of row 16k + (lane mod 16) -- row group k
// broadcast to the four groups.  Swapping the upper 32 lanes of one copy
// with the lower 32 of another gives groups (0 1 0 1) and (2 3 2 3);
// swapping odd with even groups of each with itself then gives each group
// in all four positions.
__device__ __forceinline__ void row_scales(float r, float* out) {
  const uint32_t v = __float_as_uint(r);
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  const auto lo = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
  out[0] = __uint_as_float(lo[0]);
  out[1] = __uint_as_float(lo[1]);
  out[2] = __uint_as_float(hi[0]);
  out[3] = __uint_as_float(hi[1]);
}

// The lane's index in its wave, read afresh from the hardware (the asm keeps
// the compiler from reusing, and so keeping live, an earlier copy), so that
// an epilogue need not hold its lane position in a register through the
// whole K loop.
__device__ __forceinline__ int lane_id_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // format 0 = E4M3 for both operands; zero scale operands select the plain
  // (unscaled) instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0,
                                                          0, 0);
}

// Two fp32 values to packed bf16, round to nearest even (one
// v_cvt_pk_bf16_f32; a NaN stays a NaN, its payload is not canonicalised).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Physical position of logical 16-byte chunk c of tile row r: chunks are
// XOR-permuted by (r & 7) ^ ((r >> 3) & 1).  A fragment read has lane
// (q, g) read chunk 2g (then 2g + 1) of row 16 b + q; with this permutation
// the LDS serves it without bank conflicts (4 cycles per 1 KB wave read on
// gfx950, against 8 for the (r >> 1) & 7 and r & 7 permutations).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// A lane's byte offsets, within a stage, of the two 16-byte chunks (logical
// 2g and 2g + 1) it reads from row row0 + r16 of a swizzled tile.  For any
// row0 that is a multiple of 16 the permutation of row row0 + 16 i + r16
// is that of r16, so the fragment of subtile row i lies a fixed 16 i * 128
// bytes further: one pair of offsets serves every subtile of a wave.
struct FragLane {
  uint32_t lo, hi;
};
__device__ __forceinline__ FragLane frag_lane(int row0, int r16, int g) {
  const uint32_t r = (uint32_t)(row0 + r16) * kBK;
  const int sw = swz(r16);
  return {r + (uint32_t)(((2 * g) ^ sw) << 4), r + (uint32_t)(((2 * g + 1) ^ sw) << 4)};
}

// 32 bytes of a fragment: the lane's two chunks, `off` bytes (a multiple of
// 16 rows) past its offsets in stage `tile`.
__device__ __forceinline__ v8i load_frag_at(const uint8_t* tile, int off, FragLane fl) {
  const uint8_t* base = tile + off;
  uint4 lo = *reinterpret_cast<const uint4*>(base + fl.lo);
  uint4 hi = *reinterpret_cast<const uint4*>(base + fl.hi);
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// The experts' m-tiles: expert e has ceil(valid rows / BM) of them,
// numbered expert by expert.  Each wave evaluates it on its own, 64 experts
// per pass with lane l holding expert base + l (one round of vector loads,
// then shuffles), so a tile is located in about one memory latency rather
// than a chain of dependent scalar loads per expert.  All results are
// wave-uniform.
struct SegLane {
  int s, en, nt;   // this lane's expert: valid rows [s, en), m-tiles
};

template <int BM>
__device__ __forceinline__ SegLane seg_lane(const int32_t* offsets, const int32_t* counts,
                                            int E, int rows_total, int e) {
  SegLane r{0, 0, 0};
  if (e < E) {
    expert_rows(offsets, counts, e, rows_total, r.s, r.en);
    r.nt = (r.en - r.s + BM - 1) / BM;
  }
  return r;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(x, d);
    if (lane >= d) x += t;
  }
  return x;
}

// Total number of m-tiles.
template <int BM>
__device__ __forceinline__ int total_mtiles(const int32_t* offsets, const int32_t* counts,
                                            int E, int rows_total, int lane) {
  int total = 0;
  for (int base = 0; base < E; base += 64)
    total += wave_sum(seg_lane<BM>(offsets, counts, E, rows_total, base + lane).nt);
  return __builtin_amdgcn_readfirstlane(total);
}

// The third A stage, an LDS object only where the kernel has one (a tile
// whose two A and two B stages already fill the LDS declares none).
template <int kBytes>
struct ThirdStage {
  __device__ __forceinline__ static uint8_t* get() {
    __shared__ __attribute__((aligned(1024))) uint8_t s[kBytes];
    return s;
  }
};
template <>
struct ThirdStage<0> {
  __device__ __forceinline__ static uint8_t* get() { return nullptr; }
};

// Expert, first row and segment end of m-tile mt (e_sel = -1 if none).
template <int BM>
__device__ __forceinline__ void find_mtile(const int32_t* offsets, const int32_t* counts,
                                           int E, int rows_total, int mt, int lane,
                                           int& e_sel, int& row0, int& row_end) {
  e_sel = -1;
  int before = 0;   // m-tiles of the experts of earlier passes
  for (int base = 0; base < E; base += 64) {
    const SegLane g = seg_lane<BM>(offsets, counts, E, rows_total, base + lane);
    const int incl = before + wave_inclusive_scan(g.nt, lane);
    // the first lane whose running count passes mt holds the expert (its
    // count is non-zero: the running count steps there)
    const uint64_t hit = __ballot(incl > mt);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      e_sel = base + l;
      row0 = __builtin_amdgcn_readlane(g.s, l) +
             (mt - (__builtin_amdgcn_readlane(incl, l) - __builtin_amdgcn_readlane(g.nt, l))) * BM;
      row_end = __builtin_amdgcn_readlane(g.en, l);
      return;
    }
    before = __builtin_amdgcn_readlane(incl, 63);
  }
}

// kGather: A is not the permuted buffer but the source rows x [src_rows, K];
// buffer row r of the tile is read from x[row_src[r]] (a row with no source
// reads zero), so the row permutation happens in the tile loads.
template <int BM, int BN, int WM, int WN, int GM, int kTag, bool kPow2, bool kGather>
__global__ __launch_bounds__(64 * (BM / WM) * (BN / WN)) void grouped_gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA,
    const uint8_t* __restrict__ W, const float* __restrict__ SW,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ counts,
    int E, int rows_total, int N, int K, uint16_t* __restrict__ C,
    uint8_t* __restrict__ Q, void* __restrict__ QS, int32_t* __restrict__ status,
    const int32_t* __restrict__ row_src, int src_rows) {
  constexpr int NWM = BM / WM;
  constexpr int NWN = BN / WN;
  constexpr int NW = NWM * NWN;
  constexpr int MI = WM / 16;
  constexpr int NJ = WN / 16;
  constexpr int A_CHUNKS = BM / 8;                   // 1 KB LDS chunks per stage
  constexpr int B_CHUNKS = BN / 8;
  constexpr int CA = A_CHUNKS / NW;                  // A / B chunks per wave and stage
  constexpr int CB = B_CHUNKS / NW;
  static_assert(A_CHUNKS % NW == 0 && B_CHUNKS % NW == 0, "chunks must split evenly");
  static_assert(CB % 2 == 0, "B chunk parity is static");
  static_assert(BN <= kBlock || BN % kBlock == 0, "tile N range");
  static_assert(WN <= kBlock && kBlock % WN == 0, "wave columns in one scale block");
  static_assert(CA < 64, "vmcnt range");
  // kTag 4: gate/up projection with the activation and its re-quantisation
  // fused into the epilogue (W13 rows [0, N/2) gate, [N/2, N) up).  Tile
  // column block wn holds 32 gate columns followed by the 32 up columns of
  // the same intermediate columns, so one lane holds both operands of every
  // silu(gate) * up it produces; a tile covers BN / 2 = 128 intermediate
  // columns, exactly one 1x128 scale block per row.
  constexpr bool kFused = kTag == 4;
  static_assert(!kFused || (WN == 64 && NJ == 4 && BN / 2 == kBlock), "fused tile shape");

  // A rows: three stages (k-blocks kb, kb + 1 landed or landing, kb + 2
  // in flight) when they fit beside the two B stages, else two (320-row
  // tiles: kb + 1 is loaded while kb is multiplied, like B).  Each stage is
  // its own LDS object.
  constexpr int SA_B = BM * kBK, SB_B = BN * kBK;
  constexpr int NSA = 3 * SA_B + 2 * SB_B <= kLdsBytes ? 3 : 2;
  static_assert(NSA * SA_B + 2 * SB_B <= kLdsBytes, "tile stages exceed the LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[SA_B];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[SA_B];
  uint8_t* const sA2 = ThirdStage<NSA == 3 ? SA_B : 0>::get();   // null with two stages
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[SB_B];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[SB_B];
  // stage by (compile-time) index
  auto stA = [&](int i) -> uint8_t* { return i == 0 ? sA0 : i == 1 ? sA1 : sA2; };
  auto stB = [&](int i) -> uint8_t* { return i == 0 ? sB0 : sB1; };

  // ---- which tile: grouped order over the tile list (see the XCD note above)
  constexpr bool kDense = kTag == 3;
  const int n_tiles = N / BN;
  int e_sel = 0, row0 = 0, row_end = 0;
  const int lane = threadIdx.x & 63;
  const int total_m = kDense ? (rows_total + BM - 1) / BM
                             : total_mtiles<BM>(offsets, counts, E, rows_total, lane);
  const int total = total_m * n_tiles;
  const int logical = blockIdx.x;
  // workgroup 0's first wave checks that offsets / counts describe segments
  // (a corrupt table is still clipped to the buffer; rows past the tile
  // count of the grid are then not computed, hence the flag)
  if (!kDense && logical == 0 && threadIdx.x < 64 && status &&
      segments_bad(offsets, counts, E, lane) && lane == 0)
    atomicOr(status, MOE_ERR_BAD_INDEX);
  if (logical >= total) return;
  const int group_size = GM * n_tiles;
  const int grp = logical / group_size;
  const int in_grp = logical - grp * group_size;
  const int gm0 = grp * GM;
  const int gm_cnt = min(GM, total_m - gm0);
  const int tile_n = in_grp / gm_cnt;
  const int tile_m = gm0 + (in_grp - tile_n * gm_cnt);
  if (kDense) {
    e_sel = 0;
    row0 = tile_m * BM;
    row_end = rows_total;
  } else {
    find_mtile<BM>(offsets, counts, E, rows_total, tile_m, lane, e_sel, row0, row_end);
    if (e_sel < 0) return;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave / NWN;
  const int wn = wave - wm * NWN;
  const int Kb = K / kBK;
  const int nb_w = N / kBlock;
  const int n0 = tile_n * BN;                 // first output column (unfused)
  const int Ih = N / 2;                        // fused: intermediate size
  const int ni0 = tile_n * (BN / 2);           // fused: first intermediate column

  // Loads that a step issues past the last k-block (live = false) take an
  // offset beyond every descriptor's range: they read zero without touching
  // memory, and every step issues the same loads and ends with the same
  // wait, with no branch in the step (a branch per wait left the compiler's
  // control flow with paths no execution takes).
  constexpr uint32_t kOutOfRange = 0x80000000u;
  // A lane's offset in an 8-row DMA chunk: row lane / 8, 16-byte piece
  // (lane & 7) permuted as that row sits in the even 8-row half of its
  // 16-row group; in the odd half the permutation differs by XOR 1 on the
  // piece index, i.e. XOR 16 on the offset (K is a multiple of 128, so the
  // row part leaves bit 4 alone).
  const uint32_t lane_off = (uint32_t)(lane >> 3) * (uint32_t)K +
                            (uint32_t)(((lane & 7) ^ swz(lane >> 3)) << 4);
  const long long a_bytes = kGather ? (long long)src_rows * K : (long long)(rows_total - row0) * K;
  const v4i rsrc_a = make_rsrc(kGather ? A : A + (size_t)row0 * K,
                               (uint32_t)(a_bytes > 0x7ffff000LL ? 0x7ffff000LL : a_bytes));
  // kGather: per-lane byte offsets of the wave's A chunks in x (chunk u
  // holds tile rows 8 (wave CA + u) .. + 7, the lane row lane / 8 of them),
  // read before any tile load; rows without a source get an offset out of
  // range and load zero.
  uint32_t a_off[kGather ? CA : 1];
  if constexpr (kGather) {
#pragma unroll
    for (int u = 0; u < CA; ++u) {
      const int c = wave * CA + u;
      const int r = row0 + c * 8 + (lane >> 3);
      const int src = r < rows_total ? row_src[r] : -1;
      a_off[u] = (src >= 0 && src < src_rows)
                     ? (uint32_t)src * (uint32_t)K + (uint32_t)(((lane & 7) ^ swz(lane >> 3)) << 4)
                     : kOutOfRange;   // (the odd-half XOR 16 is applied at issue)
    }
    // the offsets (and so the compiler's wait for row_src) are ready before
    // the first tile load is issued
#pragma unroll
    for (int u = 0; u < CA; ++u) asm volatile("" : "+v"(a_off[u]));
  }
  // fused: the descriptor spans the expert's whole W13 (the host checks
  // N * K < 2^31); the gate and up rows of a tile are two separate runs
  const v4i rsrc_b = kFused ? make_rsrc(W + (size_t)e_sel * N * K, (uint32_t)(N * K))
                            : make_rsrc(W + ((size_t)e_sel * N + n0) * K, (uint32_t)(BN * K));

  // Row scales go straight to registers, one step ahead: lane l loads the
  // scales of rows wm*WM + 64c + l (MI / 4 loads, into fs_raw), and the
  // scale of row wm*WM + i*16 + r that lane (g, r) needs for subtile row i
  // is then broadcast from lane 16 (i mod 4) + r of load i / 4 by lane swaps
  // (row_scales).  Rows past the buffer read another k-block's scales or
  // zero and only feed rows that are never stored.  kPow2: scales are E8M0 bytes
  // packed four k-blocks per 32-bit word (row scales [ceil(Kb/4),
  // rows_total] words, weight scales [E, N/128, ceil(Kb/4)] words); the
  // MFMA applies them itself.
  const int Kw = (Kb + 3) / 4;
  const float* SWw = SW + ((size_t)e_sel * nb_w + (n0 + wn * WN) / kBlock) * (kPow2 ? Kw : Kb);
  // fused: gate (SWw) and up (SWu) weight blocks of this wave's columns
  const float* SWg = SW + ((size_t)e_sel * nb_w + (ni0 + wn * (WN / 2)) / kBlock) * (kPow2 ? Kw : Kb);
  const float* SWu =
      SW + ((size_t)e_sel * nb_w + (Ih + ni0 + wn * (WN / 2)) / kBlock) * (kPow2 ? Kw : Kb);
  const long long sa_bytes = (long long)(kPow2 ? Kw : Kb) * rows_total * 4;
  const v4i rsrc_s = make_rsrc(SA, (uint32_t)(sa_bytes > 0x7ffff000LL ? 0x7ffff000LL : sa_bytes));
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int wcol = wn * WN;
  // fragment read offsets of the wave's A rows and B columns
  FragLane fa = frag_lane(wm * WM, r16, g);
  FragLane fb = frag_lane(wcol, r16, g);
  constexpr int NR = (MI + 3) / 4;   // 64-row scale loads (the last may overhang)
  const uint32_t srow = (uint32_t)(row0 + wm * WM + lane);
  float fs_raw[NR];
#pragma unroll
  for (int c = 0; c < NR; ++c) fs_raw[c] = 0.f;
  // The loads are inline assembly, like the tile loads: a register is
  // filled when its load completes, not when the instruction issues, so
  // fs_raw is read only after the wait_loads() that covers these loads,
  // which is also where the compiler sees the values being written.
  auto load_scales = [&](int kb, bool live) {
    const uint32_t base =
        live ? ((uint32_t)(kPow2 ? kb >> 2 : kb) * (uint32_t)rows_total + srow) * 4u : kOutOfRange;
#pragma unroll
    for (int c = 0; c < NR; ++c)
      asm volatile("buffer_load_dword %0, %1, %2, 0 offen offset:%3"
                   : "=v"(fs_raw[c]) : "v"(base), "s"(rsrc_s), "n"(c * 256) : "memory");
  };
  auto issue_a1 = [&](int kb, uint8_t* tA, int u, bool live) {
    const int c = wave * CA + u;   // wave-uniform; with CA even its parity is u's
    const uint32_t odd16 = (CA % 2 == 0 ? (u & 1) : (c & 1)) ? 16u : 0u;
    if constexpr (kGather)   // (an out-of-range offset plus kOutOfRange may wrap
                             // to a small one: a read inside x into a free stage)
      dma16_split(rsrc_a, tA + c * 1024, a_off[u], __builtin_amdgcn_readfirstlane(odd16),
                  __builtin_amdgcn_readfirstlane(live ? (uint32_t)kb * kBK : kOutOfRange));
    else
      dma16_split(rsrc_a, tA + c * 1024, lane_off, __builtin_amdgcn_readfirstlane(odd16),
                  __builtin_amdgcn_readfirstlane(
                      live ? (uint32_t)(c * 8) * (uint32_t)K + (uint32_t)kb * kBK : kOutOfRange));
  };
  auto issue_a = [&](int kb, uint8_t* tA, bool live) {
#pragma unroll
    for (int u = 0; u < CA; ++u) issue_a1(kb, tA, u, live);
  };
  // kLateA: the A rows of k-block kb + 2 are issued after the MFMAs of the
  // first subtile row of step kb instead of with the B rows at its start.
  // All waves issue their loads at once after the step barrier, and a wave
  // stalls while the CU's address unit works through them; deferring the A
  // half lets the first MFMAs start earlier.  Measured at the prefill shape:
  // 0.6-1.9% off the unfused gate/up GEMM and the down GEMM over three boxes
  // (deferring the B rows as well, or having only one wave per SIMD issue
  // all the tile loads, was slower); on the fused gate/up + activation
  // 1.5% (fp32 scales) and 2.3% (packed) at prefill, 2% and 7% on the EP72
  // and EP48 decode shares, bit-identical.  The 320-row fused kernel keeps
  // the early issue: with the late one it spills four registers.
  constexpr bool kLateA = !kFused || BM < 320;
  // The packed-scale step runs subtile rows 0 .. MI - 2 before its barrier
  // and the fp32 step rows 0 .. MI - 1, so row 1 exists in both once MI >= 3;
  // with MI = 2 the A rows go out after row 0.  (A row index no step reaches
  // would leave the stage unloaded.)
  constexpr int kLateRow = MI >= 3 ? 1 : 0;
  static_assert(!kLateA || MI >= 2, "late A issue needs a subtile row before the barrier");
  auto issue_a_row = [&](int kb, uint8_t* tA, int i, bool live) {
    if (i == kLateRow) issue_a(kb, tA, live);
  };
  auto issue_b = [&](int kb, uint8_t* tB, bool live) {
    const uint32_t kofs = (uint32_t)kb * kBK;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int c = wave * CB + u;
      int row = c * 8;   // B row of the tile's first LDS row in this chunk
      if (kFused) {      // tile column b -> W13 row (gate or up)
        const int wv = row / WN, k = row - wv * WN;
        row = (k < WN / 2 ? 0 : Ih - WN / 2) + ni0 + wv * (WN / 2) + k;
      }
      dma16_split(rsrc_b, tB + c * 1024, lane_off, (u & 1) ? 16u : 0u,
                  __builtin_amdgcn_readfirstlane(live ? (uint32_t)row * (uint32_t)K + kofs
                                                      : kOutOfRange));
    }
  };

  v4f acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  float sw_cur = 0.f;   // weight-block scale of the current step (fused: gate)
  // products of the most recent subtile row and their combined scales,
  // promoted one row later, across the step boundary for the last row
  v4f tprev[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) tprev[j] = (v4f){0.f, 0.f, 0.f, 0.f};
  float fprev = 0.f, fprevu = 0.f;
  float swu_cur = 0.f;  // fused: up weight-block scale

  // Fragments of the step about to run: the B fragments of the wave's
  // columns and the A fragment of its first subtile row (the packed-scale
  // path reads them during the previous step's last subtile row).
  v8i bf[NJ];
  v8i af_next;

  // One K step: A k-block kb in A stage SAi = kb % NSA, B in B stage
  // SBi = kb % 2.  At its start the B rows and row scales of k-block kb + 1
  // and the A rows of k-block kb + NSA - 1 are issued (into stages freed by
  // the barrier that ended the previous step's reads).  At the step barrier
  // only the A rows of kb + 2 may still be in flight (three A stages; with
  // two, every load of kb + 1 has landed).
  //
  // Packed scales: the step barrier comes once the wave's last LDS read of
  // the step (the A fragment of the last subtile row) has landed, before
  // the last row's MFMAs: those use registers only, and while they run the
  // wave already reads the next step's fragments, so the matrix core is not
  // idle while they load.  Measured at the prefill gate/up shape: 7% off the
  // GEMM, 5% off the fused GEMM + activation, 4% off the down GEMM, with
  // bit-identical results.
  auto step = [&](int kb, auto sa_i, auto sb_i) __attribute__((always_inline)) {
    constexpr int SAi = decltype(sa_i)::value;
    constexpr int SBi = decltype(sb_i)::value;
    // opaque per step: the compiler then forms each fragment address inside
    // the step (lane offset + immediate) instead of hoisting one register
    // per stage and subtile out of the K loop
    asm volatile("" : "+v"(fa.lo), "+v"(fa.hi), "+v"(fb.lo), "+v"(fb.hi));
    const uint8_t* tA = stA(SAi);
    const uint8_t* tAn = stA((SAi + 1) % NSA);   // next step's stages
    const uint8_t* tBn = stB((SBi + 1) % 2);
    float fs[4 * NR];
#pragma unroll
    for (int c = 0; c < NR; ++c) row_scales(fs_raw[c], fs + 4 * c);
    const bool rb = kb + 1 < Kb;
    const bool ra = kb + NSA - 1 < Kb;   // A rows of k-block kb + NSA - 1 to load
    uint8_t* const tAl = stA((SAi + NSA - 1) % NSA);
    issue_b(kb + 1, stB((SBi + 1) % 2), rb);
    load_scales(kb + 1, rb);
    if (!kLateA) issue_a(kb + NSA - 1, tAl, ra);
    const float sw = sw_cur;
    const float swu = swu_cur;
    const int kn = rb ? kb + 1 : kb;   // the next step's k-block (the last: unused)
    if (kFused) {
      sw_cur = SWg[kPow2 ? kn >> 2 : kn];
      swu_cur = SWu[kPow2 ? kn >> 2 : kn];
    } else {
      sw_cur = SWw[kPow2 ? kn >> 2 : kn];
    }
    // the end of the step's reads: wait for the loads of k-block kb + 1
    // (with three A stages everything but the A rows of kb + 2), then meet
    // the other waves
    auto end_reads = [&]() {
      if constexpr (NSA == 3)
        wait_loads<CA>(fs_raw);
      else
        wait_loads<0>(fs_raw);
      lds_barrier();
    };
    if constexpr (kPow2) {
      const int sh = 8 * (kb & 3);
      const int sw_e = (int)((__float_as_uint(sw) >> sh) & 0xffu);
      const int swu_e = kFused ? (int)((__float_as_uint(swu) >> sh) & 0xffu) : sw_e;
      int sa_e[MI];
#pragma unroll
      for (int i = 0; i < MI; ++i) sa_e[i] = (int)((__float_as_uint(fs[i]) >> sh) & 0xffu);
#pragma unroll
      for (int i = 0; i < MI - 1; ++i) {
        if (kLateA) issue_a_row(kb + NSA - 1, tAl, i, ra);
        const v8i af = af_next;
        af_next = load_frag_at(tA, (i + 1) * 16 * kBK, fa);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bf[j], af, acc[i][j], 0, 0, 0, (kFused && j >= NJ / 2) ? swu_e : sw_e, 0,
              sa_e[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the MFMAs so far are issued before the barrier (it orders memory
      // only, so the compiler could otherwise sink them past it)
#pragma unroll
      for (int i = 0; i < MI - 1; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(acc[i][j]));
      end_reads();
      const v8i af = af_next;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        acc[MI - 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bf[j], af, acc[MI - 1][j], 0, 0, 0, (kFused && j >= NJ / 2) ? swu_e : sw_e, 0,
            sa_e[MI - 1]);
        bf[j] = load_frag_at(tBn, j * 16 * kBK, fb);
      }
      af_next = load_frag_at(tAn, 0, fa);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(acc[MI - 1][j]));
    } else {
    // fp32 scales: the barrier stays at the end of the step (measured: the
    // early barrier of the packed-scale path gains nothing here, and its
    // longer register live ranges do not fit the fused kernel).  The
    // products of subtile row i are promoted while row i + 1 is multiplied,
    // and those of the last row at the start of the next step (tprev and
    // fprev persist across steps), so a wave reaches the step barrier right
    // after issuing its last MFMA instead of waiting for it to finish.
#pragma unroll
    for (int j = 0; j < NJ; ++j) bf[j] = load_frag_at(stB(SBi), j * 16 * kBK, fb);
    af_next = load_frag_at(tA, 0, fa);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (kLateA) issue_a_row(kb + NSA - 1, tAl, i, ra);
      const v8i af = af_next;
      if (i + 1 < MI) af_next = load_frag_at(tA, (i + 1) * 16 * kBK, fa);
      const float fcur = fs[i] * sw;
      const float fcuru = kFused ? fs[i] * swu : 0.f;
      v4f tcur[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) tcur[j] = mfma_fp8_16x16x128(bf[j], af);
      const int ip = i > 0 ? i - 1 : MI - 1;   // row whose products are complete
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float f = (kFused && j >= NJ / 2) ? fprevu : fprev;
        acc[ip][j][0] = fmaf(tprev[j][0], f, acc[ip][j][0]);
        acc[ip][j][1] = fmaf(tprev[j][1], f, acc[ip][j][1]);
        acc[ip][j][2] = fmaf(tprev[j][2], f, acc[ip][j][2]);
        acc[ip][j][3] = fmaf(tprev[j][3], f, acc[ip][j][3]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) tprev[j] = tcur[j];
      fprev = fcur;
      fprevu = fcuru;
      if (i > 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(acc[i][j]));
    end_reads();
    }
  };

  if (kFused) {
    sw_cur = SWg[0];
    swu_cur = SWu[0];
  } else {
    sw_cur = SWw[0];
  }
  issue_b(0, sB0, true);
  load_scales(0, true);
  issue_a(0, sA0, true);
  if constexpr (NSA == 3) {
    issue_a(1, sA1, Kb > 1);
    wait_loads<CA>(fs_raw);
  } else {
    wait_loads<0>(fs_raw);
  }
  lds_barrier();
  if constexpr (kPow2) {   // fp32 scales: read at the step start
#pragma unroll
    for (int j = 0; j < NJ; ++j) bf[j] = load_frag_at(sB0, j * 16 * kBK, fb);
    af_next = load_frag_at(sA0, 0, fa);
  }
  // unrolled by 6 = lcm(3, 2), so every step names its stages statically
  auto step_u = [&](int kb, auto u) __attribute__((always_inline)) {
    constexpr int U = decltype(u)::value;
    if (U == 0 || kb < Kb)
      step(kb, std::integral_constant<int, U % NSA>(), std::integral_constant<int, U % 2>());
  };
  for (int kb = 0; kb < Kb; kb += 6) {
    step_u(kb, std::integral_constant<int, 0>());
    step_u(kb + 1, std::integral_constant<int, 1>());
    step_u(kb + 2, std::integral_constant<int, 2>());
    step_u(kb + 3, std::integral_constant<int, 3>());
    step_u(kb + 4, std::integral_constant<int, 4>());
    step_u(kb + 5, std::integral_constant<int, 5>());
  }
  // With three A stages the last step leaves its (out-of-range, zero)
  // A loads in flight; they write into stage memory, which the epilogue
  // reuses, so every wave drains its loads and meets the others first.
  if constexpr (NSA == 3) {
    wait_loads<0>(fs_raw);
    lds_barrier();
  }
  if constexpr (!kPow2) {   // the last row's products
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float f = (kFused && j >= NJ / 2) ? fprevu : fprev;
      acc[MI - 1][j][0] = fmaf(tprev[j][0], f, acc[MI - 1][j][0]);
      acc[MI - 1][j][1] = fmaf(tprev[j][1], f, acc[MI - 1][j][1]);
      acc[MI - 1][j][2] = fmaf(tprev[j][2], f, acc[MI - 1][j][2]);
      acc[MI - 1][j][3] = fmaf(tprev[j][3], f, acc[MI - 1][j][3]);
    }
  }

  // packed scales: the epilogue's lane position is read afresh (frees a
  // register through the K loop; the fp32-scale kernels measured no better)
  const int lane_e = kPow2 ? lane_id_fresh() : lane;
  if constexpr (kFused) {
    const int lane = lane_e, g = lane >> 4, r16 = lane & 15;
    // ---- fused epilogue.  h = bf16(acc) -- the values the unfused path
    // stores -- then v = silu(gate) * up in fp32 exactly as the stand-alone
    // activation kernel computes it, the row's 1x128 amax over the NWN waves
    // through LDS, E4M3 codes staged in LDS (16-byte chunks XOR-permuted by
    // row & 7) and stored as 128-byte row pieces, one scale per row.  The
    // stage memory is free: every load has landed and all waves have met
    // since the last fragment read.
    (void)C;
    constexpr int NT = 64 * NW;
    static_assert(BM * NWN * 4 <= SA_B && BM * kBlock <= SA_B, "fused staging space");
    float* red = reinterpret_cast<float*>(sA1);   // [BM][NWN] partial amax
    uint8_t* qst = sA0;                            // [BM][128] codes
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      float amax = 0.f;
#pragma unroll
      for (int jj = 0; jj < NJ / 2; ++jj) {
        const uint32_t g01 = pack2_bf16(acc[i][jj][0], acc[i][jj][1]);
        const uint32_t g23 = pack2_bf16(acc[i][jj][2], acc[i][jj][3]);
        const uint32_t u01 = pack2_bf16(acc[i][jj + NJ / 2][0], acc[i][jj + NJ / 2][1]);
        const uint32_t u23 = pack2_bf16(acc[i][jj + NJ / 2][2], acc[i][jj + NJ / 2][3]);
        acc[i][jj][0] = silu_mul(bf16_to_f32(g01 & 0xffffu), bf16_to_f32(u01 & 0xffffu));
        acc[i][jj][1] = silu_mul(bf16_to_f32(g01 >> 16), bf16_to_f32(u01 >> 16));
        acc[i][jj][2] = silu_mul(bf16_to_f32(g23 & 0xffffu), bf16_to_f32(u23 & 0xffffu));
        acc[i][jj][3] = silu_mul(bf16_to_f32(g23 >> 16), bf16_to_f32(u23 >> 16));
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(acc[i][jj][0]), fabsf(acc[i][jj][1])),
                                 fmaxf(fabsf(acc[i][jj][2]), fabsf(acc[i][jj][3]))));
      }
      // the four lanes (g = 0..3) of row r16 hold this wave's 32 columns
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      if (g == 0) red[(wm * WM + i * 16 + r16) * NWN + wn] = amax;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wm * WM + i * 16 + r16;   // tile row
      float amax = 0.f;
#pragma unroll
      for (int w = 0; w < NWN; ++w) amax = fmaxf(amax, red[r * NWN + w]);
      const float v[8] = {acc[i][0][0], acc[i][0][1], acc[i][0][2], acc[i][0][3],
                          acc[i][1][0], acc[i][1][1], acc[i][1][2], acc[i][1][3]};
      uint2 out;
      const uint32_t sc = requant8<kPow2>(v, amax, out);
      // out.x: columns wn*32 + 4g .. +3, out.y: wn*32 + 16 + 4g .. +3
      *reinterpret_cast<uint32_t*>(qst + r * kBlock + (((2 * wn) ^ (r & 7)) << 4) + 4 * g) = out.x;
      *reinterpret_cast<uint32_t*>(qst + r * kBlock + (((2 * wn + 1) ^ (r & 7)) << 4) + 4 * g) =
          out.y;
      const int row = row0 + r;
      if (wn == 0 && g == 0 && row < row_end) {
        if (kPow2) {
          const int jb = ni0 / kBlock, ib = Ih / kBlock;
          uint8_t* wp = reinterpret_cast<uint8_t*>(QS) + ((size_t)(jb >> 2) * rows_total + row) * 4;
          wp[jb & 3] = (uint8_t)sc;
          if (jb == ib - 1)
            for (int q = (jb & 3) + 1; q < 4; ++q) wp[q] = 127;   // past the last block
        } else {
          reinterpret_cast<uint32_t*>(QS)[(size_t)(ni0 / kBlock) * rows_total + row] = sc;
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int p = tid; p < BM * 8; p += NT) {
      const int r = p >> 3, c = p & 7;
      const uint4 v = *reinterpret_cast<const uint4*>(qst + r * kBlock + ((c ^ (r & 7)) << 4));
      const int row = row0 + r;
      if (row < row_end)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                    reinterpret_cast<u32x4*>(Q + (size_t)row * Ih + ni0 + c * 16));
    }
  } else {
    const int lane = lane_e, g = lane >> 4, r16 = lane & 15;
    (void)Q;
    (void)QS;
    // ---- epilogue.  In subtile (i, j) a lane holds row r16 and columns
    // 4g .. 4g+3.  Stored directly, every store instruction would write 16
    // scattered 32-byte pieces; instead each wave stages its WM x WN bf16
    // sub-tile (rows of WN * 2 = 128 bytes) in a region of its own in the
    // stage memory -- free now: every load has landed and all waves have met
    // since the last fragment read -- and stores it back as 16-byte pieces, eight lanes per
    // contiguous 128-byte row.  Only the wave's own LDS accesses are ordered,
    // so no workgroup barrier is needed.  The 8-byte chunks of staged row r
    // are XOR-permuted by 2 * ((r >> 1) & 7), which keeps the chunk pairs of
    // a 16-byte read together.  The output is written with non-temporal
    // stores.  Measured at the prefill shape: GEMM2 -5%, GEMM1 -4% against
    // direct 8-byte stores; the packed hardware conversion to bf16 took
    // another 6% (GEMM2) and 3% (GEMM1) off against a bit-level rounding
    // sequence.
    // A wave's sub-tile is staged in kParts passes of PM rows when the free
    // stage memory cannot hold all NW of them at once (320-row tiles: two).
    static_assert(WN * 2 == 128, "staged rows are 128 bytes");
    constexpr auto fits = [](int parts) {
      const int region = WM / parts * WN * 2;
      return (SA_B / region) * NSA + (SB_B / region) * 2 >= NW;
    };
    constexpr int kParts = fits(1) ? 1 : fits(2) ? 2 : (MI % 3 == 0 && fits(3)) ? 3
                         : (MI % 4 == 0 && fits(4)) ? 4 : 5;
    static_assert(fits(kParts) && MI % kParts == 0, "staging space");
    constexpr int PM = WM / kParts;            // rows per pass
    constexpr int kRegion = PM * WN * 2;
    constexpr int kPerA = SA_B / kRegion, kPerB = SB_B / kRegion;
    uint8_t* region;   // regions fill the A stages, then the B stages
    if (wave < NSA * kPerA) {
      const int st = wave / kPerA;
      region = (st == 0 ? sA0 : st == 1 ? sA1 : sA2) + (wave - st * kPerA) * kRegion;
    } else {
      const int w = wave - NSA * kPerA;
      region = w < kPerB ? sB0 + w * kRegion : sB1 + (w - kPerB) * kRegion;
    }
    const int c16 = lane & 7;
  #pragma unroll
    for (int part = 0; part < kParts; ++part) {
      // the stores of a pass consume the values it read back, so those
      // reads have completed before the next pass overwrites the region
  #pragma unroll
      for (int i = part * (MI / kParts); i < (part + 1) * (MI / kParts); ++i) {
        const int r = (i - part * (MI / kParts)) * 16 + r16;
        const int f = ((r >> 1) & 7) << 1;
  #pragma unroll
        for (int j = 0; j < NJ; ++j) {
          uint2 o;
          o.x = pack2_bf16(acc[i][j][0], acc[i][j][1]);
          o.y = pack2_bf16(acc[i][j][2], acc[i][j][3]);
          *reinterpret_cast<uint2*>(region + r * 128 + (((j * 4 + g) ^ f) << 3)) = o;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  #pragma unroll
      for (int rr = 0; rr < PM; rr += 8) {
        const int r = rr + (lane >> 3);
        const uint4 v =
            *reinterpret_cast<const uint4*>(region + r * 128 + ((c16 ^ ((r >> 1) & 7)) << 4));
        const int row = row0 + wm * WM + part * PM + r;
        if (row < row_end)   // streamed out: not kept in the caches the tiles share
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                      reinterpret_cast<u32x4*>(C + (size_t)row * N + n0 + wcol + c16 * 8));
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int GM, int kTag, bool kPow2 = false, bool kGather = false>
static moe_status_t launch(const uint8_t* a, const float* a_scale, const uint8_t* w,
                           const float* w_scale, const int32_t* offsets,
                           const int32_t* counts, int E, int rows_total, int N, int K,
                           uint16_t* c, hipStream_t st, int32_t* status,
                           uint8_t* q = nullptr, void* q_scale = nullptr,
                           const int32_t* row_src = nullptr, int src_rows = 0) {
  if (N % BN != 0) return MOE_UNSUPPORTED_SHAPE;
  long long m_tiles = kTag == 3 ? ((long long)rows_total + BM - 1) / BM
                                : (long long)rows_total / BM + E;
  long long blocks = m_tiles * (N / BN);
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  if (blocks > 0x7fffffffLL) return MOE_UNSUPPORTED_SHAPE;
  constexpr int threads = 64 * (BM / WM) * (BN / WN);
  hipLaunchKernelGGL((grouped_gemm_fp8_kernel<BM, BN, WM, WN, GM, kTag, kPow2, kGather>),
                     dim3((unsigned)blocks), dim3(threads), 0, st, a, a_scale, w, w_scale,
                     offsets, counts, E, rows_total, N, K, c, q, q_scale, status, row_src,
                     src_rows);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}

// Tile configurations (BM, BN, WM, WN, GM).  256 x 256 tiles (8 waves of
// 128 x 64, two per SIMD, one workgroup per CU) unless the problem is too
// small for them (see use_big_tiles); then 128 x 128 (4 waves of 64 x 64,
// two workgroups per CU).  kTag keeps the gate/up (1) and down (2) projections and the
// dense product (3) as separate kernel symbols so that profiles attribute
// time per projection.
#ifndef MOE_GEMM_BIG
#define MOE_GEMM_BIG 256, 256, 128, 64, 2
#endif
#ifndef MOE_GEMM_SMALL
#define MOE_GEMM_SMALL 128, 128, 64, 64, 4
#endif
// Packed scales at prefill sizes: 320 x 256 tiles of 8 waves of 160 x 64
// (160 accumulator registers per lane; two A and two B stages, 144 KB of
// LDS), which the scaled MFMA's in-place accumulation leaves room for.
// 384-row tiles (192 accumulators) do not fit two waves per SIMD without
// spilling.
#ifndef MOE_GEMM_HUGE
#define MOE_GEMM_HUGE 320, 256, 160, 64, 2
#endif
// Decode shares whose large tiles fit one round on the CUs: 192 x 256 tiles
// of 8 waves of 96 x 64, as long as they still fit one round (fewer fed
// bytes per k-step: 56 KB instead of 64 KB).
#ifndef MOE_GEMM_MID
#define MOE_GEMM_MID 192, 256, 96, 64, 2
#endif
// The gate/up projection of buffers whose expert segments hold at most 128
// rows (the masked decode layout): 64 x 128 tiles of 4 waves of 32 x 64.
#ifndef MOE_GEMM_SHORT
#define MOE_GEMM_SHORT 64, 128, 32, 64, 4
#endif
// The fused gate/up + activation kernel needs a tile to cover one whole
// 1x128 block of intermediate columns (BN = 256: 128 gate + 128 up
// columns): large problems use MOE_GEMM_BIG, small ones 128 x 256 tiles of
// 8 waves of 64 x 64 (one workgroup per CU).
#ifndef MOE_GEMM_FUSED_SMALL
#define MOE_GEMM_FUSED_SMALL 128, 256, 64, 64, 2
#endif

// The tile feed (bytes a CU receives per k-step) bounds both tile sizes,
// and a 256 x 256 tile does twice the work per byte of two 128 x 128 tiles,
// so the large tiles win once they fill more than half of the CUs -- unless
// the expert segments are mostly shorter than 256 rows (the masked decode
// layout with a capacity of 128), where half of every large tile would be
// padding.  Decided from host-known sizes only, so it is the same inside
// graph capture.  Measured on the decode shares: 8% (EP72) and 7% (EP48)
// faster steps than the earlier rule of at least 512 large tiles, and 13%
// slower for the masked layout had it used large tiles.
static bool use_big_tiles(long long rows_total, int N, int E) {
  return N % 256 == 0 && rows_total >= 256LL * E && (rows_total / 256) * (N / 256) > 128;
}

// One round of workgroups: the tile count the GPU runs at once (one large
// tile per CU of an MI355X).
constexpr long long kRoundTiles = 256;

// Tiles of height BM for a buffer of rows_total rows in E segments, read as
// a contiguous buffer with 128-row alignment (M_cap = R + 127 E): R / BM plus
// half a partial tile per expert.  An estimate for the host-side rule only:
// the grid is sized by the exact bound in launch().
static long long est_tiles(long long rows_total, int N, int E, int BM) {
  long long r = rows_total - 127LL * E;
  if (r <= 0) r = rows_total;
  return ((r + BM - 1) / BM + (E + 1) / 2) * (N / 256);
}

// 64-row tiles: for the gate/up projection (K > N) when the small tiles run
// and the segments average at most 128 rows.  A segment of a few dozen rows
// then fills one 64-row tile instead of padding a 128-row one, and the
// tiles fill the CUs in whole rounds more often.  Measured on the masked
// decode share (32 experts, capacity 128, 24 of them with 1-128 rows):
// gate/up GEMM 167 -> 152 us (fp32 scales) and 169 -> 155 us (packed),
// bit-identical; its down projection (K = 2048) was 5% slower with them and
// keeps 128 rows.
static bool use_short_tiles(long long rows_total, int N, int K, int E) {
  return K > N && !use_big_tiles(rows_total, N, E) && rows_total <= 128LL * E;
}

// 192-row tiles: only where the 256-row tiles already fit one round, and
// the 192-row tiles still do -- then every tile starts at once either way and
// each moves 1/8 fewer bytes per k-step.  Measured at the EP72 decode share
// (gate/up: 10 m-tiles of 256, 13 of 192, x 16 n-tiles): gate/up GEMM 104 ->
// 91 us, fused with the activation 116 -> 99 us, bit-identical; where the
// 192-row tiles need a second round (its down GEMM, the EP48 share) they were
// 13-30% slower, hence the rule.
static bool use_mid_tiles(long long rows_total, int N, int E) {
  return use_big_tiles(rows_total, N, E) && est_tiles(rows_total, N, E, 256) <= kRoundTiles &&
         est_tiles(rows_total, N, E, 192) <= kRoundTiles;
}

// 320-row tiles (packed scales only): a tile then receives 72 KB per k-step
// for 320 x 256 outputs instead of 64 KB for 256 x 256, 10% fewer bytes per
// flop through the per-CU feed that bounds the large tiles.  Taken when the
// segments average at least 4096 rows (the partial last tile of each
// expert then wastes a few percent at most) and the tiles fill every CU.
// (At the EP72 decode share's down projection, 224 tiles of 320 rows fit one
// round where 280 of 256 need a second one for the last 24, yet the step
// measured 3-4% slower with them: each expert's ~512 rows fill 2 x 320 rows
// at 80%, and each tile is fed 72 KB per k-step instead of 64.)
static bool use_huge_tiles(long long rows_total, int N, int E) {
  return use_big_tiles(rows_total, N, E) && rows_total >= 4096LL * E &&
         (rows_total / 320) * (N / 256) >= 256;
}

}  // namespace moe

using namespace moe;

// The kernels address the row scales of the whole buffer through one buffer
// descriptor, whose byte range and offsets are 32-bit: the scale array
// (K/128 fp32 scales, or ceil(K/512) packed words, per row) must stay below
// 0x7ffff000 bytes.  (The operand descriptors start at the tile's own rows
// or weights and span far less.)
static bool scale_span_ok(long long rows_total, int K, bool pow2) {
  const long long kb = pow2 ? (K / kBK + 3) / 4 : K / kBK;
  return kb * rows_total * 4 <= 0x7ffff000LL;
}

// Gathered A (the *_gather calls): x [src_rows, K] must lie within one
// buffer descriptor's 32-bit range, and every row of the buffer names its
// source row in row_src (-1: none).
static moe_status_t gather_args_ok(const uint8_t* x, int src_rows, const int32_t* row_src,
                                   int K) {
  if (src_rows < 0) return MOE_INVALID_ARG;
  if (!row_src || (src_rows > 0 && !x)) return MOE_INVALID_ARG;
  if ((long long)src_rows * K > 0x7ffff000LL) return MOE_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

template <bool kPow2, bool kGather = false>
static moe_status_t grouped_gemm(const uint8_t* a, const float* a_scale, const uint8_t* w,
                                 const float* w_scale, const int32_t* offsets,
                                 const int32_t* counts, int E, int rows_total, int N, int K,
                                 uint16_t* c, int32_t* status, void* stream,
                                 const int32_t* row_src = nullptr, int src_rows = 0) {
  if (E <= 0 || E > MOE_MAX_EXPERTS || rows_total < 0 || N <= 0 || K <= 0)
    return MOE_INVALID_ARG;
  if (N % kBlock != 0 || K % kBK != 0) return MOE_UNSUPPORTED_SHAPE;
  if (!scale_span_ok(rows_total, K, kPow2)) return MOE_UNSUPPORTED_SHAPE;
  if (!offsets || !counts || !w || !w_scale) return MOE_INVALID_ARG;
  if (kGather) {
    const moe_status_t g = gather_args_ok(a, src_rows, row_src, K);
    if (g != MOE_OK) return g;
  }
  if (rows_total == 0) return MOE_OK;
  if ((!kGather && !a) || !a_scale || !c) return MOE_INVALID_ARG;
  if (((uintptr_t)a | (uintptr_t)w | (uintptr_t)c) & 15) return MOE_UNSUPPORTED_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if constexpr (kGather) {   // the gate/up projection's symbol, whatever the shape
    if (kPow2 && use_huge_tiles(rows_total, N, E))
      return launch<MOE_GEMM_HUGE, 1, true, true>(a, a_scale, w, w_scale, offsets, counts, E,
                                                  rows_total, N, K, c, st, status, nullptr,
                                                  nullptr, row_src, src_rows);
    if (use_mid_tiles(rows_total, N, E))
      return launch<MOE_GEMM_MID, 1, kPow2, true>(a, a_scale, w, w_scale, offsets, counts, E,
                                                  rows_total, N, K, c, st, status, nullptr,
                                                  nullptr, row_src, src_rows);
    if (use_big_tiles(rows_total, N, E))
      return launch<MOE_GEMM_BIG, 1, kPow2, true>(a, a_scale, w, w_scale, offsets, counts, E,
                                                  rows_total, N, K, c, st, status, nullptr,
                                                  nullptr, row_src, src_rows);
    if (use_short_tiles(rows_total, N, K, E))
      return launch<MOE_GEMM_SHORT, 1, kPow2, true>(a, a_scale, w, w_scale, offsets, counts, E,
                                                    rows_total, N, K, c, st, status, nullptr,
                                                    nullptr, row_src, src_rows);
    return launch<MOE_GEMM_SMALL, 1, kPow2, true>(a, a_scale, w, w_scale, offsets, counts, E,
                                                  rows_total, N, K, c, st, status, nullptr,
                                                  nullptr, row_src, src_rows);
  }
  const bool gate_up = K > N;   // gate/up: K = H > N = 2I; down: N = H > K = I
  // host-known sizes only, so the choice is the same inside graph capture
  const bool big = use_big_tiles(rows_total, N, E);
  if (kPow2 && use_huge_tiles(rows_total, N, E))
    return gate_up ? launch<MOE_GEMM_HUGE, 1, true>(a, a_scale, w, w_scale, offsets, counts,
                                                    E, rows_total, N, K, c, st, status)
                   : launch<MOE_GEMM_HUGE, 2, true>(a, a_scale, w, w_scale, offsets, counts,
                                                    E, rows_total, N, K, c, st, status);
  if (use_mid_tiles(rows_total, N, E))
    return gate_up ? launch<MOE_GEMM_MID, 1, kPow2>(a, a_scale, w, w_scale, offsets, counts,
                                                    E, rows_total, N, K, c, st, status)
                   : launch<MOE_GEMM_MID, 2, kPow2>(a, a_scale, w, w_scale, offsets, counts,
                                                    E, rows_total, N, K, c, st, status);
  if (big)
    return gate_up ? launch<MOE_GEMM_BIG, 1, kPow2>(a, a_scale, w, w_scale, offsets, counts,
                                                    E, rows_total, N, K, c, st, status)
                   : launch<MOE_GEMM_BIG, 2, kPow2>(a, a_scale, w, w_scale, offsets, counts,
                                                    E, rows_total, N, K, c, st, status);
  if (use_short_tiles(rows_total, N, K, E))
    return launch<MOE_GEMM_SHORT, 1, kPow2>(a, a_scale, w, w_scale, offsets, counts, E,
                                            rows_total, N, K, c, st, status);
  return gate_up ? launch<MOE_GEMM_SMALL, 1, kPow2>(a, a_scale, w, w_scale, offsets, counts,
                                                    E, rows_total, N, K, c, st, status)
                 : launch<MOE_GEMM_SMALL, 2, kPow2>(a, a_scale, w, w_scale, offsets, counts,
                                                    E, rows_total, N, K, c, st, status);
}

extern "C" int moe_gemm_large_tiles(long long rows_total, int N, int E) {
  if (rows_total <= 0 || N <= 0 || E <= 0) return -1;
  return use_big_tiles(rows_total, N, E) ? 1 : 0;
}

static constexpr int tile_rows(int bm, int, int, int, int) { return bm; }

extern "C" int moe_gemm_tile_rows(long long rows_total, int N, int K, int E,
                                  int packed_scales) {
  if (rows_total <= 0 || N <= 0 || K <= 0 || E <= 0) return -1;
  if (packed_scales && use_huge_tiles(rows_total, N, E)) return tile_rows(MOE_GEMM_HUGE);
  if (use_mid_tiles(rows_total, N, E)) return tile_rows(MOE_GEMM_MID);
  if (use_big_tiles(rows_total, N, E)) return tile_rows(MOE_GEMM_BIG);
  return use_short_tiles(rows_total, N, K, E) ? tile_rows(MOE_GEMM_SHORT)
                                              : tile_rows(MOE_GEMM_SMALL);
}

extern "C" moe_status_t moe_grouped_gemm_fp8(
    const uint8_t* a, const float* a_scale, const uint8_t* w,
    const float* w_scale, const int32_t* offsets, const int32_t* counts, int E,
    int rows_total, int N, int K, uint16_t* c, int32_t* status_dev,
    void* stream) {
  return grouped_gemm<false>(a, a_scale, w, w_scale, offsets, counts, E, rows_total, N, K, c,
                             status_dev, stream);
}

extern "C" moe_status_t moe_grouped_gemm_fp8_e8m0(
    const uint8_t* a, const uint32_t* a_scale, const uint8_t* w, const uint32_t* w_scale,
    const int32_t* offsets, const int32_t* counts, int E, int rows_total, int N, int K,
    uint16_t* c, int32_t* status_dev, void* stream) {
  return grouped_gemm<true>(a, reinterpret_cast<const float*>(a_scale), w,
                            reinterpret_cast<const float*>(w_scale), offsets, counts, E,
                            rows_total, N, K, c, status_dev, stream);
}

template <bool kPow2, bool kGather = false>
static moe_status_t gate_up_act(const uint8_t* a, const float* a_scale, const uint8_t* w13,
                                const float* w13_scale, const int32_t* offsets,
                                const int32_t* counts, int E, int rows_total, int I, int H,
                                uint8_t* q2, void* q2_scale, int32_t* status, void* stream,
                                const int32_t* row_src = nullptr, int src_rows = 0) {
  if (E <= 0 || E > MOE_MAX_EXPERTS || rows_total < 0 || I <= 0 || H <= 0)
    return MOE_INVALID_ARG;
  if (I % kBlock != 0 || H % kBK != 0) return MOE_UNSUPPORTED_SHAPE;
  if (2LL * I * H > 0x7ffff000LL) return MOE_UNSUPPORTED_SHAPE;   // one expert's W13 < 2 GB
  if (!scale_span_ok(rows_total, H, kPow2)) return MOE_UNSUPPORTED_SHAPE;
  if (!offsets || !counts || !w13 || !w13_scale) return MOE_INVALID_ARG;
  if (kGather) {
    const moe_status_t g = gather_args_ok(a, src_rows, row_src, H);
    if (g != MOE_OK) return g;
  }
  if (rows_total == 0) return MOE_OK;
  if ((!kGather && !a) || !a_scale || !q2 || !q2_scale) return MOE_INVALID_ARG;
  if (((uintptr_t)a | (uintptr_t)w13 | (uintptr_t)q2) & 15) return MOE_UNSUPPORTED_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int N = 2 * I;
  // the same host-side rule as the unfused gate/up GEMM
  const bool big = use_big_tiles(rows_total, N, E);
  // (gathered: the per-lane source offsets do not fit beside the 320-row
  // tile's accumulators and fused epilogue, so that call keeps 256 rows)
  if (kPow2 && !kGather && use_huge_tiles(rows_total, N, E))
    return launch<MOE_GEMM_HUGE, 4, true>(a, a_scale, w13, w13_scale, offsets, counts, E,
                                          rows_total, N, H, nullptr, st, status, q2, q2_scale);
  if (use_mid_tiles(rows_total, N, E))
    return launch<MOE_GEMM_MID, 4, kPow2, kGather>(a, a_scale, w13, w13_scale, offsets, counts,
                                                   E, rows_total, N, H, nullptr, st, status, q2,
                                                   q2_scale, row_src, src_rows);
  if (big)
    return launch<MOE_GEMM_BIG, 4, kPow2, kGather>(a, a_scale, w13, w13_scale, offsets, counts,
                                                   E, rows_total, N, H, nullptr, st, status, q2,
                                                   q2_scale, row_src, src_rows);
  return launch<MOE_GEMM_FUSED_SMALL, 4, kPow2, kGather>(a, a_scale, w13, w13_scale, offsets,
                                                         counts, E, rows_total, N, H, nullptr,
                                                         st, status, q2, q2_scale, row_src,
                                                         src_rows);
}

extern "C" moe_status_t moe_gate_up_act_fp8(const uint8_t* a, const float* a_scale,
                                            const uint8_t* w13, const float* w13_scale,
                                            const int32_t* offsets, const int32_t* counts,
                                            int E, int rows_total, int I, int H, uint8_t* q2,
                                            float* q2_scale, int32_t* status_dev,
                                            void* stream) {
  return gate_up_act<false>(a, a_scale, w13, w13_scale, offsets, counts, E, rows_total, I, H,
                            q2, q2_scale, status_dev, stream);
}

extern "C" moe_status_t moe_gate_up_act_fp8_e8m0(const uint8_t* a, const uint32_t* a_scale,
                                                 const uint8_t* w13, const uint32_t* w13_scale,
                                                 const int32_t* offsets, const int32_t* counts,
                                                 int E, int rows_total, int I, int H,
                                                 uint8_t* q2, uint32_t* q2_scale,
                                                 int32_t* status_dev, void* stream) {
  return gate_up_act<true>(a, reinterpret_cast<const float*>(a_scale), w13,
                           reinterpret_cast<const float*>(w13_scale), offsets, counts, E,
                           rows_total, I, H, q2, q2_scale, status_dev, stream);
}

extern "C" moe_status_t moe_grouped_gemm_fp8_gather(
    const uint8_t* x, int T, const int32_t* row_src, const float* a_scale, const uint8_t* w,
    const float* w_scale, const int32_t* offsets, const int32_t* counts, int E, int rows_total,
    int N, int K, uint16_t* c, int32_t* status_dev, void* stream) {
  return grouped_gemm<false, true>(x, a_scale, w, w_scale, offsets, counts, E, rows_total, N, K,
                                   c, status_dev, stream, row_src, T);
}

extern "C" moe_status_t moe_grouped_gemm_fp8_gather_e8m0(
    const uint8_t* x, int T, const int32_t* row_src, const uint32_t* a_scale, const uint8_t* w,
    const uint32_t* w_scale, const int32_t* offsets, const int32_t* counts, int E,
    int rows_total, int N, int K, uint16_t* c, int32_t* status_dev, void* stream) {
  return grouped_gemm<true, true>(x, reinterpret_cast<const float*>(a_scale), w,
                                  reinterpret_cast<const float*>(w_scale), offsets, counts, E,
                                  rows_total, N, K, c, status_dev, stream, row_src, T);
}

extern "C" moe_status_t moe_gate_up_act_fp8_gather(
    const uint8_t* x, int T, const int32_t* row_src, const float* a_scale, const uint8_t* w13,
    const float* w13_scale, const int32_t* offsets, const int32_t* counts, int E,
    int rows_total, int I, int H, uint8_t* q2, float* q2_scale, int32_t* status_dev,
    void* stream) {
  return gate_up_act<false, true>(x, a_scale, w13, w13_scale, offsets, counts, E, rows_total, I,
                                  H, q2, q2_scale, status_dev, stream, row_src, T);
}

extern "C" moe_status_t moe_gate_up_act_fp8_gather_e8m0(
    const uint8_t* x, int T, const int32_t* row_src, const uint32_t* a_scale,
    const uint8_t* w13, const uint32_t* w13_scale, const int32_t* offsets,
    const int32_t* counts, int E, int rows_total, int I, int H, uint8_t* q2,
    uint32_t* q2_scale, int32_t* status_dev, void* stream) {
  return gate_up_act<true, true>(x, reinterpret_cast<const float*>(a_scale), w13,
                                 reinterpret_cast<const float*>(w13_scale), offsets, counts, E,
                                 rows_total, I, H, q2, q2_scale, status_dev, stream, row_src, T);
}

extern "C" moe_status_t moe_gemm_fp8(const uint8_t* a, const float* a_scale, const uint8_t* w,
                                     const float* w_scale, int M, int N, int K, uint16_t* c,
                                     void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return MOE_INVALID_ARG;
  if (N % kBlock != 0 || K % kBK != 0) return MOE_UNSUPPORTED_SHAPE;
  if (!scale_span_ok(M, K, false)) return MOE_UNSUPPORTED_SHAPE;
  if (M == 0) return MOE_OK;
  if (!a || !a_scale || !w || !w_scale || !c) return MOE_INVALID_ARG;
  if (((uintptr_t)a | (uintptr_t)w | (uintptr_t)c) & 15) return MOE_UNSUPPORTED_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool big = use_big_tiles(M, N, 1);
  if (big)
    return launch<MOE_GEMM_BIG, 3>(a, a_scale, w, w_scale, nullptr, nullptr, 1, M, N, K, c,
                                   st, nullptr);
  return launch<MOE_GEMM_SMALL, 3>(a, a_scale, w, w_scale, nullptr, nullptr, 1, M, N, K, c,
                                   st, nullptr);
}
