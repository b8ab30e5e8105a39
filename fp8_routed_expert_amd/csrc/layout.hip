// Dispatch layout for the routed rows that reached this GPU: per-expert
// counts, segment offsets, a stable rank of every (token, pick) inside its
// expert, and the permuted copy of the FP8 activations and their scales.
//
// Receive side of DeepEP's token shuffle ("Deploying DeepSeek with PD
// Disaggregation and Large-Scale Expert Parallelism on 96 H100 GPUs",
// section 大规模专家并行 › 基于 DeepEP 的专家并行): the normal (prefill) mode
// feeds a contiguous grouped layout, the low-latency (decode, graph
// capturable) mode a fixed-capacity masked layout.
//
// Kernels (all stream-ordered, fixed grids, no host reads):
//   layout_count   one block per chunk of 4096 flat entries: LDS histogram
//   layout_scan    one block: per-chunk exclusive bases, counts, offsets
//   layout_fill    row_src / row_expert <- -1 over the whole buffer
//   layout_rank    one block per chunk: wave-ballot ranks in flat order,
//                  writes slot_of, row_src, row_expert
//   permute_rows   one wave per source token: reads x[t] once, writes it to
//                  each of the token's slots (16-byte accesses)
//   permute_scales the matching scales, 64 slots per workgroup transposed
//                  through LDS (contiguous reads and stores)
#include "device_common.hpp"

namespace moe {

constexpr int kLayoutThreads = 256;
constexpr int kLayoutRounds = 16;
constexpr int kChunk = kLayoutThreads * kLayoutRounds;   // flat entries per block
constexpr int kWaves = kLayoutThreads / 64;

__global__ __launch_bounds__(kLayoutThreads) void layout_count(
    const int32_t* __restrict__ idx, long long F, int E,
    int32_t* __restrict__ chunk_counts, int32_t* __restrict__ status) {
  extern __shared__ int32_t hist[];
  for (int i = threadIdx.x; i < E; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  long long base = (long long)blockIdx.x * kChunk;
  int bad = 0;
  for (int r = 0; r < kLayoutRounds; ++r) {
    long long f = base + r * kLayoutThreads + threadIdx.x;
    if (f < F) {
      int e = idx[f];
      if (e >= 0 && e < E)
        atomicAdd(&hist[e], 1);
      else if (e != -1)
        bad = 1;
    }
  }
  bad = __syncthreads_or(bad);
  for (int i = threadIdx.x; i < E; i += blockDim.x)
    chunk_counts[(long long)blockIdx.x * E + i] = hist[i];
  if (bad && threadIdx.x == 0) atomicOr(status, MOE_ERR_BAD_EXPERT);
}

__global__ __launch_bounds__(kLayoutThreads) void layout_scan(
    const int32_t* __restrict__ chunk_counts, int nchunks, int E, int layout,
    int align_m, int cap, int32_t* __restrict__ chunk_base,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  extern __shared__ int32_t tot[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int b = 0; b < nchunks; ++b) {
      long long i = (long long)b * E + e;
      chunk_base[i] = s;
      s += chunk_counts[i];
    }
    counts[e] = s;
    tot[e] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long o = 0;
    for (int e = 0; e < E; ++e) {
      if (layout == MOE_LAYOUT_MASKED) {
        offsets[e] = (int32_t)((long long)e * cap);
      } else {
        offsets[e] = (int32_t)(o > 0x7fffffffLL ? 0x7fffffffLL : o);
        o += ((long long)tot[e] + align_m - 1) / align_m * align_m;
      }
    }
    if (layout == MOE_LAYOUT_MASKED)
      offsets[E] = (int32_t)((long long)E * cap);
    else
      offsets[E] = (int32_t)(o > 0x7fffffffLL ? 0x7fffffffLL : o);
  }
}

__global__ void layout_fill(int32_t* __restrict__ row_src,
                            int32_t* __restrict__ row_expert, int rows_total) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
       i < rows_total; i += (long long)gridDim.x * blockDim.x) {
    row_src[i] = -1;
    row_expert[i] = -1;
  }
}

// Stable rank of every flat entry f = t*K + k inside its expert.  Each block
// owns one chunk and walks it in rounds of 256 consecutive entries; inside a
// wave, lanes with the same expert are found by ballots over the key bits,
// and a lane's rank is the number of lower lanes with its key.  Per-wave
// group sizes go through LDS (tagged with the round so they never need
// clearing) to order the four waves, and a running per-expert base carries
// the count across rounds, so ranks follow flat order exactly.
__global__ __launch_bounds__(kLayoutThreads) void layout_rank(
    const int32_t* __restrict__ idx, long long F, int K, int E, int key_bits,
    int layout, int rows_total, int cap, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ chunk_base, int32_t* __restrict__ slot_of,
    int32_t* __restrict__ row_src, int32_t* __restrict__ row_expert,
    int32_t* __restrict__ status) {
  extern __shared__ int32_t smem[];
  int32_t* run = smem;              // [E] running rank base
  int32_t* wcnt = smem + E;         // [kWaves][E] (round+1) << 8 | count
  int32_t* offs = wcnt + kWaves * E;  // [E] segment starts
  for (int i = threadIdx.x; i < E; i += blockDim.x) {
    run[i] = chunk_base[(long long)blockIdx.x * E + i];
    offs[i] = offsets[i];
    for (int w = 0; w < kWaves; ++w) wcnt[w * E + i] = 0;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const unsigned long long lt = (1ull << lane) - 1ull;
  long long base = (long long)blockIdx.x * kChunk;
  int overflow = 0;
  for (int r = 0; r < kLayoutRounds; ++r) {
    long long f = base + r * kLayoutThreads + threadIdx.x;
    int e = f < F ? idx[f] : -1;
    bool valid = e >= 0 && e < E;
    int key = valid ? e + 1 : 0;
    unsigned long long m = ~0ull;
    for (int b = 0; b < key_bits; ++b) {
      bool bit = (key >> b) & 1;
      unsigned long long bal = __ballot(bit);
      m &= bit ? bal : ~bal;
    }
    int lane_rank = __popcll(m & lt);
    int group = __popcll(m);
    bool leader = (m & lt) == 0;
    const int tag = (r + 1) << 8;
    if (valid && leader) wcnt[wave * E + e] = tag | group;
    __syncthreads();
    int pre = 0;
    bool last = true;
    int rank = 0;
    if (valid) {
      for (int w = 0; w < kWaves; ++w) {
        int v = wcnt[w * E + e];
        if ((v & ~0xff) == tag) {
          if (w < wave) pre += v & 0xff;
          if (w > wave) last = false;
        }
      }
      rank = run[e] + pre + lane_rank;
    }
    __syncthreads();
    if (valid && leader && last) run[e] += pre + group;
    if (f < F) {
      int slot = -1;
      if (valid) {
        long long s = (long long)offs[e] + rank;
        bool fits = layout == MOE_LAYOUT_MASKED ? rank < cap : s < rows_total;
        if (fits && s >= 0 && s < rows_total) {
          slot = (int)s;
          row_src[slot] = (int32_t)(f / K);
          row_expert[slot] = e;
        } else {
          overflow = 1;
        }
      }
      slot_of[f] = slot;
    }
  }
  overflow = __syncthreads_or(overflow);
  if (overflow && threadIdx.x == 0) atomicOr(status, MOE_ERR_OVERFLOW);
}

// One wave per source token: the token's row is read from HBM once (16-byte
// loads, 64 lanes side by side, all of a row's loads in flight together)
// and written to every slot it was given.
constexpr int kPermChunks = 8;   // 16-byte chunks per lane per pass (H <= 8192 in one pass)

__global__ __launch_bounds__(256) void permute_rows(
    const uint8_t* __restrict__ x, const int32_t* __restrict__ slot_of, int T, int K, int H,
    int rows_total, uint8_t* __restrict__ a) {
  const int lane = threadIdx.x & 63;
  const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // the token's slots and its first chunks are requested together; only the
  // stores wait for the slots
  const int s = lane < K ? slot_of[t * K + lane] : -1;
  const int n16 = H >> 4;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * H);
  for (int c0 = lane; c0 < n16; c0 += 64 * kPermChunks) {
    uint4 v[kPermChunks];
#pragma unroll
    for (int u = 0; u < kPermChunks; ++u) {
      const int c = c0 + u * 64;
      v[u] = src[c < n16 ? c : 0];   // past the row: re-read chunk 0, not stored
    }
    unsigned long long m = __ballot(s >= 0 && s < rows_total);
    while (m) {
      const int k = __ffsll((long long)m) - 1;
      m &= m - 1;
      const int slot = __builtin_amdgcn_readlane(s, k);
      uint4* dst = reinterpret_cast<uint4*>(a + (long long)slot * H);
#pragma unroll
      for (int u = 0; u < kPermChunks; ++u) {
        const int c = c0 + u * 64;
        if (c < n16) dst[c] = v[u];
      }
    }
  }
}

// Scales in the permuted, K-block-major layout: a_scale[kb, slot] =
// x_scale[row_src[slot], kb].  A workgroup takes 64 consecutive slots and
// transposes through LDS: each wave reads whole source scale rows (64
// consecutive block scales of one token) and writes 64 consecutive slots of
// one block column, so both sides are contiguous runs.
constexpr int kScTile = 64;

__global__ __launch_bounds__(256) void permute_scales(
    const float* __restrict__ x_scale, const int32_t* __restrict__ row_src, int T, int hb,
    int rows_total, float* __restrict__ a_scale) {
  __shared__ float tile[64][kScTile + 1];
  __shared__ int src_of[kScTile];
  const int slot0 = blockIdx.x * kScTile;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (threadIdx.x < kScTile) {
    const int slot = slot0 + threadIdx.x;
    const int src = slot < rows_total ? row_src[slot] : -1;
    src_of[threadIdx.x] = (src >= 0 && src < T) ? src : -1;
  }
  __syncthreads();
  for (int kb0 = 0; kb0 < hb; kb0 += 64) {
    const int kb = kb0 + lane;
#pragma unroll
    for (int r = 0; r < kScTile; r += 4) {
      const int src = src_of[r + wv];
      if (src >= 0 && kb < hb) tile[lane][r + wv] = x_scale[(long long)src * hb + kb];
    }
    __syncthreads();
    const bool live = src_of[lane] >= 0;
    const long long slot = slot0 + lane;
    for (int c = wv; c < 64 && kb0 + c < hb; c += 4)
      if (live) a_scale[(long long)(kb0 + c) * rows_total + slot] = tile[c][lane];
    __syncthreads();
  }
}

static int key_bits_for(int E) {
  int b = 0;
  while ((1 << b) < E + 1) ++b;
  return b;
}

static long long n_chunks(int T, int K) {
  long long F = (long long)T * K;
  return (F + kChunk - 1) / kChunk;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_layout_workspace_bytes(int T, int K, int E) {
  if (T < 0 || K <= 0 || E <= 0) return 0;
  long long nc = n_chunks(T, K);
  if (nc < 1) nc = 1;
  return (size_t)(2 * nc * E) * sizeof(int32_t);
}

extern "C" moe_status_t moe_dispatch_layout(
    const int32_t* topk_idx, const uint8_t* x, const float* x_scale, int T,
    int K, int E, int H, int layout, int align_m, int rows, int32_t* counts,
    int32_t* offsets, int32_t* slot_of, int32_t* row_src, int32_t* row_expert,
    uint8_t* a, float* a_scale, void* workspace, size_t workspace_bytes,
    int32_t* status_dev, void* stream) {
  if (T < 0 || K <= 0 || K > MOE_MAX_TOPK || E <= 0 || E > MOE_MAX_EXPERTS ||
      H <= 0 || rows < 0)
    return MOE_INVALID_ARG;
  if (layout != MOE_LAYOUT_CONTIGUOUS && layout != MOE_LAYOUT_MASKED)
    return MOE_INVALID_ARG;
  if (layout == MOE_LAYOUT_CONTIGUOUS && align_m < 1) return MOE_INVALID_ARG;
  if (H % kBlock != 0) return MOE_UNSUPPORTED_SHAPE;
  if (!counts || !offsets || !status_dev || !workspace) return MOE_INVALID_ARG;
  long long rows_total =
      layout == MOE_LAYOUT_MASKED ? (long long)E * rows : (long long)rows;
  if (rows_total > 0x7fffffffLL) return MOE_UNSUPPORTED_SHAPE;
  if ((long long)T * K > 0x7fffffffLL) return MOE_UNSUPPORTED_SHAPE;
  if (workspace_bytes < moe_layout_workspace_bytes(T, K, E))
    return MOE_INVALID_ARG;
  if (T > 0 && (!topk_idx || !x || !x_scale || !slot_of)) return MOE_INVALID_ARG;
  if (rows_total > 0 && (!row_src || !row_expert || !a || !a_scale))
    return MOE_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)a) & 15) return MOE_UNSUPPORTED_SHAPE;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const long long F = (long long)T * K;
  long long nc = n_chunks(T, K);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(workspace);
  int32_t* chunk_base = chunk_counts + (nc < 1 ? 1 : nc) * E;
  const int cap = layout == MOE_LAYOUT_MASKED ? rows : 0;

  if (nc > 0)
    hipLaunchKernelGGL(layout_count, dim3((unsigned)nc), dim3(kLayoutThreads),
                       E * sizeof(int32_t), st, topk_idx, F, E, chunk_counts,
                       status_dev);
  hipLaunchKernelGGL(layout_scan, dim3(1), dim3(kLayoutThreads),
                     E * sizeof(int32_t), st, chunk_counts, (int)nc, E, layout,
                     align_m, cap, chunk_base, counts, offsets);
  if (rows_total > 0) {
    long long blocks = (rows_total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(layout_fill, dim3((unsigned)blocks), dim3(256), 0, st,
                       row_src, row_expert, (int)rows_total);
  }
  if (nc > 0)
    hipLaunchKernelGGL(layout_rank, dim3((unsigned)nc), dim3(kLayoutThreads),
                       (2 + kWaves) * E * sizeof(int32_t), st, topk_idx, F, K,
                       E, key_bits_for(E), layout, (int)rows_total, cap,
                       offsets, chunk_base, slot_of, row_src, row_expert,
                       status_dev);
  if (T > 0 && rows_total > 0) {
    hipLaunchKernelGGL(permute_rows, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, x,
                       slot_of, T, K, H, (int)rows_total, a);
    hipLaunchKernelGGL(permute_scales, dim3((unsigned)((rows_total + kScTile - 1) / kScTile)),
                       dim3(256), 0, st, x_scale, row_src, T, H / kBlock, (int)rows_total,
                       a_scale);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
