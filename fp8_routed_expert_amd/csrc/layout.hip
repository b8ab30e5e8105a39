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
//   layout_count   one block per chunk of 1024 flat entries: LDS histogram
//                  (ballot-grouped atomics); also row_src / row_expert <- -1
//   layout_scan    one block: per-chunk exclusive bases, counts, offsets
//                  (skipped when chunks x experts is small: layout_rank
//                  then computes them itself)
//   layout_rank    one block per chunk: wave-ballot ranks in flat order,
//                  writes slot_of, row_src, row_expert
//   permute_kernel one launch of two kinds of workgroups:
//                  scales: 64 slots per workgroup transposed through LDS
//                  (contiguous reads and stores);
//                  rows: one wave per piece of a source row, which reads
//                  x[t] once and writes it to each of the token's slots
//                  (16-byte accesses)
#include <mutex>

#include "device_common.hpp"

namespace moe {

constexpr int kLayoutThreads = 256;
constexpr int kLayoutRounds = 4;
constexpr int kChunk = kLayoutThreads * kLayoutRounds;   // flat entries per block
constexpr int kWaves = kLayoutThreads / 64;
constexpr int kScanThreads = 1024;
constexpr long long kFoldMax = 8192;   // chunk x expert counts a rank block sums itself

// Lanes of the wave whose key equals this lane's (ballots over the key bits).
__device__ __forceinline__ unsigned long long match_key(int key, int key_bits) {
  unsigned long long m = __ballot(1);
  for (int b = 0; b < key_bits; ++b) {
    const bool bit = (key >> b) & 1;
    const unsigned long long bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

// Per-chunk expert histogram.  A chunk's entries are requested at once;
// lanes of a wave with the same expert are grouped by ballots and the lowest
// of them adds the group size, so there is one LDS atomic per expert per
// wave and round.  The same grid also sets row_src / row_expert to -1 over
// the whole buffer (layout_rank, the next kernel, overwrites filled rows).
__global__ __launch_bounds__(kLayoutThreads) void layout_count(
    const int32_t* __restrict__ idx, long long F, int E, int key_bits,
    int32_t* __restrict__ chunk_counts, int32_t* __restrict__ row_src,
    int32_t* __restrict__ row_expert, int rows_total, int32_t* __restrict__ status) {
  extern __shared__ int32_t hist[];
  const long long base = (long long)blockIdx.x * kChunk;
  int ev[kLayoutRounds];
#pragma unroll
  for (int r = 0; r < kLayoutRounds; ++r) {
    const long long f = base + r * kLayoutThreads + threadIdx.x;
    ev[r] = f < F ? idx[f] : -1;
  }
  for (int i = threadIdx.x; i < E; i += blockDim.x) hist[i] = 0;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < rows_total;
       i += (long long)gridDim.x * blockDim.x) {
    row_src[i] = -1;
    row_expert[i] = -1;
  }
  __syncthreads();
  const unsigned long long lt = (1ull << (threadIdx.x & 63)) - 1ull;
  int bad = 0;
#pragma unroll
  for (int r = 0; r < kLayoutRounds; ++r) {
    const int e = ev[r];
    const bool valid = e >= 0 && e < E;
    if (!valid && e != -1) bad = 1;
    const unsigned long long m = match_key(valid ? e + 1 : 0, key_bits);
    if (valid && (m & lt) == 0) atomicAdd(&hist[e], __popcll(m));
  }
  bad = __syncthreads_or(bad);
  for (int i = threadIdx.x; i < E; i += blockDim.x)
    chunk_counts[(long long)blockIdx.x * E + i] = hist[i];
  if (bad && threadIdx.x == 0) atomicOr(status, MOE_ERR_BAD_EXPERT);
}

// Exclusive prefix over chunks of every expert's count (chunk_base), the
// totals (counts) and the segment starts (offsets).  Each expert gets a
// group of `group` lanes (64 when E <= 16); a lane sums its own range of
// chunks, the group scans the partial sums with shuffles, and the lane then
// writes its range's bases.  Offsets are a block-wide scan over experts of
// the totals rounded up to align_m (contiguous) or e * cap (masked).
__global__ __launch_bounds__(kScanThreads) void layout_scan(
    const int32_t* __restrict__ chunk_counts, int nchunks, int E, int group, int layout,
    int align_m, int cap, int32_t* __restrict__ chunk_base,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[MOE_MAX_EXPERTS];
  __shared__ long long wsum[kScanThreads / 64];
  const int lg = threadIdx.x % group, grp = threadIdx.x / group;
  const int ngrp = kScanThreads / group;
  const int per = (nchunks + group - 1) / group;
  const int b0 = min(lg * per, nchunks), b1 = min(b0 + per, nchunks);
  for (int e0 = 0; e0 < E; e0 += ngrp) {   // uniform trip count: shuffles stay converged
    const int e = e0 + grp;
    const bool live = e < E;
    int local = 0;
    if (live) {
#pragma unroll 8
      for (int b = b0; b < b1; ++b) local += chunk_counts[(long long)b * E + e];
    }
    int incl = local;
    for (int d = 1; d < group; d <<= 1) {
      const int v = __shfl_up(incl, d, group);
      if (lg >= d) incl += v;
    }
    if (live) {
      int run = incl - local;
#pragma unroll 8
      for (int b = b0; b < b1; ++b) {
        const long long i = (long long)b * E + e;
        const int c = chunk_counts[i];
        chunk_base[i] = run;
        run += c;
      }
      if (lg == group - 1) {
        counts[e] = incl;
        tot[e] = incl;
      }
    }
  }
  __syncthreads();
  const int e = threadIdx.x;   // E <= MOE_MAX_EXPERTS == kScanThreads
  if (layout == MOE_LAYOUT_MASKED) {
    if (e < E) offsets[e] = (int32_t)((long long)e * cap);
    if (e == 0) offsets[E] = (int32_t)((long long)E * cap);
    return;
  }
  const long long mine =
      e < E ? ((long long)tot[e] + align_m - 1) / align_m * align_m : 0;
  long long incl = mine;
  for (int d = 1; d < 64; d <<= 1) {
    const long long v = __shfl_up(incl, d, 64);
    if ((threadIdx.x & 63) >= d) incl += v;
  }
  if ((threadIdx.x & 63) == 63) wsum[threadIdx.x >> 6] = incl;
  __syncthreads();
  long long before = 0;
  for (int w = 0; w < (threadIdx.x >> 6); ++w) before += wsum[w];
  incl += before;
  const long long lim = 0x7fffffffLL;
  if (e < E) offsets[e] = (int32_t)(incl - mine > lim ? lim : incl - mine);
  if (e == E - 1) offsets[E] = (int32_t)(incl > lim ? lim : incl);
}

// Stable rank of every flat entry f = t*K + k inside its expert.  Each block
// owns one chunk and walks it in rounds of 256 consecutive entries; inside a
// wave, lanes with the same expert are found by ballots over the key bits,
// and a lane's rank is the number of lower lanes with its key.  Per-wave
// group sizes go through LDS (tagged with the round so they never need
// clearing) to order the four waves, and a running per-expert base carries
// the count across rounds, so ranks follow flat order exactly.
//
// fold != 0 (few chunks, E <= kLayoutThreads): layout_scan is not launched.
// Each block sums the chunk counts itself -- all of them for the expert
// totals and segment starts, those of the earlier chunks for its own bases
// -- and block 0 writes counts and offsets; the values equal layout_scan's.
__global__ __launch_bounds__(kLayoutThreads) void layout_rank(
    const int32_t* __restrict__ idx, long long F, int K, int E, int key_bits,
    int layout, int rows_total, int cap, int32_t* __restrict__ offsets,
    const int32_t* __restrict__ chunk_base, int32_t* __restrict__ slot_of,
    int32_t* __restrict__ row_src, int32_t* __restrict__ row_expert,
    int32_t* __restrict__ status, int fold, const int32_t* __restrict__ chunk_counts,
    int nchunks, int align_m, int32_t* __restrict__ counts) {
  extern __shared__ int32_t smem[];
  int32_t* run = smem;              // [E] running rank base
  int32_t* wcnt = smem + E;         // [kWaves][E] (round+1) << 8 | count
  int32_t* offs = wcnt + kWaves * E;  // [E] segment starts
  int32_t* tot = offs + E;          // [E] expert totals (fold)
  __shared__ long long wsum[kWaves];
  for (int i = threadIdx.x; i < E; i += blockDim.x) {
    if (fold) {
      run[i] = 0;
      tot[i] = 0;
    } else {
      run[i] = chunk_base[(long long)blockIdx.x * E + i];
      offs[i] = offsets[i];
    }
    for (int w = 0; w < kWaves; ++w) wcnt[w * E + i] = 0;
  }
  __syncthreads();
  if (fold) {
    // kLayoutThreads / E threads per expert, each summing a strided share of
    // the chunks in registers, then one LDS add each
    const int tpe = kLayoutThreads / E;
    if ((int)threadIdx.x < tpe * E) {
      const int e = threadIdx.x % E;
      int sum = 0, before = 0;
      for (int c = threadIdx.x / E; c < nchunks; c += tpe) {
        const int v = chunk_counts[(long long)c * E + e];
        sum += v;
        if (c < (int)blockIdx.x) before += v;
      }
      atomicAdd(&tot[e], sum);
      atomicAdd(&run[e], before);
    }
    __syncthreads();
    // segment starts: exclusive scan over the experts (one per thread)
    const int e = threadIdx.x;
    long long mine = 0;
    if (e < E)
      mine = layout == MOE_LAYOUT_MASKED ? (long long)cap
                                         : ((long long)tot[e] + align_m - 1) / align_m * align_m;
    long long incl = mine;
    for (int d = 1; d < 64; d <<= 1) {
      const long long v = __shfl_up(incl, d, 64);
      if ((threadIdx.x & 63) >= d) incl += v;
    }
    if ((threadIdx.x & 63) == 63) wsum[threadIdx.x >> 6] = incl;
    __syncthreads();
    for (int w = 0; w < (int)(threadIdx.x >> 6); ++w) incl += wsum[w];
    const long long lim = 0x7fffffffLL;
    if (e < E) {
      offs[e] = (int32_t)(incl - mine > lim ? lim : incl - mine);
      if (blockIdx.x == 0) {
        counts[e] = tot[e];
        offsets[e] = offs[e];
        if (e == E - 1) offsets[E] = (int32_t)(incl > lim ? lim : incl);
      }
    }
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const unsigned long long lt = (1ull << lane) - 1ull;
  long long base = (long long)blockIdx.x * kChunk;
  int ev[kLayoutRounds];
#pragma unroll
  for (int r = 0; r < kLayoutRounds; ++r) {
    const long long f = base + r * kLayoutThreads + threadIdx.x;
    ev[r] = f < F ? idx[f] : -1;
  }
  int overflow = 0;
#pragma unroll
  for (int r = 0; r < kLayoutRounds; ++r) {
    long long f = base + r * kLayoutThreads + threadIdx.x;
    int e = ev[r];
    bool valid = e >= 0 && e < E;
    int key = valid ? e + 1 : 0;
    const unsigned long long m = match_key(key, key_bits);
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
#ifndef MOE_PERM_CHUNKS
#define MOE_PERM_CHUNKS 2
#endif
constexpr int kPermChunks = MOE_PERM_CHUNKS;   // 16-byte chunks per lane

// One wave per piece of a source row: the row's H/16 chunks are cut into
// `pieces` pieces of at most `plen` <= 64 * kPermChunks chunks (H = 7168:
// four pieces of 112), so a row is read once by a few waves that each hold
// their piece in registers and store it to every slot of the token.  The
// token's slots and the piece are requested together; only the stores wait
// for the slots.
__device__ __forceinline__ void permute_rows(
    int blk, const uint8_t* __restrict__ x, const int32_t* __restrict__ slot_of, int T, int K,
    int H, int pieces, int plen, int rows_total, uint8_t* __restrict__ a) {
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blk * 4 + (threadIdx.x >> 6);
  const long long t = w / pieces;
  if (t >= T) return;
  const int n16 = H >> 4;
  const int c0 = (int)(w - t * pieces) * plen;
  const int cend = min(c0 + plen, n16);
  const int s = lane < K ? slot_of[t * K + lane] : -1;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * H);
  uint4 v[kPermChunks];
#pragma unroll
  for (int u = 0; u < kPermChunks; ++u) {
    const int c = c0 + lane + u * 64;
    v[u] = src[c < cend ? c : c0];   // past the piece: re-read its first chunk, not stored
  }
  unsigned long long m = __ballot(s >= 0 && s < rows_total);
  while (m) {
    const int k = __ffsll((long long)m) - 1;
    m &= m - 1;
    const int slot = __builtin_amdgcn_readlane(s, k);
    uint4* dst = reinterpret_cast<uint4*>(a + (long long)slot * H);
#pragma unroll
    for (int u = 0; u < kPermChunks; ++u) {
      const int c = c0 + lane + u * 64;
      if (c < cend) dst[c] = v[u];
    }
  }
}

// Scales in the permuted, K-block-major layout: a_scale[kb, slot] =
// x_scale[row_src[slot], kb], moved as 4-byte words (an fp32 scale, or four
// packed E8M0 exponents; hb is the number of words per source row).  A workgroup takes 64 consecutive slots and
// transposes through LDS: each wave reads whole source scale rows (64
// consecutive block scales of one token) and writes 64 consecutive slots of
// one block column, so both sides are contiguous runs.
constexpr int kScTile = 64;

__device__ __forceinline__ void permute_scales(
    int blk, const uint32_t* __restrict__ x_scale, const int32_t* __restrict__ row_src, int T,
    int hb, int rows_total, uint32_t* __restrict__ a_scale) {
  __shared__ uint32_t tile[64][kScTile + 1];
  __shared__ int src_of[kScTile];
  const int slot0 = blk * kScTile;
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

// Rows and scales in one launch: the first scale_blocks workgroups permute
// the scales (latency-bound, few bytes), the rest the rows (bandwidth-bound),
// so the two overlap instead of running back to back.
__global__ __launch_bounds__(256) void permute_kernel(
    const uint8_t* __restrict__ x, const int32_t* __restrict__ slot_of, int T, int K, int H,
    int pieces, int plen, int rows_total, uint8_t* __restrict__ a,
    const uint32_t* __restrict__ x_scale, const int32_t* __restrict__ row_src, int hw,
    uint32_t* __restrict__ a_scale, int scale_blocks) {
  const int b = (int)blockIdx.x;
  if (b < scale_blocks)
    permute_scales(b, x_scale, row_src, T, hw, rows_total, a_scale);
  else
    permute_rows(b - scale_blocks, x, slot_of, T, K, H, pieces, plen, rows_total, a);
}

static int key_bits_for(int E) {
  int b = 0;
  while ((1 << b) < E + 1) ++b;
  return b;
}

// Lanes per expert in layout_scan: the block's 1024 threads shared out over
// the experts (rounded up to a power of two), at most one wave per expert.
static int scan_group(int E) {
  int p = 1;
  while (p < E) p <<= 1;
  const int g = kScanThreads / p;
  return g > 64 ? 64 : (g < 1 ? 1 : g);
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

// hw = 4-byte scale words per source row (H/128 fp32 scales, or H/512
// rounded up of packed E8M0 words).
static moe_status_t dispatch(
    const int32_t* topk_idx, const uint8_t* x, const uint32_t* x_scale, int T,
    int K, int E, int H, int hw, int layout, int align_m, int rows, int32_t* counts,
    int32_t* offsets, int32_t* slot_of, int32_t* row_src, int32_t* row_expert,
    uint8_t* a, uint32_t* a_scale, void* workspace, size_t workspace_bytes,
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
  // a == nullptr: the rows are not copied (the *_gather GEMM calls read them
  // from x through row_src); indices and permuted scales are still written
  if (T > 0 && (!topk_idx || (a && !x) || !x_scale || !slot_of)) return MOE_INVALID_ARG;
  if (rows_total > 0 && (!row_src || !row_expert || !a_scale))
    return MOE_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)a) & 15) return MOE_UNSUPPORTED_SHAPE;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const long long F = (long long)T * K;
  long long nc = n_chunks(T, K);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(workspace);
  int32_t* chunk_base = chunk_counts + (nc < 1 ? 1 : nc) * E;
  const int cap = layout == MOE_LAYOUT_MASKED ? rows : 0;

  const int ncl = (int)(nc < 1 ? 1 : nc);   // count always runs: it also clears row_src
  hipLaunchKernelGGL(layout_count, dim3((unsigned)ncl), dim3(kLayoutThreads),
                     E * sizeof(int32_t), st, topk_idx, F, E, key_bits_for(E), chunk_counts,
                     row_src, row_expert, (int)rows_total, status_dev);
  // few chunks: the rank blocks compute the scan themselves (one launch less)
  const int fold = nc > 0 && E <= kLayoutThreads && nc * (long long)E <= kFoldMax;
  if (!fold)
    hipLaunchKernelGGL(layout_scan, dim3(1), dim3(kScanThreads), 0, st, chunk_counts, ncl, E,
                       scan_group(E), layout, align_m, cap, chunk_base, counts, offsets);
  if (nc > 0)
    hipLaunchKernelGGL(layout_rank, dim3((unsigned)nc), dim3(kLayoutThreads),
                       (3 + kWaves) * E * sizeof(int32_t), st, topk_idx, F, K,
                       E, key_bits_for(E), layout, (int)rows_total, cap,
                       offsets, chunk_base, slot_of, row_src, row_expert,
                       status_dev, fold, chunk_counts, ncl, align_m, counts);
  if (T > 0 && rows_total > 0) {
    const int n16 = H / 16;
    const int pieces = (n16 + 64 * kPermChunks - 1) / (64 * kPermChunks);
    const int plen = (n16 + pieces - 1) / pieces;
    const long long waves = (long long)T * pieces;
    const long long row_blocks = a ? (waves + 3) / 4 : 0;
    const long long scale_blocks = (rows_total + kScTile - 1) / kScTile;
    if (row_blocks + scale_blocks > 0x7fffffffLL) return MOE_UNSUPPORTED_SHAPE;
    hipLaunchKernelGGL(permute_kernel, dim3((unsigned)(row_blocks + scale_blocks)), dim3(256),
                       0, st, x, slot_of, T, K, H, pieces, plen, (int)rows_total, a, x_scale,
                       row_src, hw, a_scale, (int)scale_blocks);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}

extern "C" moe_status_t moe_dispatch_layout(
    const int32_t* topk_idx, const uint8_t* x, const float* x_scale, int T, int K, int E,
    int H, int layout, int align_m, int rows, int32_t* counts, int32_t* offsets,
    int32_t* slot_of, int32_t* row_src, int32_t* row_expert, uint8_t* a, float* a_scale,
    void* workspace, size_t workspace_bytes, int32_t* status_dev, void* stream) {
  return dispatch(topk_idx, x, reinterpret_cast<const uint32_t*>(x_scale), T, K, E, H,
                  H / kBlock, layout, align_m, rows, counts, offsets, slot_of, row_src,
                  row_expert, a, reinterpret_cast<uint32_t*>(a_scale), workspace,
                  workspace_bytes, status_dev, stream);
}

// ---------------------------------------------------------------------
// Allocation-free dispatch.  The per-chunk histograms and bases live in a
// file-scope device array instead of a caller workspace; each GPU holds its
// own copy for the life of the process.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up
// once per device with hipGetSymbolAddress and only that address is used.
// The array needs no clearing: layout_count writes every histogram entry
// the later kernels read, and layout_scan every base.
constexpr size_t kScratchBytes = size_t(1) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static moe_status_t scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_HIP_ERROR;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_HIP_ERROR;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

extern "C" moe_status_t moe_dispatch_layout_noalloc(
    const int32_t* topk_idx, const uint8_t* x, const float* x_scale, int T, int K, int E,
    int H, int layout, int align_m, int rows, int32_t* counts, int32_t* offsets,
    int32_t* slot_of, int32_t* row_src, int32_t* row_expert, uint8_t* a, float* a_scale,
    int32_t* status_dev, void* stream) {
  if (T < 0 || K <= 0 || K > MOE_MAX_TOPK || E <= 0 || E > MOE_MAX_EXPERTS)
    return MOE_INVALID_ARG;
  if (moe_layout_workspace_bytes(T, K, E) > kScratchBytes) return MOE_SCRATCH_LIMIT;
  void* ws = nullptr;
  const moe_status_t r = scratch_on_current_device(&ws);
  if (r != MOE_OK) return r;
  return dispatch(topk_idx, x, reinterpret_cast<const uint32_t*>(x_scale), T, K, E, H,
                  H / kBlock, layout, align_m, rows, counts, offsets, slot_of, row_src,
                  row_expert, a, reinterpret_cast<uint32_t*>(a_scale), ws, kScratchBytes,
                  status_dev, stream);
}

extern "C" moe_status_t moe_dispatch_layout_e8m0(
    const int32_t* topk_idx, const uint8_t* x, const uint32_t* x_scale, int T, int K, int E,
    int H, int layout, int align_m, int rows, int32_t* counts, int32_t* offsets,
    int32_t* slot_of, int32_t* row_src, int32_t* row_expert, uint8_t* a, uint32_t* a_scale,
    void* workspace, size_t workspace_bytes, int32_t* status_dev, void* stream) {
  return dispatch(topk_idx, x, x_scale, T, K, E, H, (H / kBlock + 3) / 4, layout, align_m,
                  rows, counts, offsets, slot_of, row_src, row_expert, a, a_scale, workspace,
                  workspace_bytes, status_dev, stream);
}
