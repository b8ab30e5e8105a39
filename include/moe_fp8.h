/*
 * moe_fp8.h — C ABI of the MI355X (gfx950) FP8 routed-expert MoE library.
 *
 * One GPU's share of a routed-expert MoE layer under expert parallelism: the
 * token-rows already dispatched to this GPU's local experts are counted per
 * expert, prefix-summed and permuted (the receive side of DeepEP's token
 * shuffle), pushed through two FP8 grouped GEMMs with a SiLU-gated
 * re-quantisation between them (the DeepGEMM grouped GEMMs), and summed back
 * per source token with their top-k weights (the combine).
 *
 * Sources:
 *   [H100-EP] "Deploying DeepSeek with PD Disaggregation and Large-Scale
 *             Expert Parallelism on 96 H100 GPUs", section 大规模专家并行
 *             (large-scale expert parallelism): subsections 基于 DeepEP 的
 *             专家并行 (DeepEP dispatch/combine; normal mode for prefill,
 *             low-latency CUDA-graph-compatible mode for decode, and the
 *             mode-compatibility table) and DeepGEMM 集成 (two FP8 grouped
 *             GEMM functions for MoE, one per inference phase).
 *   [GB200]   "Deploying DeepSeek on GB200 NVL72 with PD and Large Scale EP
 *             (Part I): 2.7x Higher Decoding Throughput", sections 怎么做的
 *             (how it is done) and 方法实现细节 (method details): FP8 GEMM
 *             library whose API quantises and packs input scales; DeepEP
 *             shuffles tokens to routed experts.
 * The pages give no kernel-level definitions; block sizes, rounding and the
 * activation are readings, stated with each call.
 *
 * Conventions for every call
 *   - All array arguments are device pointers to caller-owned memory; the
 *     library never allocates, frees or synchronises, and keeps no pointer
 *     after returning.  Work is enqueued on `stream` (a hipStream_t; NULL is
 *     the legacy default stream).  Every call is safe inside hipGraph stream
 *     capture (fixed grids, no host reads of device data, no memset nodes).
 *   - FP8 is OCP E4M3FN (max 448), stored one byte per value.  bf16 is stored
 *     as uint16_t bit patterns.  Scales are fp32.
 *   - Activation scales live K-block-major ("MN-major"): for a buffer of
 *     `rows` rows and hidden size H the scale of row m, block kb (covering
 *     columns [128 kb, 128 kb + 128)) is at scale[kb * rows + m].  Source
 *     activation scales (x_scale) are row-major [T, H/128].  Weight scales
 *     are [E, N/128, K/128] row-major, one per 128x128 block.
 *   - Matrices are row-major; weights are [E, N, K] with K contiguous.
 *   - Pointers must be 16-byte aligned; H, I, N, K must be multiples of 128.
 *   - Host-side argument errors return a non-zero moe_status_t and launch
 *     nothing.  Data errors found on the device (bad expert id, a row that
 *     does not fit, an index outside a buffer) are OR-ed into the caller's
 *     int32 word *status_dev (caller zeroes it; the library never reads it
 *     back) and the offending entry is skipped deterministically.
 *   - A valid permuted row is one inside an expert segment: rows
 *     [offsets[e], offsets[e] + min(counts[e], offsets[e+1] - offsets[e]))
 *     clipped to the buffer.  Outputs for other rows are unspecified.
 */
#ifndef MOE_FP8_H_
#define MOE_FP8_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;

#define MOE_OK 0
#define MOE_INVALID_ARG 1       /* null pointer, negative size, bad enum   */
#define MOE_UNSUPPORTED_SHAPE 2 /* size not a multiple of 128, misaligned   */
#define MOE_HIP_ERROR 3         /* a kernel launch failed                   */
#define MOE_SCRATCH_LIMIT 4     /* beyond the allocation-free call's scratch */

#define MOE_LAYOUT_CONTIGUOUS 0 /* prefill: expert segments stacked along M */
#define MOE_LAYOUT_MASKED 1     /* decode: fixed [E, C, .] + device counts  */

/* bits OR-ed into *status_dev */
#define MOE_ERR_BAD_EXPERT 1 /* topk id outside [-1, E): entry skipped     */
#define MOE_ERR_OVERFLOW 2   /* row did not fit: dropped in stable order  */
#define MOE_ERR_BAD_INDEX 4  /* slot / offset outside a buffer: skipped   */

#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 64

/* ABI version of this header (increments on any signature change). */
int moe_abi_version(void);

/* Static text for a status code; never NULL. */
const char* moe_status_string(moe_status_t status);

/* Bytes of device workspace moe_dispatch_layout needs for T tokens with K
 * top-k columns and E local experts (per-chunk expert histograms). */
size_t moe_layout_workspace_bytes(int T, int K, int E);

/* Whether the grouped GEMM calls (moe_grouped_gemm_fp8, moe_gate_up_act_fp8,
 * their _e8m0 forms; N = 2I for the gate/up projection) and moe_gemm_fp8
 * (E = 1, rows_total = M) run a problem of this size with large tiles (1:
 * 256 x 256, or 320 x 256 or 192 x 256 at the sizes where
 * moe_gemm_tile_rows says so) or small ones (0: 128 x 128, or 64 x 128
 * where moe_gemm_tile_rows says 64; 128 x 256 for the fused gate/up +
 * activation).  A host-side rule of the sizes alone, so
 * it is the same under graph capture; the rule itself is stated where it is
 * implemented.  Returns -1 for negative or zero sizes.  Callers use it to
 * choose between the fused and the separate gate/up + activation calls. */
int moe_gemm_large_tiles(long long rows_total, int N, int E);

/* The row height of the output tiles the grouped calls use for a product
 * of N outputs over K inputs (gate/up: N = 2I, K = H; down: N = H, K = I):
 * 320, 256, 192, 128 or 64.  packed_scales != 0 asks about the _e8m0 calls
 * (the only ones with 320-row tiles, which the gathered fused call does not
 * take: it keeps 256 there), 0 about the fp32-scale calls.  192 marks the
 * sizes whose large tiles fit one round on the CUs either way (decode
 * shares); 64 the gate/up products (K > N) of buffers with at most 128 rows
 * per expert on small tiles (the masked decode layout), which the
 * moe_grouped_gemm_fp8 calls run with 64-row tiles and the fused call with
 * its 128 x 256 ones.  moe_gemm_fp8 always uses 256 rows when
 * moe_gemm_large_tiles is 1.  -1 for negative or zero sizes. */
int moe_gemm_tile_rows(long long rows_total, int N, int K, int E, int packed_scales);

/*
 * moe_dispatch_layout — count, prefix-sum, stably rank and permute the
 * routed rows (steps: count per expert, prefix sum, permute) [H100-EP
 * 基于 DeepEP 的专家并行: tokens are routed to the experts that own them;
 * normal mode feeds prefill (contiguous layout), low-latency mode feeds
 * decode inside a graph (masked layout)].
 *
 *   topk_idx  [T, K] int32   local expert id per (token, pick), -1 = none
 *   x         [T, H] e4m3    source activations
 *   x_scale   [T, H/128] f32 their 1x128 block scales (row-major)
 *   layout    MOE_LAYOUT_CONTIGUOUS or MOE_LAYOUT_MASKED
 *   align_m   contiguous: every expert segment is padded to a multiple of
 *             align_m rows (>= 1); ignored for masked
 *   rows      contiguous: rows of the permuted buffer (M_cap);
 *             masked: capacity C rows per expert (buffer has E*C rows)
 * Outputs (rows_total = rows for contiguous, E*C for masked):
 *   counts    [E]      rows routed to each expert (before drops)
 *   offsets   [E+1]    segment starts: contiguous = prefix sum of counts
 *                      rounded up to align_m; masked = e*C
 *   slot_of   [T, K]   permuted row of each (t, k); -1 = none / dropped
 *   row_src   [rows_total]  source token of each row, -1 if no entry
 *   row_expert[rows_total]  expert of each row, -1 if no entry
 *   a         [rows_total, H] e4m3   a[slot] = x[row_src[slot]]; may be
 *             NULL: the rows are then not copied (the *_gather calls read
 *             them from x through row_src) and x may be NULL too; indices
 *             and a_scale are written as usual
 *   a_scale   [H/128, rows_total] f32 (K-block-major) matching scales
 *   workspace moe_layout_workspace_bytes(T, K, E) bytes of device memory
 * Rows of one expert are ordered by flat index t*K + k.  Rows that do not
 * fit (contiguous: slot >= rows; masked: rank >= C) are dropped and set
 * MOE_ERR_OVERFLOW; ids outside [-1, E) are skipped and set
 * MOE_ERR_BAD_EXPERT.  Rows of `a` / `a_scale` holding no entry are left
 * untouched.
 */
moe_status_t moe_dispatch_layout(const int32_t* topk_idx, const uint8_t* x,
                                 const float* x_scale, int T, int K, int E,
                                 int H, int layout, int align_m, int rows,
                                 int32_t* counts, int32_t* offsets,
                                 int32_t* slot_of, int32_t* row_src,
                                 int32_t* row_expert, uint8_t* a,
                                 float* a_scale, void* workspace,
                                 size_t workspace_bytes, int32_t* status_dev,
                                 void* stream);

/*
 * moe_dispatch_layout_noalloc — moe_dispatch_layout without a workspace
 * argument, for callers that cannot allocate device memory (code under
 * hipGraph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, outputs, status bits and results as moe_dispatch_layout
 * (bit for bit), minus workspace / workspace_bytes.
 *
 * The per-chunk histograms go to a fixed 1 MiB array in device memory
 * owned by the library: each GPU the library runs on holds one such array
 * until the process ends.  The call allocates nothing.  Limit:
 * moe_layout_workspace_bytes(T, K, E) <= 1 MiB (about 4M routed entries at
 * 32 experts); larger problems return MOE_SCRATCH_LIMIT and launch nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (two streams, or two host threads) race and give undefined results;
 * serialise them.  The first call on each device resolves the array's
 * device address (hipGetSymbolAddress, with that device current): make it
 * outside stream capture; later calls are capturable.
 */
moe_status_t moe_dispatch_layout_noalloc(const int32_t* topk_idx, const uint8_t* x,
                                         const float* x_scale, int T, int K, int E,
                                         int H, int layout, int align_m, int rows,
                                         int32_t* counts, int32_t* offsets,
                                         int32_t* slot_of, int32_t* row_src,
                                         int32_t* row_expert, uint8_t* a,
                                         float* a_scale, int32_t* status_dev,
                                         void* stream);

/*
 * moe_grouped_gemm_fp8 — block-scaled FP8 grouped GEMM over the expert
 * segments [H100-EP DeepGEMM 集成: FP8 grouped GEMMs for MoE; GB200 方法实现
 * 细节: FP8 GEMM whose API takes quantised input scales].  For every valid
 * row m of expert e and every n in [0, N):
 *
 *   c[m, n] = bf16_rne( sum_kb  a_scale[kb, m] * w_scale[e, n/128, kb]
 *                               * sum_{k in block kb} a[m, k] * w[e, n, k] )
 *
 * with fp32 accumulation (the 128-wide inner sums are exact products of
 * E4M3 values summed in fp32 by the matrix cores; the scales are applied in
 * fp32 once per 128-column block).  Used twice per layer: gate/up
 * (N = 2I, K = H; rows [0, I) of w are the gate, [I, 2I) the up projection)
 * and down (N = H, K = I).
 *
 *   a        [rows_total, K] e4m3      a_scale [K/128, rows_total] f32
 *   w        [E, N, K] e4m3            w_scale [E, N/128, K/128] f32
 *   offsets  [E+1], counts [E] int32 on the device (from moe_dispatch_layout)
 *   c        [rows_total, N] bf16; only valid rows are written
 * Segments reaching outside the buffer are clipped to it (rows the layout
 * call dropped are reported there, with MOE_ERR_OVERFLOW).  A table that
 * does not describe segments (a negative start or count, or starts that
 * decrease) sets MOE_ERR_BAD_INDEX in *status_dev (NULL: not reported); the
 * rows computed are still clipped to the buffer, and some may be missing.
 * MOE_UNSUPPORTED_SHAPE when the row-scale array (K/128 scales per row, or
 * ceil(K/512) packed words) reaches 0x7ffff000 bytes: the kernels address it
 * with 32-bit offsets.
 */
moe_status_t moe_grouped_gemm_fp8(const uint8_t* a, const float* a_scale,
                                  const uint8_t* w, const float* w_scale,
                                  const int32_t* offsets,
                                  const int32_t* counts, int E,
                                  int rows_total, int N, int K, uint16_t* c,
                                  int32_t* status_dev, void* stream);

/*
 * moe_gemm_fp8 -- dense block-scaled FP8 product for the linears outside
 * the MoE block [H100-EP DeepGEMM 集成: besides the grouped MoE GEMMs the
 * library offers a general GEMM kernel for non-MoE operations].  For every
 * m in [0, M), n in [0, N):
 *
 *   c[m, n] = bf16_rne( sum_kb  a_scale[kb, m] * w_scale[n/128, kb]
 *                               * sum_{k in block kb} a[m, k] * w[n, k] )
 *
 * with the same arithmetic as moe_grouped_gemm_fp8 (it is that kernel with
 * one weight matrix and every row valid).
 *
 *   a        [M, K] e4m3               a_scale [K/128, M] f32 (K-block-major)
 *   w        [N, K] e4m3               w_scale [N/128, K/128] f32
 *   c        [M, N] bf16
 * N and K must be multiples of 128; M >= 0 is arbitrary (M = 0 launches
 * nothing); (K/128) * M * 4 bytes of row scales must stay below 0x7ffff000
 * (MOE_UNSUPPORTED_SHAPE otherwise).  No device status word: the call has no
 * data-dependent errors.
 */
moe_status_t moe_gemm_fp8(const uint8_t* a, const float* a_scale,
                          const uint8_t* w, const float* w_scale, int M, int N,
                          int K, uint16_t* c, void* stream);

/*
 * moe_act_requant — SiLU(gate) * up, re-quantised to E4M3 with fresh 1x128
 * scales (reading: SiLU and the gate/up order are not on the pages).  For
 * every valid row m and j in [0, I):
 *   v = silu(h[m, j]) * h[m, I + j],  silu(g) = g / (1 + exp(-g))
 *       (fp32; exp and the reciprocal from the hardware, ~1 ulp each)
 *   per block jb of 128 columns: s = amax|v| / 448 (1 if amax == 0)
 *   q[m, j] = e4m3_rne(clamp(v / s, -448, 448)); q_scale[jb, m] = s
 *       (v / s correctly rounded in fp32, as the quantiser's decision)
 *
 *   h        [rows_total, 2I] bf16
 *   q        [rows_total, I] e4m3     q_scale [I/128, rows_total] f32
 * I must be a multiple of 128 (MOE_UNSUPPORTED_SHAPE otherwise).  Valid
 * rows come from offsets / counts as for moe_grouped_gemm_fp8, and a table
 * that does not describe segments sets MOE_ERR_BAD_INDEX the same way.
 */
moe_status_t moe_act_requant(const uint16_t* h, const int32_t* offsets,
                             const int32_t* counts, int E, int rows_total,
                             int I, uint8_t* q, float* q_scale,
                             int32_t* status_dev, void* stream);

/*
 * moe_gate_up_act_fp8 — the gate/up grouped GEMM and moe_act_requant fused
 * into one kernel (the GEMM of "Deploying DeepSeek with PD Disaggregation
 * and Large-Scale Expert Parallelism on 96 H100 GPUs", section 大规模专家并行
 * › DeepGEMM 集成, followed by the activation read above).  For every valid
 * row m the result is exactly that of
 *   moe_grouped_gemm_fp8(a, a_scale, w13, w13_scale, ..., N = 2I, K = H, h)
 *   moe_act_requant(h, ..., I, q2, q2_scale)
 * -- the same codes and scales bit for bit: each h value is rounded to
 * bf16 as the GEMM stores it before the activation reads it -- but h is
 * never written to memory.
 *
 *   a        [rows_total, H] e4m3      a_scale [H/128, rows_total] f32
 *   w13      [E, 2I, H] e4m3 (rows [0, I) gate, [I, 2I) up)
 *   w13_scale [E, 2I/128, H/128] f32
 *   q2       [rows_total, I] e4m3      q2_scale [I/128, rows_total] f32
 * I and H must be multiples of 128 and one expert's W13 (2 I H bytes)
 * below 2 GB, and the row scales within moe_grouped_gemm_fp8's limit
 * (MOE_UNSUPPORTED_SHAPE otherwise); a, w13 and q2 16-byte aligned.  Rows
 * outside every expert's valid range are not written.  MOE_ERR_BAD_INDEX as
 * for moe_grouped_gemm_fp8.
 */
moe_status_t moe_gate_up_act_fp8(const uint8_t* a, const float* a_scale,
                                 const uint8_t* w13, const float* w13_scale,
                                 const int32_t* offsets, const int32_t* counts,
                                 int E, int rows_total, int I, int H, uint8_t* q2,
                                 float* q2_scale, int32_t* status_dev,
                                 void* stream);

/*
 * moe_combine — un-permute and sum each token's rows weighted by its top-k
 * weights [H100-EP 基于 DeepEP 的专家并行: combine returns expert outputs to
 * their source tokens]:
 *   out[t, :] = bf16_rne( sum_{k = 0..K-1, slot_of[t,k] >= 0}
 *                          topk_w[t, k] * y[slot_of[t, k], :] )
 * accumulated in fp32 in ascending k; a token with no valid row gets 0.
 * Deterministic (gather, no atomics).
 *
 *   y        [rows_total, H] bf16
 *   slot_of  [T, K] int32; topk_w [T, K] f32
 *   out      [T, H] bf16
 * Slots >= rows_total are skipped and set MOE_ERR_BAD_INDEX.
 */
moe_status_t moe_combine(const uint16_t* y, int rows_total,
                         const int32_t* slot_of, const float* topk_w, int T,
                         int K, int H, uint16_t* out, int32_t* status_dev,
                         void* stream);

/*
 * moe_quantize_fp8 — source-side block quantisation to E4M3 [GB200 方法实现
 * 细节: the FP8 GEMM API quantises the input scales].  Produces the inputs
 * the layer consumes: activations with one scale per 1x128 block
 * (block_rows = 1, scale [rows, cols/128] row-major) and weights with one
 * scale per 128x128 block (block_rows = 128, scale [rows/128, cols/128];
 * stacked expert weights [E, N, K] are rows = E*N).  Per block:
 *   s = amax|x| / 448 (1 if amax == 0);  q = e4m3_rne(clamp(x / s, +-448)).
 *
 *   x        [rows, cols], bf16 (x_is_f32 = 0) or f32 (x_is_f32 = 1)
 *   q        [rows, cols] e4m3, scale as above
 */
moe_status_t moe_quantize_fp8(const void* x, int x_is_f32, int rows, int cols,
                              int block_rows, uint8_t* q, float* scale,
                              void* stream);

/*
 * Packed power-of-two scales (E8M0) [GB200 方法实现细节: the FP8 GEMM API
 * quantises and packs the input scales].  Reading: a block's scale is the
 * smallest power of two not below fp32(amax / 448) (1 for an all-zero
 * block, 2^-127 when the quotient underflows), so q = e4m3_rne(v / s) is
 * exact scaling; the scale is stored as its biased exponent byte e + 127,
 * four consecutive 128-wide blocks along K per little-endian 32-bit word
 * (byte j of word w holds block 4w + j; bytes past a row's last block are
 * 127).  The matrix cores apply these scales themselves
 * (v_mfma_scale_f32_16x16x128_f8f6f4), with no fp32 promotion step.  Each
 * call below is its fp32-scale counterpart above with these scale arrays:
 *   moe_quantize_fp8_e8m0     scale: block_rows 1 -> [rows, ceil(cols/512)]
 *                             words (row-major per row, as dispatched with
 *                             the token); block_rows 128 -> [rows/128,
 *                             ceil(cols/512)]
 *   moe_dispatch_layout_e8m0  x_scale [T, ceil(H/512)] words ->
 *                             a_scale [ceil(H/512), rows_total] words
 *                             (K-word-major)
 *   moe_grouped_gemm_fp8_e8m0 a_scale [ceil(K/512), rows_total] words,
 *                             w_scale [E, N/128, ceil(K/512)] words;
 *                             c = bf16_rne(sum_kb 2^(ea + ew) * block product)
 *   moe_act_requant_e8m0      q_scale [ceil(I/512), rows_total] words
 *   moe_gate_up_act_fp8_e8m0  a_scale, w13_scale as the grouped GEMM's,
 *                             q2_scale [ceil(I/512), rows_total] words;
 *                             equal to moe_grouped_gemm_fp8_e8m0 followed by
 *                             moe_act_requant_e8m0
 * Argument checks, status bits and layouts otherwise as above.
 */
moe_status_t moe_quantize_fp8_e8m0(const void* x, int x_is_f32, int rows,
                                   int cols, int block_rows, uint8_t* q,
                                   uint32_t* scale, void* stream);
moe_status_t moe_dispatch_layout_e8m0(
    const int32_t* topk_idx, const uint8_t* x, const uint32_t* x_scale, int T,
    int K, int E, int H, int layout, int align_m, int rows, int32_t* counts,
    int32_t* offsets, int32_t* slot_of, int32_t* row_src, int32_t* row_expert,
    uint8_t* a, uint32_t* a_scale, void* workspace, size_t workspace_bytes,
    int32_t* status_dev, void* stream);
moe_status_t moe_grouped_gemm_fp8_e8m0(const uint8_t* a, const uint32_t* a_scale,
                                       const uint8_t* w, const uint32_t* w_scale,
                                       const int32_t* offsets,
                                       const int32_t* counts, int E,
                                       int rows_total, int N, int K,
                                       uint16_t* c, int32_t* status_dev,
                                       void* stream);
moe_status_t moe_act_requant_e8m0(const uint16_t* h, const int32_t* offsets,
                                  const int32_t* counts, int E, int rows_total,
                                  int I, uint8_t* q, uint32_t* q_scale,
                                  int32_t* status_dev, void* stream);
moe_status_t moe_gate_up_act_fp8_e8m0(const uint8_t* a, const uint32_t* a_scale,
                                      const uint8_t* w13, const uint32_t* w13_scale,
                                      const int32_t* offsets, const int32_t* counts,
                                      int E, int rows_total, int I, int H,
                                      uint8_t* q2, uint32_t* q2_scale,
                                      int32_t* status_dev, void* stream);

/*
 * The gate/up calls with the permutation of the rows done in their tile
 * loads [H100-EP 基于 DeepEP 的专家并行 and DeepGEMM 集成: the routed rows
 * grouped per expert feed the grouped GEMM]: instead of the permuted buffer
 * `a`, they take the source rows x [T, K] e4m3 (K = H, the contraction
 * width) and row_src [rows_total] (as moe_dispatch_layout writes it) and
 * read buffer row r from x[row_src[r]]; a row with row_src < 0 or >= T is
 * read as zero.  The row scales are the permuted a_scale as before (so the
 * dispatch can run with a == NULL).  Results equal the plain calls on the
 * permuted buffer bit for bit.  Extra checks: T < 0, row_src NULL, or x NULL
 * with T > 0 -> MOE_INVALID_ARG; T * K > 0x7ffff000 bytes (one buffer
 * descriptor) -> MOE_UNSUPPORTED_SHAPE.  Otherwise as the plain calls; the
 * fused packed-scale form keeps 256-row tiles where the others use 320.
 */
moe_status_t moe_grouped_gemm_fp8_gather(const uint8_t* x, int T, const int32_t* row_src,
                                         const float* a_scale, const uint8_t* w,
                                         const float* w_scale, const int32_t* offsets,
                                         const int32_t* counts, int E, int rows_total,
                                         int N, int K, uint16_t* c, int32_t* status_dev,
                                         void* stream);
moe_status_t moe_grouped_gemm_fp8_gather_e8m0(const uint8_t* x, int T, const int32_t* row_src,
                                              const uint32_t* a_scale, const uint8_t* w,
                                              const uint32_t* w_scale, const int32_t* offsets,
                                              const int32_t* counts, int E, int rows_total,
                                              int N, int K, uint16_t* c, int32_t* status_dev,
                                              void* stream);
moe_status_t moe_gate_up_act_fp8_gather(const uint8_t* x, int T, const int32_t* row_src,
                                        const float* a_scale, const uint8_t* w13,
                                        const float* w13_scale, const int32_t* offsets,
                                        const int32_t* counts, int E, int rows_total, int I,
                                        int H, uint8_t* q2, float* q2_scale,
                                        int32_t* status_dev, void* stream);
moe_status_t moe_gate_up_act_fp8_gather_e8m0(const uint8_t* x, int T, const int32_t* row_src,
                                             const uint32_t* a_scale, const uint8_t* w13,
                                             const uint32_t* w13_scale, const int32_t* offsets,
                                             const int32_t* counts, int E, int rows_total,
                                             int I, int H, uint8_t* q2, uint32_t* q2_scale,
                                             int32_t* status_dev, void* stream);

/*
 * Measurement helpers (not steps of the layer).  They time the two
 * resources the layer's kernels are bound by, so that a kernel can be
 * reported against what the GPU sustains as well as against its published
 * peaks (HBM 8 TB/s, dense FP8 5.0 PFLOP/s).
 *
 * moe_ceiling_copy     dst[i] = src[i] for `bytes` bytes (a multiple of 16;
 *                      both pointers 16-byte aligned, else INVALID_ARG): one
 *                      16-byte load and store per lane, grid-stride.  Moves
 *                      2 * bytes through HBM.
 * moe_ceiling_mfma_fp8 `workgroups` workgroups of 4 waves, each wave running
 *                      `iters` rounds of 8 independent E4M3 16x16x128 MFMAs
 *                      on register operands (the instruction of the GEMMs);
 *                      *flops (host pointer, may be NULL) receives the
 *                      launch's flop count.  `sink` is a device array of
 *                      `workgroups` floats that is (practically) never
 *                      written; it keeps the chain from being optimised out.
 */
moe_status_t moe_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream);
moe_status_t moe_ceiling_mfma_fp8(int workgroups, int iters, float* sink, double* flops,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H_ */
