/*
 * fp8gg.h -- C ABI of the FP8 (e4m3fn) rowwise-scaled grouped GEMM for MI355X (gfx950).
 *
 * Per expert group g the library computes
 *
 *     Y_g[m, n] = bf16_rne( (sum_k XQ_g[m, k] * WQ[g, n, k]) * x_scale[m] * w_scale[g, n] )
 *
 * with fp8 e4m3fn operands, fp32 accumulation of the unscaled products, the two
 * scales applied once after the reduction, and round-to-nearest-even to bf16.
 * Source of the operation: MSLK pull request 471, "Back the FP8 rowwise grouped
 * GEMM ops with FlyDSL on ROCm" -- Summary (op table: the stacked op with [G]
 * int64 row counts, the dynamic op with [G, M, K] slabs and a runtime valid-row
 * count, and the preshuffle siblings) and Design notes (rowwise scales factor out
 * of the K loop and are applied once in the epilogue).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers.  All tensors are dense and row-major
 *     (contiguous); there are no stride arguments.  The caller owns every buffer.
 *   - fp8 operands are raw e4m3fn bytes (uint8_t); Y is raw bf16 bits (uint16_t).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is only
 *     enqueued: no entry point copies between host and device or synchronises.
 *     Every call may be captured into a HIP graph.
 *   - No workspace: the library allocates no device memory.  Stacked, offsets and
 *     batched calls with at least 256 rows per group (on average) run on a
 *     persistent grid, one workgroup per compute unit; when the output tiles do
 *     not fill a whole number of rounds of that grid, the tiles of the last round
 *     may be computed as four quarter tiles each.  Every output element is still computed by one
 *     workgroup in one fixed K order, so results are deterministic and equal,
 *     bit for bit, to those of the one-tile-per-workgroup schedule.
 *   - Device-side metadata (M_sizes, zero_start_index_M) is never read by the host.
 *     The kernels clamp it (negative counts -> 0, cumulative row ends -> total_M,
 *     valid rows -> [0, expected_m]), so inconsistent metadata can never cause an
 *     out-of-bounds access; the values computed for it are then unspecified.
 *   - Size limits: every dimension (and G * expected_m) below 2^31 - 256, every
 *     tensor below 2^48 bytes (FP8GG_ERR_UNSUPPORTED_SHAPE otherwise).
 *   - Shape rules: K % 16 == 0 and N % 8 == 0 (a 16-byte load granule along K and
 *     an 8-column store granule along N; MSLK #471 commits on the K-tail and N-tail
 *     variants).  K need not be a multiple of the K tile, N not of the N tile.
 *   - Alignment: XQ, WQ, w_scale and Y must be 16-byte aligned; x_scale 4-byte.
 *   - Y must not overlap any input.
 *   - K == 0: the whole output is zero-filled (a contraction over nothing sums to
 *     zero; MSLK #471 commit on zero-length reductions).  An output with no
 *     elements launches nothing.
 *   - Errors: every check runs on the host before anything is enqueued.  A failed
 *     check returns a non-zero status, enqueues nothing and leaves a message for
 *     f8f8bf16_last_error().  A launch failure returns FP8GG_ERR_HIP.
 *   - The library is re-entrant; calls on different streams may run concurrently.
 */
#ifndef FP8GG_H_
#define FP8GG_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8GG_OK = 0,
  FP8GG_ERR_INVALID_ARGUMENT = 1,  /* null pointer, negative size, misalignment, aliasing */
  FP8GG_ERR_UNSUPPORTED_SHAPE = 2, /* K % 16 != 0, N % 8 != 0, preshuffle granules, limits */
  FP8GG_ERR_HIP = 3                /* the HIP runtime reported an error at launch */
} fp8gg_status;

/*
 * Stacked layout (MSLK #471: Summary op table, stacked row; commit adding the
 * layout enum, layout "sizes").  Groups are concatenated along M: group g owns
 * the next M_sizes[g] rows of XQ / x_scale / Y, starting after groups 0..g-1.
 *
 *   XQ        [total_M, K]   fp8 e4m3fn activations
 *   WQ        [G, N, K]      fp8 e4m3fn weights (one [N, K] matrix per group)
 *   x_scale   [total_M]      fp32, one scale per row of XQ
 *   w_scale   [G, N]         fp32, one scale per output column of each group
 *   M_sizes   [G]            int64 row counts, on the device
 *   Y         [total_M, N]   bf16 output
 *
 * Rows at or beyond sum(M_sizes) (clamped to total_M) are not written.
 */
fp8gg_status f8f8bf16_rowwise_grouped_stacked(
    const uint8_t* XQ, const uint8_t* WQ, const float* x_scale, const float* w_scale,
    const int64_t* M_sizes, uint16_t* Y,
    int64_t G, int64_t total_M, int64_t N, int64_t K, void* stream);

/*
 * Padded ("dynamic") layout (MSLK #471: Summary op table, dynamic row; commits
 * adding the padded layout and its test).  Each group owns a slab of expected_m
 * rows; only the first zero_start_index_M[g] rows of slab g are valid.
 *
 *   XQ                  [G, expected_m, K]  fp8 e4m3fn
 *   WQ                  [G, N, K]           fp8 e4m3fn
 *   x_scale             [G, expected_m]     fp32
 *   w_scale             [G, N]              fp32
 *   zero_start_index_M  [G]                 int64 valid-row counts, on the device
 *   Y                   [G, expected_m, N]  bf16
 *   zeroing_output_tensor  non-zero: padding rows of Y are written as +0.0;
 *                          zero: padding rows are left untouched.
 *
 * Padding rows of XQ and x_scale may hold anything (NaN included): they never
 * reach a written output.
 */
fp8gg_status f8f8bf16_rowwise_grouped_dynamic(
    const uint8_t* XQ, const uint8_t* WQ, const float* x_scale, const float* w_scale,
    const int64_t* zero_start_index_M, uint16_t* Y,
    int64_t G, int64_t expected_m, int64_t N, int64_t K,
    int zeroing_output_tensor, void* stream);

/*
 * Offsets layout (MSLK #471: commit adding the offsets layout; commit mapping the
 * grouped mm op's 2D-3D operand ranks onto it).  Groups are concatenated along M
 * as in the stacked layout, but their boundaries come as an inclusive prefix
 * sum: group g owns rows [offsets[g-1], offsets[g]) of XQ / x_scale / Y, with
 * offsets[-1] = 0.
 *
 *   XQ, WQ, x_scale, w_scale, Y   as in the stacked layout
 *   offsets   [G]   int32 inclusive prefix sums of the group row counts, on the device
 *
 * Group g ends at min(max(offsets[g], end of group g-1), total_M): an offset below
 * its predecessor gives an empty group.  Rows past the last end are not written.
 */
fp8gg_status f8f8bf16_rowwise_grouped_offsets(
    const uint8_t* XQ, const uint8_t* WQ, const float* x_scale, const float* w_scale,
    const int32_t* offsets, uint16_t* Y,
    int64_t G, int64_t total_M, int64_t N, int64_t K, void* stream);

/*
 * Batched layout (MSLK #471: commit adding the batched layout; the grouped mm
 * op's 3D-3D ranks).  Every group owns a full slab of M rows, all of them valid;
 * there is no row metadata.
 *
 *   XQ        [G, M, K]   fp8 e4m3fn
 *   WQ        [G, N, K]   fp8 e4m3fn
 *   x_scale   [G, M]      fp32
 *   w_scale   [G, N]      fp32
 *   Y         [G, M, N]   bf16, every row written
 */
fp8gg_status f8f8bf16_rowwise_grouped_batched(
    const uint8_t* XQ, const uint8_t* WQ, const float* x_scale, const float* w_scale,
    uint16_t* Y, int64_t G, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Pre-shuffled weights (MSLK #471: commit registering the stacked op and its
 * preshuffle sibling; Design notes on preshuffled B: offered only where each
 * group owns a whole [N, K]).  WQs is WQ rearranged once by f8f8bf16_shuffle_b
 * into the order in which the matrix cores consume it; it has the same byte
 * count as WQ.  Additional shape rule: N % FP8GG_SHUFFLE_N == 0 and
 * K % FP8GG_SHUFFLE_K == 0 (the shuffle interleaves N and K, so a partial block
 * cannot be masked).  All other arguments are as in the plain entry points.
 */
#define FP8GG_SHUFFLE_N 32
#define FP8GG_SHUFFLE_K 64

fp8gg_status f8f8bf16_rowwise_grouped_stacked_preshuffle(
    const uint8_t* XQ, const uint8_t* WQs, const float* x_scale, const float* w_scale,
    const int64_t* M_sizes, uint16_t* Y,
    int64_t G, int64_t total_M, int64_t N, int64_t K, void* stream);

fp8gg_status f8f8bf16_rowwise_grouped_dynamic_preshuffle(
    const uint8_t* XQ, const uint8_t* WQs, const float* x_scale, const float* w_scale,
    const int64_t* zero_start_index_M, uint16_t* Y,
    int64_t G, int64_t expected_m, int64_t N, int64_t K,
    int zeroing_output_tensor, void* stream);

fp8gg_status f8f8bf16_rowwise_grouped_offsets_preshuffle(
    const uint8_t* XQ, const uint8_t* WQs, const float* x_scale, const float* w_scale,
    const int32_t* offsets, uint16_t* Y,
    int64_t G, int64_t total_M, int64_t N, int64_t K, void* stream);

fp8gg_status f8f8bf16_rowwise_grouped_batched_preshuffle(
    const uint8_t* XQ, const uint8_t* WQs, const float* x_scale, const float* w_scale,
    uint16_t* Y, int64_t G, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * N-offsets layout (the 3D-2D ranks of the grouped mm: MSLK #471, commit adding
 * that form, and the commit that predicates stores on their last column): the
 * weights are one matrix whose rows (the output columns) the groups partition;
 * group g multiplies its own slab of XQ against its rows of WQ, and the results
 * sit side by side in Y.
 *
 *   XQ        [G, M, K]     fp8 e4m3fn, one slab of M rows per group
 *   WQ        [N, K]        fp8 e4m3fn, N = total_N over all groups
 *   x_scale   [G, M]        fp32
 *   w_scale   [N]           fp32, one per row of WQ
 *   n_offsets [G]           int32 inclusive prefix: group g owns W rows / output
 *                           columns [n_offsets[g-1], n_offsets[g]) (n_offsets[-1] = 0)
 *   Y         [M, N]        bf16:  Y[m, n] = (sum_k XQ[g, m, k] WQ[n, k]) x_scale[g, m] w_scale[n]
 *
 * The offsets are clamped in-kernel like those of the offsets layout (an end below
 * its predecessor gives an empty group, ends are cut at N); columns past the last
 * end are left untouched.  A group's columns may start and end anywhere: every
 * column of every group is written (vectors that straddle a group boundary are
 * stored column by column).  Plain WQ only: pre-shuffled weights interleave N
 * across group boundaries (MSLK #471, commit adding the mm preshuffle entry
 * point), so this layout has no _preshuffle sibling.  Shape rules as above
 * (K % 16 == 0, N % 8 == 0).
 */
fp8gg_status f8f8bf16_rowwise_grouped_n_offsets(
    const uint8_t* XQ, const uint8_t* WQ, const float* x_scale, const float* w_scale,
    const int32_t* n_offsets, uint16_t* Y,
    int64_t G, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * K-offsets layout (the 2D-2D ranks of the grouped mm: MSLK #471, commit adding
 * that form, and the commit keying the K-tail predicate on the group's own slice):
 * both operands are one matrix whose K columns the groups slice; every group
 * contracts over its own slice and produces a whole [M, N] output.
 *
 *   XQ        [M, K]        fp8 e4m3fn, K = total_K over all groups
 *   WQ        [N, K]        fp8 e4m3fn
 *   x_scale   [G, M]        fp32, one per row of each group's slice of XQ
 *   w_scale   [G, N]        fp32, one per row of each group's slice of WQ
 *   k_offsets [G]           int32 inclusive prefix: group g contracts over
 *                           [k_offsets[g-1], k_offsets[g]) (k_offsets[-1] = 0)
 *   Y         [G, M, N]     bf16:  Y[g, m, n] = (sum_{k in slice g} XQ[m, k] WQ[n, k]) x_scale[g, m] w_scale[g, n]
 *
 * Every element of Y is written; an empty slice gives (0 * x_scale) * w_scale.
 * The offsets must be multiples of 16 (the load granule); in-kernel they are
 * clamped like the offsets layout's (ends cut at K, an end below its predecessor
 * gives an empty slice) and rounded down to a multiple of 16, so other values
 * never cause an out-of-bounds access but give unspecified results.  Plain WQ
 * only (no _preshuffle sibling).  Shape rules as above.
 */
fp8gg_status f8f8bf16_rowwise_grouped_k_offsets(
    const uint8_t* XQ, const uint8_t* WQ, const float* x_scale, const float* w_scale,
    const int32_t* k_offsets, uint16_t* Y,
    int64_t G, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Block (groupwise) scaling, stacked layout (MSLK #471, first commit of the list:
 * block scaling carries one scale per (scale_block_k x scale_block_n) block of B
 * and scales each block's partial sum inside the K loop; the A-side granularity,
 * one scale per row and K block, is this library's reading).  Blocks are 128 x 128:
 *
 *   XQ        [total_M, K]             fp8 e4m3fn
 *   WQ        [G, N, K]                fp8 e4m3fn
 *   x_scale   [total_M, K / 128]       fp32, 4-byte aligned
 *   w_scale   [G, N / 128, K / 128]    fp32, 4-byte aligned
 *   M_sizes   [G]                      int64 row counts (as the stacked op)
 *   Y         [total_M, N]             bf16:
 *       Y[m, n] = sum_kb (sum_{k in block kb} XQ[m, k] WQ[g, n, k]) x_scale[m, kb] w_scale[g, n / 128, kb]
 *
 * Shape rule: K % 128 == 0 and N % 128 == 0 (whole scale blocks; the pages require
 * the block bound under block scaling), else FP8GG_ERR_UNSUPPORTED_SHAPE.  Each
 * block's products accumulate in fp32 and are scaled in fp32 before they join the
 * running sum.  Row classes, clamping and K == 0 as for the stacked op.
 */
fp8gg_status f8f8bf16_groupwise_grouped_stacked(
    const uint8_t* XQ, const uint8_t* WQ, const float* x_scale, const float* w_scale,
    const int64_t* M_sizes, uint16_t* Y,
    int64_t G, int64_t total_M, int64_t N, int64_t K, void* stream);

/* As f8f8bf16_groupwise_grouped_stacked, with WQs produced by f8f8bf16_shuffle_b
 * (one kernel serves both B layouts under either scaling scheme: MSLK #471, commit
 * moving the host-side work into the shared grouped dispatch).  The 128-wide
 * scale blocks are whole pre-shuffle blocks, so the shape rule is unchanged. */
fp8gg_status f8f8bf16_groupwise_grouped_stacked_preshuffle(
    const uint8_t* XQ, const uint8_t* WQs, const float* x_scale, const float* w_scale,
    const int64_t* M_sizes, uint16_t* Y,
    int64_t G, int64_t total_M, int64_t N, int64_t K, void* stream);

/* Block scaling in the offsets layout (int32 inclusive prefix of the group row
 * counts, clamped as for f8f8bf16_rowwise_grouped_offsets) and in the batched
 * layout (XQ [G, M, K], x_scale [G, M, K / 128], Y [G, M, N], every row valid, no
 * metadata).  Scales, block sizes and shape rule as for the stacked op. */
fp8gg_status f8f8bf16_groupwise_grouped_offsets(
    const uint8_t* XQ, const uint8_t* WQ, const float* x_scale, const float* w_scale,
    const int32_t* offsets, uint16_t* Y,
    int64_t G, int64_t total_M, int64_t N, int64_t K, void* stream);

fp8gg_status f8f8bf16_groupwise_grouped_offsets_preshuffle(
    const uint8_t* XQ, const uint8_t* WQs, const float* x_scale, const float* w_scale,
    const int32_t* offsets, uint16_t* Y,
    int64_t G, int64_t total_M, int64_t N, int64_t K, void* stream);

fp8gg_status f8f8bf16_groupwise_grouped_batched(
    const uint8_t* XQ, const uint8_t* WQ, const float* x_scale, const float* w_scale,
    uint16_t* Y, int64_t G, int64_t M, int64_t N, int64_t K, void* stream);

fp8gg_status f8f8bf16_groupwise_grouped_batched_preshuffle(
    const uint8_t* XQ, const uint8_t* WQs, const float* x_scale, const float* w_scale,
    uint16_t* Y, int64_t G, int64_t M, int64_t N, int64_t K, void* stream);

/* Block scaling in the padded ("dynamic") layout: XQ [G, expected_m, K], x_scale
 * [G, expected_m, K / 128], w_scale [G, N / 128, K / 128], zero_start_index_M [G]
 * (int64, on device, clamped to [0, expected_m]), Y [G, expected_m, N].  Rows of
 * slab g at or past zero_start_index_M[g] are written as zero when
 * zeroing_output_tensor is non-zero, else left untouched; K == 0 zero-fills Y.
 * Same block sizes and shape rule as the stacked op; with WQs from
 * f8f8bf16_shuffle_b in the _preshuffle sibling. */
fp8gg_status f8f8bf16_groupwise_grouped_dynamic(
    const uint8_t* XQ, const uint8_t* WQ, const float* x_scale, const float* w_scale,
    const int64_t* zero_start_index_M, uint16_t* Y,
    int64_t G, int64_t expected_m, int64_t N, int64_t K, int zeroing_output_tensor, void* stream);

fp8gg_status f8f8bf16_groupwise_grouped_dynamic_preshuffle(
    const uint8_t* XQ, const uint8_t* WQs, const float* x_scale, const float* w_scale,
    const int64_t* zero_start_index_M, uint16_t* Y,
    int64_t G, int64_t expected_m, int64_t N, int64_t K, int zeroing_output_tensor, void* stream);

/*
 * Rearranges WQ [G, N, K] into the pre-shuffled order WQs (same size, must not
 * overlap WQ).  Byte layout: for group g, N-block nb (FP8GG_SHUFFLE_N rows) and
 * K-block kb (FP8GG_SHUFFLE_K bytes), the 2048-byte block at
 *     ((g * N/32 + nb) * K/64 + kb) * 2048
 * holds, for lane l in [0, 64) and half h in {0, 1}, at offset h*1024 + l*16, the
 * 16 bytes WQ[g, nb*32 + perm32(l % 32), kb*64 + (l / 32)*32 + h*16 .. +16), with
 * perm32(r) = 16*((r >> 2) & 1) + 4*(r >> 3) + (r & 3).  Same shape rules as the
 * preshuffled GEMMs.
 */
fp8gg_status f8f8bf16_shuffle_b(const uint8_t* WQ, uint8_t* WQs,
                                int64_t G, int64_t N, int64_t K, void* stream);

/*
 * Rowwise fp8 quantisation of bf16 activations: produces the XQ and x_scale
 * operands of the GEMMs above (one scale per row, constant along K: MSLK #471,
 * Design notes, scaling-scheme paragraph; the amax choice of the scale is this
 * library's).  Per row r of X:
 *     x_scale[r] = amax_k |X[r, k]| / 448   (fp32, IEEE division; 1 if amax == 0)
 *     XQ[r, k]   = e4m3fn_rne(clamp(X[r, k] / x_scale[r], -448, 448))   (fp32 quotient)
 *
 *   X         [rows, K]   bf16 (raw bits), 16-byte aligned
 *   XQ        [rows, K]   fp8 e4m3fn output, 8-byte aligned
 *   x_scale   [rows]      fp32 output
 *
 * Shape rule: K % 8 == 0.  Inputs are expected finite: a NaN is ignored by amax
 * and gives an unspecified code.  The three buffers must not overlap.
 */
fp8gg_status f8f8bf16_quantize_rowwise(const uint16_t* X, uint8_t* XQ, float* x_scale,
                                       int64_t rows, int64_t K, void* stream);

/* Message describing the last failure on the calling thread ("" if none). */
const char* f8f8bf16_last_error(void);

/*
 * Launch plan, computed on the host only (no HIP call).  Exposed so that tests
 * and offline tuning can see what a call would launch.
 */
typedef struct {
  int32_t config_id;  /* index of the kernel configuration; -1 = nothing to compute */
  int32_t BM, BN, BK; /* workgroup tile: rows of XQ, columns of Y, bytes of K      */
  int32_t threads;    /* threads per workgroup                                      */
  int32_t stages;     /* LDS pipeline depth                                         */
  int32_t k_tail;     /* 1 if K % BK != 0 (the last K tile is masked)               */
  int32_t n_tail;     /* 1 if N % BN != 0 (the last N tile is masked)               */
  int64_t m_tiles;    /* stacked: upper bound of M tiles; padded: tiles per slab    */
  int64_t n_tiles;
  int64_t grid;       /* workgroups of the data-parallel schedule (one per tile)     */
  int32_t zero_fill;  /* 1 if the call zero-fills Y instead (K == 0)                */
  int32_t lds_bytes;  /* LDS per workgroup                                          */
  int32_t persistent; /* 1: persistent grid (one workgroup per compute unit); the
                         grid above is then the tile count of the data-parallel
                         schedule                                                   */
} fp8gg_plan;

enum {
  FP8GG_LAYOUT_STACKED = 0,
  FP8GG_LAYOUT_PADDED = 1,
  FP8GG_LAYOUT_OFFSETS = 2,
  FP8GG_LAYOUT_BATCHED = 3,
  FP8GG_LAYOUT_N_OFFSETS = 4,
  FP8GG_LAYOUT_K_OFFSETS = 5
};

/* M is total_M for the stacked and offsets layouts, expected_m for the padded one
 * and the slab height for the batched, n_offsets and k_offsets ones; N is total_N
 * for n_offsets and K is total_K for k_offsets.
 * Performs the same shape checks as the GEMM entry points. */
fp8gg_status f8f8bf16_plan(int layout, int preshuffled, int64_t G, int64_t M,
                           int64_t N, int64_t K, fp8gg_plan* out);

/* Number of kernel configurations compiled into the library (for tuning). */
int32_t f8f8bf16_num_configs(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8GG_H_ */
