/*
 * mxg.h -- C ABI of libmxg.so: the ragged MoE expert path on one gfx950 GPU.
 *
 * Six operations, each one asynchronous launch sequence on the caller's HIP
 * stream:
 *   mx_grouped_quantize       BF16 activations -> FP8 e4m3 + per-row fp32 scale,
 *                             or MX (32-element blocks, E8M0 scale, e4m3 or e2m1)
 *   mx_grouped_quantize_gather  the same, reading each routed row from its
 *                             source row (token) through an index list
 *   mx_grouped_matmul         ragged grouped GEMM, FP8 rowwise or MX block-scaled,
 *                             fp32 accumulation, BF16 output
 *   mx_grouped_matmul_swiglu  MX grouped GEMM against interleaved gate/up weights,
 *                             fused with SwiGLU and an MXFP4 requant
 *   mx_silu_quantize          the unfused second half: SwiGLU + MXFP4 requant of a
 *                             BF16 gate/up tensor
 *   mx_grouped_quantize_nvfp4 BF16 activations -> NVFP4 (16-element blocks, E4M3
 *                             scale, e2m1 codes) under a per-expert tensor scale
 *   mx_grouped_matmul_nvfp4   ragged grouped GEMM of NVFP4 operands with a
 *                             per-expert epilogue scale, BF16 output
 *   mx_grouped_matmul_swiglu_nvfp4  NVFP4 gate/up grouped GEMM fused with SwiGLU
 *                             and an NVFP4 requant of the activation
 *   mx_silu_quantize_nvfp4    its unfused second half
 *   mx_grouped_quantize_padded, mx_grouped_matmul_padded,
 *   mx_grouped_matmul_swiglu_padded, mx_grouped_quantize_nvfp4_padded,
 *   mx_grouped_matmul_nvfp4_padded
 *                             MX / NVFP4 quantize, GEMM (and MX fused GEMM) with
 *                             the activation scales in a padded or expert-slot
 *                             layout
 *   mx_prepare_weights_fp8, mx_prepared_weights_bytes, mx_grouped_matmul_prepared
 *                             FP8 rowwise weights rearranged once into the
 *                             layout the GEMM's load ring copies as it is, and
 *                             the grouped GEMM that reads them
 *   mx_grouped_quantize_scatter  the same in token-major form: each token row
 *                             is read once and stored to its routed rows
 *   mx_moe_combine            after the down-projection: each token's row is the
 *                             router-weighted sum of its routed rows
 *   mxg_clock_probe           measurement aid: the engine clock over a window
 *   mxg_validation_message, mxg_routing_violation
 *                             the MXG_VALIDATE debug check of routing metadata
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *     allocates no memory and keeps no state between calls.  Tensors are dense
 *     and row-major with the last-named dimension innermost.  Code and BF16
 *     tensors must start on a 16-byte boundary; fp32 scale tensors on 4 bytes.
 *   - Calls only enqueue work on `stream` (0 = the null stream) and return; no
 *     host synchronisation and no device-to-host copy happens inside a call.
 *   - Groups.  row_offsets is uint32 [num_groups + 1]; group g owns the rows
 *     [row_offsets[g], row_offsets[g+1]) of the routed-row dimension, and
 *     expert_ids[g] (int32) names the expert whose weights those rows use
 *     (grouped_matmul_rowwise_dynamic_scaled_fp8, Args: a_offsets, expert_ids).
 *     Offsets are expected non-decreasing and <= total_rows.  Malformed device
 *     data never causes an out-of-bounds access: offsets are clamped to
 *     total_rows, a group whose start exceeds its end or whose expert id lies
 *     outside [0, num_experts) is skipped, and output rows that no taken group
 *     covers are left untouched.  Overlapping groups give unspecified values
 *     in the overlap.
 *   - FP4 (e2m1) tensors hold two elements per byte, element 2i in bits 0..3
 *     and element 2i+1 in bits 4..7.  E8M0 scales are one byte, 2^(code-127).
 *   - Element encodings: e4m3 is OCP OFP8 E4M3 (no infinities, max 448), e2m1
 *     is OCP MX E2M1 (max 6).  Encoding rounds to nearest, ties to even, and
 *     saturates to the largest finite code; the sign of a value that rounds to
 *     zero is kept.
 *   - Errors are returned before anything is enqueued (nothing is launched on
 *     an error).  MXG_ERROR_LAUNCH reports a failed kernel launch.  With
 *     total_rows == 0 or num_groups == 0 a call (after its enum and size
 *     checks) is a no-op that examines no pointer.
 *   - Debug mode: with the environment variable MXG_VALIDATE set (to anything
 *     but "" or "0"), every entry point that takes row_offsets first copies
 *     row_offsets (and, where it takes num_experts, expert_ids) to the host,
 *     synchronising `stream`, and returns MXG_ERROR_INVALID_VALUE without
 *     launching anything if an offset exceeds total_rows, an offset is below
 *     the one before it, or an expert id lies outside [0, num_experts);
 *     mxg_validation_message() then names the first violation.  (The
 *     malformed-routing convention of NvMxf4f8Strategy,
 *     prepare_swiglu_operands(), Raises: refuse instead of proceeding.)
 *     Without it, malformed routing is handled as described above.
 *   - Tile override: the FP8 rowwise GEMMs run 256-row tiles of 384 or 256
 *     columns where they use 256-row tiles at all (both give the same bits),
 *     chosen from total_rows, num_groups, N and the device's compute units;
 *     the environment variable MXG_FP8_TILE set to "256x384" or "256x256"
 *     forces one (read at each call; other values are ignored; 256x384 still
 *     needs N % 8 == 0).  For tuning and tests; mxg_fp8_tile reports the
 *     choice.
 */
#ifndef MXG_H
#define MXG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MXG_SUCCESS = 0,
    MXG_ERROR_INVALID_VALUE = 1, /* null pointer, bad enum, bad size, misaligned pointer */
    MXG_ERROR_NOT_SUPPORTED = 2, /* K or I not a multiple of 32, K past MXG_MAX_K, too many groups, format not offered */
    MXG_ERROR_LAUNCH = 3         /* the HIP runtime refused a launch */
} mxg_status;

typedef enum {
    MXG_FP8_E4M3_ROWWISE = 0, /* e4m3 codes, one fp32 scale per row (per-token / per-channel) */
    MXG_MXFP8_E4M3 = 1,       /* e4m3 codes, one E8M0 scale per 32 elements along K */
    MXG_MXFP4_E2M1 = 2        /* e2m1 codes packed 2 per byte, one E8M0 scale per 32 elements */
} mxg_format;

/* Largest num_groups any entry point accepts. */
#define MXG_MAX_GROUPS 1024

/* Largest K (elements per row) the grouped GEMM entry points accept: the
 * operand loads address a tile's rows from 32-bit offsets (up to 384 rows or,
 * on prepared weights, two 256-column blocks of K * 256 bytes).  Larger K
 * returns MXG_ERROR_NOT_SUPPORTED. */
#define MXG_MAX_K (1 << 22)

/*
 * mx_grouped_quantize -- per-expert dynamic quantization of BF16 rows.
 * (grouped_quantize_dynamic_scaled_fp4_async_kernel, description;
 *  NvMxf4f8Strategy, grouped_quantize() and quantize() -- the latter is the
 *  num_groups = 1, row_offsets = {0, total_rows} case;
 *  grouped_matmul_rowwise_dynamic_scaled_fp8, Args: a_scales.)
 *
 *   x_bf16   [total_rows, K] bf16 input.
 *   q        MXG_FP8_E4M3_ROWWISE, MXG_MXFP8_E4M3: [total_rows, K] u8;
 *            MXG_MXFP4_E2M1: [total_rows, K/2] u8.
 *   scales   MXG_FP8_E4M3_ROWWISE: fp32 [total_rows]; MX: u8 E8M0 [total_rows, K/32].
 *   row_offsets / num_groups as above.  Only covered rows of q and scales are
 *            written.
 *   expert_ids may be NULL; it is not read (these formats carry no per-expert
 *            tensor scale) and is accepted so the same routing tuple can be
 *            handed to quantize and matmul.
 *
 * Rowwise: amax = max |x| over the row; scale = amax / 448 (IEEE fp32
 * division); code = e4m3(x / scale) (IEEE fp32 division); a zero row gets
 * scale 0 and signed-zero codes.  MX: per 32-element block, X =
 * clamp(floor(log2 amax) - emax, -127, 127) with emax = 8 (e4m3) or 2 (e2m1),
 * scale code X + 127 (0 for an all-zero block), code = enc(x * 2^-X).
 * Weights are prepared with the same call (one group of num_experts*N rows).
 *
 * Errors: INVALID_VALUE for a null x/q/scales/row_offsets, a bad fmt,
 * K <= 0, total_rows < 0, num_groups < 0, misalignment; NOT_SUPPORTED for
 * K % 32 != 0 or num_groups > MXG_MAX_GROUPS.
 */
mxg_status mx_grouped_quantize(mxg_format fmt, const void* x_bf16, void* q, void* scales,
                               const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                               int64_t total_rows, int64_t K, hipStream_t stream);

/*
 * mx_grouped_quantize_gather -- mx_grouped_quantize with the routed rows
 * gathered from the source activations on the fly, so the permuted BF16
 * copy of the activations is never written.
 * (NvMxf4f8Strategy, grouped_quantize(): parameters indices and
 *  indices_divisor.  The page names them without defining them; the reading
 *  taken here: routed row t is source row indices[t] / indices_divisor,
 *  integer division -- with indices holding flat (token * top_k + k) slots
 *  and indices_divisor = top_k, the token's row.)
 *
 *   x_bf16          [num_src_rows, K] bf16 source rows (e.g. one per token).
 *   num_src_rows    rows of x_bf16.
 *   indices         [total_rows] int32, device.  Read for every row below
 *                   total_rows; a row whose entry is negative or whose
 *                   quotient is >= num_src_rows is skipped (left untouched),
 *                   so no read leaves x_bf16.
 *   indices_divisor >= 1.
 *   q, scales, row_offsets, expert_ids, num_groups, total_rows, K, stream:
 *                   as in mx_grouped_quantize; the results of a covered row
 *                   equal mx_grouped_quantize applied to its source row.
 *
 * Errors: those of mx_grouped_quantize, plus INVALID_VALUE for a null
 * indices, num_src_rows < 0, indices_divisor < 1 or a misaligned indices.
 */
mxg_status mx_grouped_quantize_gather(mxg_format fmt, const void* x_bf16, int64_t num_src_rows,
                                      const int32_t* indices, int32_t indices_divisor, void* q, void* scales,
                                      const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                                      int64_t total_rows, int64_t K, hipStream_t stream);

/*
 * mx_grouped_quantize_scatter -- the gathered quantize in token-major form:
 * each token row is read and quantized once and its result is stored to every
 * routed row that token feeds, through the inverse slot map (the row_of_slot
 * table mx_moe_combine takes).  A routed row is a copy of its token's row, so
 * the results equal mx_grouped_quantize_gather's for the same routing while
 * the token rows are read once instead of once per slot.
 * (NvMxf4f8Strategy, grouped_quantize(), Args indices and indices_divisor,
 *  with the reading given at mx_grouped_quantize_gather.)
 *
 *   x_tokens     [num_tokens, K] bf16 token rows.
 *   row_of_slot  int32 [num_tokens * top_k], device: the routed row of slot
 *                (token s, k).  Slots naming a row outside [0, total_rows)
 *                or a row no group covers are dropped.  A routed row named
 *                by several slots receives one of their results.
 *   top_k        slots per token, 1 .. 64.
 *   q, scales, row_offsets, expert_ids, num_groups, total_rows, K, stream:
 *                as in mx_grouped_quantize; routed rows no slot names are
 *                left untouched.
 *
 * Errors: INVALID_VALUE for a bad fmt, K <= 0, total_rows / num_groups /
 * num_tokens < 0, top_k < 1, a null pointer (x_tokens, row_of_slot, q,
 * scales, row_offsets) or misalignment (x_tokens and q on 16 bytes, fp32
 * scales, row_offsets and row_of_slot on 4); NOT_SUPPORTED for K % 32 != 0,
 * num_groups > MXG_MAX_GROUPS, top_k > 64, FP8 rowwise rows longer than 8192
 * elements, or num_tokens * top_k > INT32_MAX.  total_rows, num_groups or
 * num_tokens of 0 is a no-op.
 */
mxg_status mx_grouped_quantize_scatter(mxg_format fmt, const void* x_tokens, int64_t num_tokens,
                                       const int32_t* row_of_slot, int32_t top_k, void* q, void* scales,
                                       const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                                       int64_t total_rows, int64_t K, hipStream_t stream);

/*
 * mx_grouped_matmul -- ragged grouped GEMM with BF16 output.
 * (grouped_matmul_rowwise_dynamic_scaled_fp8, description and Args;
 *  NvMxf4f8Strategy, grouped_matmul().)
 *
 * For each taken group g with e = expert_ids[g], each row t it owns and each
 * n in [0, N):
 *   MXG_FP8_E4M3_ROWWISE:
 *     c[t,n] = bf16( (sum_k a[t,k] * b[e,n,k]) * a_scales[t] * b_scales[e,n] )
 *     with the sum accumulated in fp32 and the two scales applied once after
 *     it, in that order, in fp32.
 *   MX formats:
 *     c[t,n] = bf16( sum_blocks 2^(sa[t,blk]-127) * 2^(sb[e,n,blk]-127)
 *                    * sum_{k in blk} a[t,k] * b[e,n,k] ), fp32 accumulation.
 *
 *   a_q       [total_rows, K] u8 (e4m3) or [total_rows, K/2] u8 (e2m1).
 *   a_scales  fp32 [total_rows] (rowwise) or u8 [total_rows, K/32] (MX).
 *   b_q       [num_experts, N, K] u8 or [num_experts, N, K/2] u8 -- K innermost
 *             (the weight is already transposed).
 *   b_scales  fp32 [num_experts, N] (rowwise) or u8 [num_experts, N, K/32] (MX).
 *   c_bf16    [total_rows, N] bf16 output; only covered rows are written.
 *   max_rows_per_group_hint  largest group size if the host knows it, else 0.
 *             It only steers the choice of tile shape; results never depend
 *             on it (grouped_matmul_rowwise_dynamic_scaled_fp8, Args:
 *             max_num_tokens_per_expert).
 *
 * Errors: INVALID_VALUE for null pointers, a bad fmt, K/N/num_experts <= 0,
 * total_rows/num_groups < 0, misalignment (codes and c on 16 bytes; rowwise
 * fp32 scales on 4; MX scale tensors on 16, since they are streamed in
 * 16-byte pieces); NOT_SUPPORTED for K % 32 != 0, K > MXG_MAX_K or
 * num_groups > MXG_MAX_GROUPS.  The same pointer rules hold for
 * mx_grouped_matmul_swiglu.
 */
mxg_status mx_grouped_matmul(mxg_format fmt, const void* a_q, const void* a_scales, const void* b_q,
                             const void* b_scales, void* c_bf16, const uint32_t* row_offsets,
                             const int32_t* expert_ids, int32_t num_groups, int32_t num_experts,
                             int64_t total_rows, int64_t N, int64_t K, int64_t max_rows_per_group_hint,
                             hipStream_t stream);

/*
 * mx_prepare_weights_fp8, mx_prepared_weights_bytes,
 * mx_grouped_matmul_prepared -- FP8 rowwise expert weights rearranged once
 * into the layout the GEMM's load ring copies to LDS as it is, and the grouped
 * GEMM that reads them.  (The counterpart here of the weight preparation step
 * of NvMxf4f8Strategy, prepare_weight_scales(), which rearranges weight
 * scales into its kernel's layout; the arithmetic is mx_grouped_matmul's.)
 *
 * The ring streams each row of a weight tile 64 bytes of K at a time; in the plain [E, N, K] layout each such piece is half a 128-byte line
 * of its own row, and the per-request cost of the load path, not its bytes,
 * sets the GEMM's pace.  Prepared, the 256 x 64-byte block of 256 columns
 * and one stage is contiguous (16 KiB, rows in the order and 16-byte piece order the
 * ring places them in LDS), so each load instruction reads whole lines.
 *
 * mx_prepared_weights_bytes(E, N, K): bytes of the prepared weights,
 *   E * ceil(N / 256) * 256 * K; -1 if E, N or K <= 0 or K % 64 != 0.
 * mx_prepare_weights_fp8(b_q, E, N, K, b_prepared, stream): b_q [E, N, K] u8
 *   e4m3 codes (K innermost, as mx_grouped_matmul takes them); b_prepared
 *   receives mx_prepared_weights_bytes(E, N, K) bytes: for expert e, tile
 *   nt = n / 256 and stage s = k / 64, block (e * ceil(N / 256) + nt) *
 *   (K / 64) + s of 256 * 64 bytes; in it row r = n % 256 at byte 64 r, the
 *   16-byte pieces of the row permuted as the ring's LDS swizzle permutes them
 *   (piece position p holds piece p ^ ((r >> 2) & 3)).  Rows past N are zero.
 *   The layout is private to this library: only mx_grouped_matmul_prepared
 *   reads it.  Asynchronous on `stream`.
 * mx_grouped_matmul_prepared(...): mx_grouped_matmul for MXG_FP8_E4M3_ROWWISE
 *   with b_prepared in place of b_q; every other argument as there (no tile
 *   hint: it always runs 256-row tiles, of 384 or 256 columns as described
 *   under the tile override above; a 384-column tile reads one and a half
 *   256-column blocks per stage).  Results are
 *   bit-identical to mx_grouped_matmul on the weights the prepared ones came
 *   from.
 *
 * Errors: INVALID_VALUE for null pointers, sizes <= 0 (total_rows /
 * num_groups < 0), misalignment (codes, prepared weights and c on 16 bytes,
 * scales on 4); NOT_SUPPORTED for K % 64 != 0, num_groups > MXG_MAX_GROUPS,
 * N > INT32_MAX / 2 or total_rows > INT32_MAX, and for the GEMM also
 * K > MXG_MAX_K.  total_rows or num_groups of 0 is a no-op.
 */
int64_t mx_prepared_weights_bytes(int64_t num_experts, int64_t N, int64_t K);
mxg_status mx_prepare_weights_fp8(const void* b_q, int32_t num_experts, int64_t N, int64_t K, void* b_prepared,
                                  hipStream_t stream);
mxg_status mx_grouped_matmul_prepared(const void* a_q, const void* a_scales, const void* b_prepared,
                                      const void* b_scales, void* c_bf16, const uint32_t* row_offsets,
                                      const int32_t* expert_ids, int32_t num_groups, int32_t num_experts,
                                      int64_t total_rows, int64_t N, int64_t K, hipStream_t stream);

/*
 * mx_grouped_matmul_nvfp4 -- ragged grouped GEMM of NVFP4 operands.
 * (NvMxf4f8Strategy, grouped_matmul(), description and Args expert_scales;
 *  is_nvfp4.  The pages name one scale per expert, applied after the
 *  product, and give no arithmetic; reading:)
 *
 *   out[t, n] = bf16( expert_scales[e] * sum_b sa[t, b] * sb[e, n, b] *
 *                     sum_{k in block b} qa[t, k] * qb[e, n, k] )
 * with e = expert_ids[g] for the group g covering row t, 16-element blocks,
 * sa / sb the E4M3 values of the scale codes and qa / qb the e2m1 values.
 *
 *   a_q       [total_rows, K/2] u8 e2m1 codes (mx_grouped_quantize_nvfp4).
 *   a_scales  [total_rows, K/16] u8 E4M3.
 *   b_q       [num_experts, N, K/2] u8; b_scales [num_experts, N, K/16] u8.
 *   expert_scales  fp32 [num_experts] (e.g. 1 / (sf_a * sf_w) for the tensor
 *             scales the operands were quantized with).
 *   c_bf16    [total_rows, N] bf16; only covered rows are written.
 *
 * gfx950's scaled matrix-core ops take E8M0 scales per 32 elements only, so
 * each NVFP4 element becomes an exact f16 value (code times block scale)
 * and the product runs on the f16 matrix cores with fp32 accumulation.
 *
 * Errors: INVALID_VALUE for a null pointer, K/N <= 0, num_experts <= 0,
 * total_rows/num_groups < 0, misalignment (codes, scales and c on 16 bytes);
 * NOT_SUPPORTED for K % 512 != 0, K > MXG_MAX_K, num_groups > MXG_MAX_GROUPS
 * or sizes past the int32 range.
 */
mxg_status mx_grouped_matmul_nvfp4(const void* a_q, const void* a_scales, const void* b_q, const void* b_scales,
                                   const float* expert_scales, void* c_bf16, const uint32_t* row_offsets,
                                   const int32_t* expert_ids, int32_t num_groups, int32_t num_experts,
                                   int64_t total_rows, int64_t N, int64_t K, int64_t max_rows_per_group_hint,
                                   hipStream_t stream);

/*
 * mx_grouped_matmul_swiglu_nvfp4 -- NVFP4 gate/up grouped GEMM + SwiGLU +
 * NVFP4 requant, fused.
 * (NvMxf4f8Strategy, grouped_matmul_swiglu(), Args expert_scales,
 *  input_scales and a_row_scales; prepare_swiglu_operands(), Returns.  In
 *  short: one epilogue factor per expert; one output-side scale per expert,
 *  which the caller hands over already inverted; and, for this format, an
 *  optional BF16 factor per routed row that multiplies in together with the
 *  expert factor, ahead of the activation.  The arithmetic is not given;
 *  reading:)
 *
 *   g_j, u_j = bf16( acc * fl32(expert_scales[e] * a_row_scales[t]) ) for
 *              columns 2j, 2j+1 of the NVFP4 GEMM against W[e] (rows
 *              interleaved gate, up), acc its fp32 sum;
 *   y_j      = bf16( g_j / (1 + e^-g_j) * u_j ), fp32;
 *   (y_q, y_scales) = the NVFP4 quantization of y along j (blocks of 16)
 *              under sf = y_tensor_scales[e], exactly as
 *              mx_grouped_quantize_nvfp4 quantizes a row.
 *
 *   a_q, a_scales, w_q [E, 2I, K/2], w_scales [E, 2I, K/16], expert_scales
 *              as mx_grouped_matmul_nvfp4.
 *   a_row_scales_bf16  bf16 [total_rows] or NULL (all 1).
 *   y_tensor_scales    fp32 [num_experts], encode side (1 / input_scale).
 *   y_q [total_rows, I/2] u8; y_scales [total_rows, I/16] u8 E4M3.
 * Without row scales the result equals mx_grouped_matmul_nvfp4 followed by
 * mx_silu_quantize_nvfp4, byte for byte.
 *
 * Errors: as mx_grouped_matmul_nvfp4; NOT_SUPPORTED also for I % 32 != 0.
 */
mxg_status mx_grouped_matmul_swiglu_nvfp4(const void* a_q, const void* a_scales, const void* w_q,
                                          const void* w_scales, const float* expert_scales,
                                          const void* a_row_scales_bf16, const float* y_tensor_scales, void* y_q,
                                          void* y_scales, const uint32_t* row_offsets, const int32_t* expert_ids,
                                          int32_t num_groups, int32_t num_experts, int64_t total_rows, int64_t I,
                                          int64_t K, int64_t max_rows_per_group_hint, hipStream_t stream);

/*
 * mx_silu_quantize_nvfp4 -- SwiGLU + NVFP4 requant of a BF16 gate/up tensor.
 * (NvMxf4f8Strategy, fused_silu_quantize(input_scales): the gated activation,
 *  then quantization, with the inverted per-expert scale.)
 *
 *   h_bf16    [total_rows, 2I] bf16, column 2j = gate_j, 2j+1 = up_j.
 *   y_tensor_scales  fp32 [num_experts], encode side; rows of group g use
 *             y_tensor_scales[expert_ids[g]]; a group whose id lies outside
 *             [0, num_experts) is skipped.
 *   y_q [total_rows, I/2] u8; y_scales [total_rows, I/16] u8 E4M3; only
 *             covered rows are written.
 *
 * Errors: INVALID_VALUE for a null pointer, I <= 0, negative sizes,
 * num_experts <= 0, misalignment; NOT_SUPPORTED for I % 16 != 0 or
 * num_groups > MXG_MAX_GROUPS.
 */
mxg_status mx_silu_quantize_nvfp4(const void* h_bf16, void* y_q, void* y_scales, const float* y_tensor_scales,
                                  const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                                  int32_t num_experts, int64_t total_rows, int64_t I, hipStream_t stream);

/*
 * mx_grouped_matmul_swiglu -- fused gate/up grouped GEMM + SwiGLU + MXFP4 requant.
 * (NvMxf4f8Strategy, grouped_matmul_swiglu(): the grouped matmul followed by
 *  fused_silu_quantize(), folded into one kernel, byte-identical to the
 *  chained path; weights arrive (gate, up)-interleaved.)
 *
 *   fmt       MXG_MXFP4_E2M1 or MXG_MXFP8_E4M3 (the input format of a_q / w_q).
 *   a_q, a_scales  as mx_grouped_matmul (MX layouts).
 *   w_q       [num_experts, 2I, K] u8 (e4m3) or [num_experts, 2I, K/2] u8 (e2m1);
 *             row 2j is gate_j and row 2j+1 is up_j.
 *   w_scales  u8 [num_experts, 2I, K/32], rows as w_q.
 *   y_q       [total_rows, I/2] u8, e2m1 codes of y (element 2i low nibble).
 *   y_scales  [total_rows, I/32] u8 E8M0.
 *
 * g_j and u_j are the BF16 outputs mx_grouped_matmul would produce for
 * columns 2j and 2j+1 (bit-identical: same accumulation order), y_j =
 * bf16( g_j / (1 + e^-g_j) * u_j ) computed in fp32, and (y_q, y_scales) is
 * the MXFP4 quantization of y along j in blocks of 32 -- exactly what
 * mx_grouped_matmul followed by mx_silu_quantize produces.
 *
 * Errors: as mx_grouped_matmul; NOT_SUPPORTED also for I % 32 != 0 or a
 * rowwise fmt.
 */
mxg_status mx_grouped_matmul_swiglu(mxg_format fmt, const void* a_q, const void* a_scales, const void* w_q,
                                    const void* w_scales, void* y_q, void* y_scales,
                                    const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                                    int32_t num_experts, int64_t total_rows, int64_t I, int64_t K,
                                    int64_t max_rows_per_group_hint, hipStream_t stream);

/*
 * mx_silu_quantize -- SwiGLU + MXFP4 requant of a BF16 gate/up tensor.
 * (NvMxf4f8Strategy, fused_silu_quantize(): apply the gated activation, then
 *  quantize.)
 *
 *   h_bf16    [total_rows, 2I] bf16; column 2j is gate_j, column 2j+1 is up_j
 *             (the output of mx_grouped_matmul against interleaved weights).
 *   y_q, y_scales  as mx_grouped_matmul_swiglu.  Only covered rows are written.
 *
 * Errors: INVALID_VALUE for null pointers, I <= 0, total_rows/num_groups < 0,
 * misalignment; NOT_SUPPORTED for I % 32 != 0 or num_groups > MXG_MAX_GROUPS.
 */
mxg_status mx_silu_quantize(const void* h_bf16, void* y_q, void* y_scales, const uint32_t* row_offsets,
                            int32_t num_groups, int64_t total_rows, int64_t I, hipStream_t stream);

/*
 * mx_grouped_quantize_nvfp4 -- per-expert dynamic quantization of BF16 rows to
 * NVFP4.
 * (NvMxf4f8Strategy, is_nvfp4 and grouped_quantize(input_scale);
 *  grouped_quantize_dynamic_scaled_fp4_async_kernel, Args: sf_tensor, one
 *  tensor-level scale for each expert.  The pages name the format and the
 *  scale without their arithmetic; the reading taken here follows.)
 *
 *   x_bf16         [total_rows, K] bf16 input.
 *   q              [total_rows, K/2] u8, e2m1 codes, element 2i in bits 0..3.
 *   scales         [total_rows, K/16] u8, one E4M3 code per 16-element block.
 *   tensor_scales  fp32 [num_experts]: the encode-side tensor scale sf of each
 *                  expert; the rows of group g use tensor_scales[expert_ids[g]].
 *   row_offsets / expert_ids / num_groups as above; a group whose expert id
 *                  lies outside [0, num_experts) is skipped (its rows are not
 *                  written), and only covered rows of q and scales are written.
 *
 * Per block, with amax its largest |x|: scale code = e4m3(min(fl32(fl32(amax /
 * 6) * sf), 448)); with s that code's value, r = fl32(sf / s) (0 when s is 0)
 * and each code = e2m1(fl32(x * r)).  Every fl32 step is one IEEE binary32
 * operation; so x is about e2m1 * s / sf.  sf is expected finite and > 0.
 * Weights are prepared with the same call: one group of N rows per expert,
 * expert_ids = 0 .. E-1, tensor_scales = the weights' own.
 *
 * Errors: INVALID_VALUE for a null pointer, K <= 0, total_rows < 0,
 * num_groups < 0, num_experts <= 0, misalignment; NOT_SUPPORTED for
 * K % 16 != 0 or num_groups > MXG_MAX_GROUPS.
 */
mxg_status mx_grouped_quantize_nvfp4(const void* x_bf16, void* q, void* scales, const float* tensor_scales,
                                     const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                                     int32_t num_experts, int64_t total_rows, int64_t K, hipStream_t stream);

/*
 * mx_grouped_quantize_padded, mx_grouped_matmul_padded,
 * mx_grouped_matmul_swiglu_padded -- the MX entry points with the activation
 * block scales in a padded / slot-strided layout.
 * (grouped_quantize_dynamic_scaled_fp4_async_kernel: scales_offsets, the
 *  per-expert offsets into the scale tensor, found with row_offsets by
 *  binary search; NvMxf4f8Strategy, grouped_quantize(): "padded scale
 *  alignment", scales_offset, and a_scales_max_padded_m of grouped_matmul();
 *  Struct_ep_dispatch_mxfp4: the slot layout [n_local_experts *
 *  max_padded_M, K_SCALES] with slot stride max_padded_M * K_SCALES.  The
 *  pages give no formula; reading:)
 *
 * Routed row t of group g keeps its K/32 E8M0 scale bytes in row
 *   scales_offsets[g] + (t - row_offsets[g])
 * of a scale tensor [scale_rows, K/32] u8 (the slot layout is scales_offsets[g]
 * = expert_ids[g] * max_padded_M, scale_rows = n_local_experts *
 * max_padded_M).  scales_offsets is uint32 [num_groups] (device).  The quantize
 * writes the codes of row t as mx_grouped_quantize does and its scales into
 * that row; a row whose scale row lies at or past scale_rows is left
 * untouched (codes too); scale rows nothing maps to (the padding) are never
 * written.  The GEMMs read A's scales through the same map (weights keep the
 * dense layout); a row whose scale row lies at or past scale_rows is not
 * computed and its output row is left untouched, whatever tile shape is
 * chosen.  Results are otherwise
 * identical to the dense entry points.  Other arguments, layouts and errors as
 * mx_grouped_quantize / mx_grouped_matmul / mx_grouped_matmul_swiglu;
 * NOT_SUPPORTED also for MXG_FP8_E4M3_ROWWISE (its scale is per row, not per
 * block); INVALID_VALUE also for scale_rows < 0, a null or misaligned
 * scales_offsets (4 bytes), or a_scales not on 16 bytes.
 */
mxg_status mx_grouped_quantize_padded(mxg_format fmt, const void* x_bf16, void* q, void* scales,
                                      const uint32_t* scales_offsets, int64_t scale_rows,
                                      const uint32_t* row_offsets, int32_t num_groups, int64_t total_rows, int64_t K,
                                      hipStream_t stream);

mxg_status mx_grouped_matmul_padded(mxg_format fmt, const void* a_q, const void* a_scales,
                                    const uint32_t* a_scales_offsets, int64_t a_scale_rows, const void* b_q,
                                    const void* b_scales, void* c_bf16, const uint32_t* row_offsets,
                                    const int32_t* expert_ids, int32_t num_groups, int32_t num_experts,
                                    int64_t total_rows, int64_t N, int64_t K, int64_t max_rows_per_group_hint,
                                    hipStream_t stream);

mxg_status mx_grouped_matmul_swiglu_padded(mxg_format fmt, const void* a_q, const void* a_scales,
                                           const uint32_t* a_scales_offsets, int64_t a_scale_rows, const void* w_q,
                                           const void* w_scales, void* y_q, void* y_scales,
                                           const uint32_t* row_offsets, const int32_t* expert_ids,
                                           int32_t num_groups, int32_t num_experts, int64_t total_rows, int64_t I,
                                           int64_t K, int64_t max_rows_per_group_hint, hipStream_t stream);

/*
 * mx_grouped_quantize_nvfp4_padded, mx_grouped_matmul_nvfp4_padded -- the
 * NVFP4 quantize and grouped GEMM with the activation block scales in the
 * padded / slot-strided layout above (the offsets-into-the-scale-tensor
 * argument of grouped_quantize_dynamic_scaled_fp4_async_kernel covers NVFP4
 * as well as the MX formats).  Routed row t of group g keeps its K/16 E4M3
 * scale bytes in row scales_offsets[g] + (t - row_offsets[g]) of a
 * [scale_rows, K/16] u8 tensor; the rest as for MX: the quantize leaves a
 * row whose scale row lies at or past scale_rows untouched (codes too) and
 * never writes padding rows; the GEMM reads A's scales through the map and
 * leaves such rows of c untouched.  Other arguments, layouts and errors as
 * mx_grouped_quantize_nvfp4 / mx_grouped_matmul_nvfp4, plus INVALID_VALUE
 * for scale_rows < 0 or a null or misaligned scales_offsets (4 bytes); the
 * GEMM's a_scales must be on 16 bytes.
 */
mxg_status mx_grouped_quantize_nvfp4_padded(const void* x_bf16, void* q, void* scales, const float* tensor_scales,
                                            const uint32_t* scales_offsets, int64_t scale_rows,
                                            const uint32_t* row_offsets, const int32_t* expert_ids,
                                            int32_t num_groups, int32_t num_experts, int64_t total_rows, int64_t K,
                                            hipStream_t stream);
mxg_status mx_grouped_matmul_nvfp4_padded(const void* a_q, const void* a_scales, const uint32_t* a_scales_offsets,
                                          int64_t a_scale_rows, const void* b_q, const void* b_scales,
                                          const float* expert_scales, void* c_bf16, const uint32_t* row_offsets,
                                          const int32_t* expert_ids, int32_t num_groups, int32_t num_experts,
                                          int64_t total_rows, int64_t N, int64_t K, int64_t max_rows_per_group_hint,
                                          hipStream_t stream);

/*
 * mx_moe_combine -- the MoE combine after the down-projection (itself
 * mx_grouped_matmul with K = I on the fused output): for every token t,
 *   out[t, n] = bf16( sum_{k < top_k} weights[t*top_k + k] *
 *                                     y[row_of_slot[t*top_k + k], n] ).
 * (grouped_matmul_rowwise_dynamic_scaled_fp8, Parameters:
 *  elementwise_lambda_fn, the output epilogue at (global_row, n) where the
 *  weighting and combine attach; NvMxf4f8Strategy, prepare_swiglu_operands(),
 *  the EP-combine path; Struct_ep_dispatch_mxfp4, src_info.  The pages name
 *  the combine without defining it; the reading taken is the router-weighted
 *  sum above, with the token's slots summed in order k = 0, 1, ....)
 *
 *   y_bf16       [total_rows, H] bf16 routed rows (the down-projection output).
 *   row_of_slot  int32 [num_tokens * top_k]: the routed row of slot
 *                (t, k), or any value outside [0, total_rows) for a slot
 *                that was dropped (it contributes nothing).
 *   weights      fp32 [num_tokens * top_k] router weights.
 *   out_bf16     [num_tokens, H] bf16; every row is written (a token with no
 *                live slot gets zeros).
 * The sum is accumulated in fp32 (fused multiply-add per slot) and rounded
 * once to bf16, nearest-even.  Deterministic: no atomics.
 *
 * Errors: INVALID_VALUE for H <= 0, total_rows < 0, num_tokens < 0,
 * top_k < 1, a null row_of_slot / weights / out_bf16 (or y_bf16 with
 * total_rows > 0) or misalignment; NOT_SUPPORTED for H % 8 != 0 or
 * num_tokens * top_k > INT32_MAX.  num_tokens == 0 is a no-op.
 */
mxg_status mx_moe_combine(const void* y_bf16, int64_t total_rows, int64_t H, const int32_t* row_of_slot,
                          const float* weights, int64_t num_tokens, int32_t top_k, void* out_bf16,
                          hipStream_t stream);

/*
 * mxg_clock_probe -- a measurement aid, not part of the path: one wave on
 * `stream` sleeps for window_us microseconds of the GPU's constant 100 MHz
 * counter and counts the shader clock meanwhile.  On completion
 *   out[0] = shader-clock ticks, out[1] = 100 MHz ticks of the window,
 * so the average engine clock is 100 MHz * out[0] / out[1].  Enqueued on a
 * stream of its own beside other work, it measures the clock that work runs
 * at (it holds one wave slot of one compute unit).  out: device uint64 [2],
 * 8-byte aligned.  INVALID_VALUE for a null or misaligned out, or window_us
 * outside [1, MXG_CLOCK_PROBE_MAX_US].
 */
#define MXG_CLOCK_PROBE_MAX_US 10000000

/*
 * mxg_fp8_tile -- which tile an FP8 rowwise grouped GEMM of this size would
 * run (not a step of the path: for tuning and for tests of the choice).  The
 * host sees only the sizes, as the GEMM does: num_groups, total_rows, N, K,
 * the hint of mx_grouped_matmul and whether the weights are prepared
 * (mx_grouped_matmul_prepared).  Returns 384 or 256 for 256-row tiles of that
 * many columns, 32 for the 32 x 256 tile of the few-rows-per-group regime,
 * and 0 where such a call would launch nothing or be refused (sizes <= 0, K
 * not a multiple of 32 (of 64 for prepared weights) or past MXG_MAX_K, too
 * many groups).  Follows MXG_FP8_TILE and the device's compute units as the
 * GEMM does (256 when no device is visible).  Touches no device memory.
 */
int32_t mxg_fp8_tile(int32_t num_groups, int64_t total_rows, int64_t N, int64_t K,
                     int64_t max_rows_per_group_hint, int32_t prepared);
mxg_status mxg_clock_probe(unsigned long long* out, int64_t window_us, hipStream_t stream);

/*
 * mxg_validation_message -- under MXG_VALIDATE, the first violation found by
 * the calling thread's last refused call ("" if its last validated call
 * passed).  Valid until that thread's next validated call.
 *
 * mxg_routing_violation -- the same check on host arrays: row_offsets_host
 * [num_groups + 1]; expert_ids_host [num_groups] or NULL (ids not checked,
 * nor when num_experts <= 0).  Returns 1 and writes a description into msg
 * (msg_len bytes, NUL-terminated; msg may be NULL) for malformed routing, 0
 * for well-formed routing (msg gets ""), -1 for a NULL row_offsets_host or a
 * negative num_groups / total_rows.  Host memory only; no GPU is touched.
 */
const char* mxg_validation_message(void);
int mxg_routing_violation(const uint32_t* row_offsets_host, const int32_t* expert_ids_host, int32_t num_groups,
                          int32_t num_experts, int64_t total_rows, char* msg, int64_t msg_len);

/* Static, human-readable name of a status code. */
const char* mxg_status_string(mxg_status status);

#ifdef __cplusplus
}
#endif

#endif /* MXG_H */
