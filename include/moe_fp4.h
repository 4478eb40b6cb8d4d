/*
 * moe_fp4.h -- C ABI of the MI355X (gfx950) NVFP4 block-scaled MoE grouped GEMM.
 *
 * The operation: in Mixture-of-Experts decode the router sends every token to
 * a few experts, and each expert multiplies only its own tokens by its weights,
 * so one launch serves many small GEMMs whose heights differ ("Peering into the
 * CUTLASS Kernel Cache", section "Knowledge Required", the MoE grouped GEMM
 * item; "Peering into the CUTLASS Kernel", section "Input Knowledge Required",
 * item 4).  Operands are NVFP4: 4-bit codes, two to a byte, and an 8-bit float
 * scale for every 16 consecutive codes ("Peering into the CUTLASS
 * SharedStorage", section "Input Knowledge", item 3).  Tile M is the tokens of
 * one expert, N the output features, K the reduction dimension (same page,
 * item 5).  Accumulation is FP32 and the output BF16 (same page, "Why This
 * Message Was Written", the epilogue staging estimate).
 *
 * Formats and conventions used by every entry point:
 *   - FP4 element: E2M1 (OCP Microscaling v1.0): magnitudes 0, .5, 1, 1.5, 2,
 *     3, 4, 6; bit 3 is the sign.  Element 2i of a row is the low nibble of
 *     byte i, element 2i+1 the high nibble.
 *   - Block scale: E4M3 (OCP OFP8 v1.0, no Inf, 0x7F/0xFF NaN), one per 16
 *     consecutive elements along K, blocks starting at multiples of 16.
 *   - Tensor scale: an FP32 decode multiplier.  An element's value is
 *     E2M1(code) * E4M3(block scale) * tensor scale.  Activations have one
 *     tensor scale; weights have one per expert.
 *   - Matrices are row-major with K contiguous: activations q[rows][k/2],
 *     sf[rows][k/16]; weights w_q[E][n][k/2], w_sf[E][n][k/16].
 *
 * Ownership: the caller owns every buffer; the library allocates no device
 * memory, keeps no pointer after a call returns and holds no per-call state,
 * so calls on different streams may run concurrently.
 * Asynchrony: each call validates its arguments on the host, enqueues its
 * kernels on `stream` (a hipStream_t; NULL = the default stream) and returns.
 * A call that returns an error has enqueued nothing (except MOE_FP4_ERR_HIP,
 * which reports a failed launch).  Results are visible after the stream
 * synchronises.  Device pointers must be device (or managed) memory.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  MOE_FP4_OK = 0,
  MOE_FP4_ERR_NULL = 1,        /* a required pointer is NULL                        */
  MOE_FP4_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent   */
  MOE_FP4_ERR_ALIGN = 3,       /* a pointer or leading dimension is misaligned       */
  MOE_FP4_ERR_UNSUPPORTED = 4, /* well-formed but outside what the kernels handle    */
  MOE_FP4_ERR_HIP = 5,         /* the HIP runtime reported an error                  */
  MOE_FP4_ERR_ARG = 6          /* an enumerated argument has an unknown value, or    */
                               /* buffers that must be distinct overlap              */
};

/* Input element types of moe_fp4_quantize. */
enum { MOE_FP4_IN_BF16 = 0, MOE_FP4_IN_FP32 = 1 };

/* Tensor-scale modes of moe_fp4_quantize. */
enum {
  MOE_FP4_SCALE_STATIC = 0, /* use *tensor_scale as given (a calibrated scale, > 0)  */
  MOE_FP4_SCALE_DYNAMIC = 1 /* compute it from the data and write it to *tensor_scale */
};

/*
 * moe_fp4_quantize -- NVFP4-quantise a [rows][k] matrix (activations).
 *
 * The pages give the packing (two 4-bit values per byte) and the 16-element
 * FP8 block scale ("Peering into the CUTLASS SharedStorage", "Input
 * Knowledge", item 3) but not the recipe; this library defines it as follows,
 * with fl() one IEEE binary32 operation rounded to nearest even and division a
 * true division (not a reciprocal multiply):
 *   1. tensor scale g: DYNAMIC: g = amax > 0 ? fl(amax / 2688) : 1, where amax
 *      is the largest |x| of the whole matrix and 2688 = 6 * 448; written to
 *      *tensor_scale.  STATIC: g = *tensor_scale.
 *   2. per row, per block of 16: r = fl(max|x_block| / fl(6 g)),
 *      sf = E4M3(r) rounded to nearest even, saturating at 448;
 *      s = fl(E4M3value(sf) * g).
 *   3. per element: y = (s == 0) ? +0 : fl(x / s); code = E2M1(y) rounded to
 *      nearest even, saturating at 6; the sign bit is the sign of y.
 * The result is bit-exact: the same q, sf and g bits on every run and stream.
 *
 *   x            device, [rows][ld_x] elements of in_dtype (BF16 or FP32); the
 *                first k of each row are used.  16-byte aligned base, and
 *                ld_x * sizeof(element) a multiple of 16.
 *   in_dtype     MOE_FP4_IN_BF16 or MOE_FP4_IN_FP32.
 *   rows         >= 0 (0 is a no-op apart from the DYNAMIC scale, which is 1).
 *   k            > 0, a multiple of 16.
 *   ld_x         >= k.
 *   q            device, [rows][k/2] bytes, 8-byte aligned.
 *   sf           device, [rows][k/16] bytes.
 *   tensor_scale device, one float: input (STATIC, must be finite and > 0) or
 *                output (DYNAMIC).  4-byte aligned.
 *   scale_mode   MOE_FP4_SCALE_STATIC or MOE_FP4_SCALE_DYNAMIC.
 *   stream       hipStream_t or NULL.
 * Inputs must be finite; the result for NaN or Inf inputs is unspecified.
 * DYNAMIC mode also needs amax = 0 or fl(amax / 2688) > 0 (amax above about
 * 2^-138); below that g underflows to 0 and the block scales are undefined.
 * x, q, sf and tensor_scale must not overlap (q also carries values between
 * the two passes of the DYNAMIC mode).
 * Block indices are 32-bit integers up to about 2.1e9 blocks and 64-bit above;
 * the environment variable MOE_FP4_INDEX64=1 selects the 64-bit build for every
 * size (the same bits; it exists so that build can be tested on small inputs).
 * Errors: NULL (x, q, sf or tensor_scale NULL with rows > 0; tensor_scale
 * NULL always), SHAPE (rows < 0, k <= 0, k % 16, ld_x < k, or x's extent
 * not representable in 64 bits), ALIGN, ARG
 * (unknown in_dtype or scale_mode; overlapping buffers), HIP.
 */
int moe_fp4_quantize(const void* x, int in_dtype, int64_t rows, int64_t k, int64_t ld_x,
                     uint8_t* q, uint8_t* sf, float* tensor_scale, int scale_mode,
                     void* stream);

/*
 * moe_grouped_gemm_fp4 -- NVFP4 block-scaled grouped GEMM over experts.
 *
 * For each expert e and each output row r in [off[e], off[e+1]) and column
 * j in [0, n):
 *     out[r][j] = bf16( a_scale * w_scale[e] * sum_k A(src(r), k) * W(e, j, k) )
 * where A(i, k) = E2M1(a_q code) * E4M3(a_sf[i][k/16]),
 *       W(e, j, k) = E2M1(w_q code) * E4M3(w_sf[e][j][k/16]),
 *       src(r) = a_row_index ? a_row_index[r] : r,
 * the sum is accumulated in FP32 from exactly dequantised products, and bf16()
 * rounds to nearest even.  Multiplying many expert GEMMs in one launch is the
 * grouped problem of "Peering into the CUTLASS Kernel", "Input Knowledge
 * Required", item 4.  Columns j >= n of `out` and rows outside
 * [off[0], off[E]) are never written; an empty expert writes nothing.
 *
 *   a_q          device, [a_rows][k/2] packed activation codes, 16-byte aligned.
 *   a_sf         device, [a_rows][k/16] activation block scales, 16-byte aligned.
 *   a_scale      device, one float: activation tensor scale.
 *   a_rows       rows of a_q / a_sf; >= m_total when a_row_index is NULL.
 *   a_row_index  device, [m_total] int32 in [0, a_rows), or NULL for identity.
 *                Lets rows be gathered in expert order without a copy (each
 *                token quantised once, read once per expert it is routed to).
 *   w_q          device, [num_experts][n][k/2] packed weight codes, 16-byte aligned.
 *   w_sf         device, [num_experts][n][k/16] weight block scales, 16-byte aligned.
 *   w_scale      device, [num_experts] floats: per-expert weight tensor scales.
 *   expert_offsets device, [num_experts+1] int32, offsets[0] = 0, non-decreasing,
 *                offsets[E] = m_total.  These are device-side preconditions, not
 *                checked; the kernel clamps every offset into [0, m_total] and
 *                every gathered row into [0, a_rows), so a violation cannot
 *                read or write outside the buffers described here.
 *   num_experts  >= 1.
 *   m_total      >= 0 (0 is a no-op).
 *   n            >= 1, a multiple of 16.
 *   k            >= 1, a multiple of 256 (UNSUPPORTED otherwise).
 *   out          device, [m_total][ldo] BF16 (uint16 bit patterns), 16-byte
 *                aligned; ldo >= n and a multiple of 8.
 *   stream       hipStream_t or NULL.
 * No host synchronisation, no device allocation and no workspace (see
 * moe_grouped_gemm_fp4_workspace_size).  Deterministic: the same inputs give
 * the same output bits (no atomics in the accumulation).
 * Tile choice: by the average rows per expert (moe_grouped_gemm_fp4_plan).  A
 * workgroup tile whose 128 or 256 output rows span 2^31 - 4096 bytes or more
 * at this ldo (ldo above about 2^22) is replaced by per-wavefront items of 64
 * rows, which address one item's rows with 32-bit offsets; the result is the
 * same to the parity bar.  With the environment variable MOE_FP4_LOG set (not
 * "0"), each GEMM entry point prints its sizes and chosen tile to stderr
 * whenever they differ from the previous call's.
 * Errors: NULL, SHAPE (num_experts < 1, m_total < 0, n < 1, k < 1, ldo < n,
 * a_rows < m_total without an index, a_rows < 1 with m_total > 0),
 * ALIGN, UNSUPPORTED (n % 16, k % 256, num_experts > 8192, sizes whose byte
 * offsets need more than 32 bits: n * k/2 or a_rows * k/2 >= 2^31 - 4096,
 * m_total >= 2^29 - 1024, ldo > 2^23), HIP.
 */
int moe_grouped_gemm_fp4(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale,
                         int64_t a_rows, const int32_t* a_row_index,
                         const uint8_t* w_q, const uint8_t* w_sf, const float* w_scale,
                         const int32_t* expert_offsets, int32_t num_experts,
                         int64_t m_total, int64_t n, int64_t k,
                         uint16_t* out, int64_t ldo, void* stream);

/*
 * Packed weight-code layout (MOE_FP4 "packed"), the layout
 * moe_grouped_gemm_fp4_packed reads.  Expert weights are constant across
 * calls, so they can be rearranged once, off the critical path, into the order
 * the GEMM's wavefronts load them: every load instruction then reads one
 * contiguous 1 KB and every pipeline stage one contiguous block, instead of 64
 * row segments a row pitch apart.  It permutes the bytes of w_q only (w_sf
 * keeps the row-major layout above) and keeps each expert's size and position:
 *   G  = 512 if k % 512 == 0, else 256   (K elements per granule)
 *   GB = G / 2                           (code bytes of one row per granule)
 *   Rows are taken in groups of 64 (the last group of an expert may hold
 *   16*rg rows, rg = 1..3).  Group q occupies the bytes that rows 64q .. of
 *   the row-major layout occupy, starting at 64*q*(k/2).
 *   Inside group q, granule t, row block j (rows 64q + 16j .. +15) is a block
 *   of 8*G bytes at offset (t*rg + j) * 8*G (rg = 4 for a full group).
 *   Inside a block, the 16-byte piece at offset 16*(((2*s + h)*4 + g)*16 + r)
 *   (s < G/256, h < 2, g < 4, r < 16) holds row 64q + 16j + r, row-major code
 *   bytes t*GB + (GB/4)*g + 32*s + 16*h .. +15.
 */

/*
 * moe_fp4_pack_weights -- rearrange row-major weight codes w_q
 * [num_experts][n][k/2] into the packed layout above (w_packed, same size).
 * moe_fp4_unpack_weights is the inverse.  A pure byte permutation.
 *   src, dst     device, num_experts * n * k/2 bytes each, 16-byte aligned, not
 *                overlapping.
 *   n            >= 1, a multiple of 16; k >= 1, a multiple of 256.
 * Errors: NULL, SHAPE (num_experts < 1, n < 1, k < 1), ALIGN, UNSUPPORTED
 * (n % 16, k % 256, n * k/2 >= 2^31 - 4096), ARG (src and dst overlap), HIP.
 */
int moe_fp4_pack_weights(const uint8_t* w_q, uint8_t* w_packed, int32_t num_experts,
                         int64_t n, int64_t k, void* stream);
int moe_fp4_unpack_weights(const uint8_t* w_packed, uint8_t* w_q, int32_t num_experts,
                           int64_t n, int64_t k, void* stream);

/*
 * moe_grouped_gemm_fp4_packed -- moe_grouped_gemm_fp4 with w_q in the packed
 * layout (written by moe_fp4_pack_weights).  Same arguments, result bits,
 * preconditions and errors; in addition UNSUPPORTED when MOE_FP4_TILE asks
 * for a K step other than the granule G or a width other than 64 columns per
 * wavefront.
 */
int moe_grouped_gemm_fp4_packed(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale,
                                int64_t a_rows, const int32_t* a_row_index,
                                const uint8_t* w_packed, const uint8_t* w_sf,
                                const float* w_scale, const int32_t* expert_offsets,
                                int32_t num_experts, int64_t m_total, int64_t n, int64_t k,
                                uint16_t* out, int64_t ldo, void* stream);

/*
 * moe_grouped_gemm_fp4_finalize -- the grouped GEMM with the Mixture-of-Experts
 * finalize step in its epilogue: every routed row's result, times that row's
 * routing weight, is added into its token's FP32 output row, so the top-k rows
 * of a token (computed by different experts) are summed in token order without
 * writing the per-row BF16 result.  The pages name the epilogue that performs
 * the final output write FINALIZE ("Peering into the CUTLASS Kernel", section
 * "Input Knowledge Required", item 5); this library reads it, for the down
 * projection, as this routing-weighted sum.
 *
 *     out[out_token[r]][j] += row_weight[r] * a_scale * w_scale[e]
 *                             * sum_k A(src(r), k) * W(e, j, k)
 *
 * for every routed row r of expert e (rows [off[e], off[e+1])) and j < n, with
 * A, W, src and the exact FP32-accumulated sum as in moe_grouped_gemm_fp4; the
 * product is rounded to FP32 as fl(fl(acc * fl(a_scale * w_scale[e])) * row_weight[r]).
 * Arguments as moe_grouped_gemm_fp4 (w_packed: 0 = row-major w_q, 1 = the packed
 * layout), plus:
 *   out_token   device, [m_total] int32: destination token of each routed row;
 *               a row whose token is outside [0, num_tokens) adds nothing.
 *   row_weight  device, [m_total] float: routing weight of each routed row.
 *   out         device, [num_tokens][ldo] FP32, accumulated into (+=): zero it for
 *               the plain sum, or pass a residual stream to add onto it.  4-byte
 *               aligned, ldo >= n.  Columns >= n are never touched.
 *   num_tokens  rows of out (>= 1).
 * The additions into one element run concurrently (FP32 atomic adds), so their
 * order, and therefore the last bits of the sum, can differ between runs.  The
 * kernel runs per-wavefront 64-column items (experts of any size; large ones
 * are not given the workgroup tile).
 * Speed: on MI355X the plain GEMM followed by moe_fp4_combine is the faster
 * finalize and the one to use; this entry point is kept as the fused form.
 * Device-wide FP32 atomic adds complete at about 3.2e11 per second however
 * the destinations are spread over the XCDs, so the top-k adds alone take
 * longer than the whole two-pass finalize (down-projection shard: 50 million
 * adds, at least 156 us, against 80 us for GEMM and combine).
 * Errors: as moe_grouped_gemm_fp4, plus NULL (out_token, row_weight), SHAPE
 * (num_tokens < 1), ALIGN (out_token, row_weight, out not 4-byte aligned), ARG
 * (w_packed not 0 or 1), UNSUPPORTED (num_tokens * ldo * 4 >= 2^31 - 4096, or a
 * MOE_FP4_TILE override this epilogue does not run).
 */
int moe_grouped_gemm_fp4_finalize(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale,
                                  int64_t a_rows, const int32_t* a_row_index,
                                  const uint8_t* w_q, const uint8_t* w_sf, const float* w_scale,
                                  int w_packed, const int32_t* expert_offsets,
                                  int32_t num_experts, int64_t m_total, int64_t n, int64_t k,
                                  const int32_t* out_token, const float* row_weight, float* out,
                                  int64_t ldo, int64_t num_tokens, void* stream);

/*
 * moe_grouped_gemm_fp4_swiglu -- the gate+up projection of a Mixture-of-Experts
 * FFN with the activation and the down projection's input quantisation in its
 * epilogue: the grouped GEMM's result is never written; each routed row leaves
 * as the NVFP4 encoding of its SwiGLU activation, ready to be the activations
 * (a_q, a_sf, a_scale = h_scale) of the down projection's grouped GEMM.  The
 * pages allow the final-write epilogue to apply an activation and a
 * quantisation ("Peering into the CUTLASS Kernel", section "Input Knowledge
 * Required", item 5); this library reads that as the gated SiLU between the two
 * projections, followed by this library's NVFP4 recipe at a static scale.
 *
 * The weights have n = 2I rows per expert: rows 0 .. I-1 are the gate, rows
 * I .. 2I-1 the up projection.  For routed row r of expert e and i < I, in FP32:
 *
 *     gate = fl(acc(r, i) * alpha),  up = fl(acc(r, I + i) * alpha)
 *     h    = fl(silu(gate) * up),    silu(x) = x / (1 + e^-x)
 *
 * with acc and alpha = fl(a_scale * w_scale[e]) as in moe_grouped_gemm_fp4 (the
 * value the plain GEMM rounds to BF16), e^-x from the device math library.  Then,
 * per row and block of 16 consecutive intermediate columns, with g = *h_scale:
 *
 *     sf = E4M3_RNE(fl(amax |h| / fl(6 g))),  s = fl(E4M3(sf) * g),
 *     code = E2M1_RNE(fl(h / s))  (0 when s = 0)
 *
 * exactly the steps of moe_fp4_quantize in MOE_FP4_SCALE_STATIC mode.  A single
 * pass cannot know the intermediate's amax before every row is done, so the
 * tensor scale is static: a calibrated value the caller supplies.
 * Arguments as moe_grouped_gemm_fp4_finalize for the GEMM (w_packed: 0 =
 * row-major w_q, 1 = the packed layout), plus:
 *   n        2I, a multiple of 32; with w_packed, I a multiple of 64.
 *   h_scale  device, 1 float: g, positive and finite (not checked).
 *   h_q      device, [m_total][n/4] bytes (I/2 per row, two codes a byte, element
 *            2i in the low nibble), 16-byte aligned; written for every routed row.
 *   h_sf     device, [m_total][n/32] E4M3 block scales, 16-byte aligned.
 * Rows follow the routed order (row r of expert e's range), like out of
 * moe_grouped_gemm_fp4.  Deterministic.  The kernel runs per-wavefront items
 * of 32 intermediate columns (experts of any size).
 * Errors: as moe_grouped_gemm_fp4, plus NULL (h_scale, h_q, h_sf), ALIGN (h_q,
 * h_sf not 16-byte aligned; h_scale not 4-byte aligned), ARG (w_packed not 0 or
 * 1; h_q, h_sf, a_q, a_sf overlapping), UNSUPPORTED (n % 32, or I % 64 with
 * packed weights, or a MOE_FP4_TILE override this epilogue does not run).
 * m_total == 0 is a no-op.
 */
int moe_grouped_gemm_fp4_swiglu(const uint8_t* a_q, const uint8_t* a_sf, const float* a_scale,
                                int64_t a_rows, const int32_t* a_row_index,
                                const uint8_t* w_q, const uint8_t* w_sf, const float* w_scale,
                                int w_packed, const int32_t* expert_offsets, int32_t num_experts,
                                int64_t m_total, int64_t n, int64_t k, const float* h_scale,
                                uint8_t* h_q, uint8_t* h_sf, void* stream);

/* Output element types of moe_fp4_combine. */
enum { MOE_FP4_OUT_BF16 = 0, MOE_FP4_OUT_FP32 = 1 };

/*
 * moe_fp4_combine -- the Mixture-of-Experts finalize step as a pass of its own:
 * each token's output row is the routing-weighted sum of its top-k routed rows
 * of the grouped GEMM's BF16 output (the final output write, "Peering into the
 * CUTLASS Kernel", section "Input Knowledge Required", item 5, read as in
 * moe_grouped_gemm_fp4_finalize).  For token t and column j < n:
 *
 *     acc = 0;  for s = 0 .. topk-1 with 0 <= r = token_rows[t][s] < m_total:
 *                   acc = fl(acc + fl(token_weights[t][s] * rows[r][j]))
 *     out[t][j] = round(residual ? fl(residual[t][j] + acc) : acc)
 *
 * in FP32, slots in order, rounded to BF16 (nearest even) or written as FP32.
 * Deterministic: the same inputs give the same bits.  Unlike the finalize
 * epilogue it needs the GEMM's per-row output, but it reads it with plain
 * coalesced loads in one pass, where the epilogue adds every element with a
 * device-wide atomic; on MI355X this pass plus the plain GEMM is the faster way.
 *   rows          device, [m_total][ld_rows] BF16 (moe_grouped_gemm_fp4's out),
 *                 16-byte aligned, ld_rows >= n and a multiple of 8.
 *   token_rows    device, [num_tokens][topk] int32: the routed rows of each token,
 *                 in summation order; an entry outside [0, m_total) is skipped.
 *   token_weights device, [num_tokens][topk] float.
 *   residual      device, [num_tokens][ld_res] FP32 added to the sum, or NULL;
 *                 16-byte aligned, ld_res >= n and a multiple of 4.  out may be the
 *                 same buffer (FP32 output, ldo == ld_res).
 *   out           device, [num_tokens][ldo] of out_dtype, 16-byte aligned, ldo >= n,
 *                 ldo a multiple of 8 (BF16) or 4 (FP32).  Columns >= n untouched.
 *   n             a multiple of 16 (UNSUPPORTED otherwise).
 * Errors: NULL, SHAPE (m_total < 0, num_tokens < 0, topk < 1, n < 1, ld_rows / ldo /
 * ld_res < n), ALIGN, ARG (out_dtype), UNSUPPORTED (n % 16, any of the three
 * buffers 2^31 - 4096 bytes or larger), HIP.  num_tokens == 0 is a no-op.
 */
int moe_fp4_combine(const uint16_t* rows, int64_t ld_rows, int64_t m_total,
                    const int32_t* token_rows, const float* token_weights, int32_t topk,
                    int64_t num_tokens, int64_t n, const float* residual, int64_t ld_res,
                    void* out, int out_dtype, int64_t ldo, void* stream);

/*
 * moe_grouped_gemm_fp4_workspace_size -- device workspace bytes the grouped GEMM
 * entry points need for these sizes.  Always 0: every kernel builds its work
 * list of (expert, M-tile, N-tile) items in LDS from the device offsets, at the
 * start of each workgroup, so no entry point takes a workspace argument and the
 * library never allocates.  Kept so that a caller written against a
 * workspace-taking grouped GEMM can size its buffer the usual way; what passes
 * validation launches without one ("Peering into the CUTLASS SharedStorage",
 * section "Why This Message Was Written": a configuration the size check
 * accepted failed later at initialisation; here there is nothing to fail).
 * Host only; no GPU call; the arguments are not validated.
 */
size_t moe_grouped_gemm_fp4_workspace_size(int32_t num_experts, int64_t m_total, int64_t n,
                                           int64_t k);

/* Kernel configuration the GEMM picks for a problem (host-only, no GPU call). */
typedef struct {
  int32_t tile_m;          /* rows of one expert per work item                       */
  int32_t tile_n;          /* output columns per work item                           */
  int32_t k_step;          /* K elements per main-loop iteration                     */
  int32_t waves_per_group; /* wavefronts (64 lanes) per workgroup                    */
  int64_t lds_bytes;       /* LDS per workgroup                                      */
} moe_fp4_gemm_plan;

/*
 * moe_grouped_gemm_fp4_plan -- the configuration moe_grouped_gemm_fp4 would use
 * for these sizes (m_total / num_experts rows per expert on average).
 * Returns MOE_FP4_OK, or NULL / SHAPE / UNSUPPORTED as the GEMM would.
 * The MOE_FP4_TILE environment variable ("MxN", e.g. "32x64") overrides the
 * choice of tile_m x tile_n when it names a supported tile: per-wave items
 * "16x64", "32x64", "64x64", "16x32", "32x32", "64x32" (optionally "xK" with K
 * 256, 512 or 1024 elements per stage, and "r" to keep the weight scales in
 * registers); workgroup items "128x128", "256x256" (experts of 96 rows or more;
 * per-wave items for the rest), "256x256!" (every expert), "256x256f8" and
 * "256x256f8!" (the same with K split by scale block on the FP8 MFMA),
 * "48x512" (every expert), and the splits by expert size "256x256m" (256 x 256
 * from 96 rows, 48 x 512 below: the default when experts average 96 rows or
 * more and K is a multiple of 512), "48x512p" (48 x 512 from 17 rows, per-wave
 * items below) and "256x256mp" (all three).  The 48 x 512 items need K to be a
 * multiple of 512; asked for otherwise, the default choice stands.
 */
int moe_grouped_gemm_fp4_plan(int32_t num_experts, int64_t m_total, int64_t n, int64_t k,
                              moe_fp4_gemm_plan* plan);

/*
 * moe_fp4_stage_bytes -- bytes one pipeline stage of a bm x bn x bk tile moves
 * into on-chip memory: packed FP4 for both operands plus their E4M3 block
 * scales, (bm + bn) * bk * (1/2 + 1/16).  This is the per-stage transaction
 * count of the block-scaled mainloop printed on "Peering into the CUTLASS
 * SharedStorage" (section "The Message": bytes of the A tile and its scales
 * plus bytes of the B tile and its scales).  Returns -1 unless bm, bn >= 1 and
 * bk is a positive multiple of 16.
 */
int64_t moe_fp4_stage_bytes(int64_t bm, int64_t bn, int64_t bk);

/* Human-readable name of a status code (never NULL). */
const char* moe_fp4_status_string(int status);

/* ABI version: bumped whenever a signature or a layout above changes. */
int moe_fp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP4_H */
