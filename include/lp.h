/*
 * lp.h - backward pass of block-scaled low-precision linear and grouped
 * (per-expert) matmuls on AMD Instinct MI355X (gfx950).
 *
 * The saved forward operands are block-scaled low-precision tensors; the
 * backward dequantizes them to bf16 and computes, in bf16 x bf16 -> fp32
 * contractions:
 *
 *     grad_X = grad_out @ W          [M,N] x [N,K] -> [M,K]
 *     grad_W = grad_out^T @ X        [N,M] x [M,K] -> [N,K]
 *
 * ("Add Autograd Backward Support for FP4 GEMM Custom Ops", Implementation
 * Method: dequantize-then-compute in BF16; "Train adapters on top of FP8
 * weights", FP8LinearFunction.backward and FP8GroupedMatmulFunction.backward;
 * "perf: defer mxfp8 backward quantization", MXFP8GMMFunction.op_dx.)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer to tensor data is a DEVICE pointer.  The caller allocates
 *   and owns every buffer; the library calls no device allocator, frees
 *   nothing and keeps no pointer after a call returns.  Between calls it
 *   keeps only facts it looks up once per device (the compute-unit count,
 *   the address of lp_linear_bwd_noalloc's workspace array), and it is safe
 *   to call from several host threads.
 * - Work is enqueued on `stream` (a hipStream_t; NULL is the default
 *   stream) and runs asynchronously.  The status covers argument checking
 *   and the launch only.  Argument errors (LP_ERR_NULL, LP_ERR_SHAPE,
 *   LP_ERR_FORMAT, LP_ERR_ALIGN) are found before anything is enqueued:
 *   nothing runs and no output is written.  LP_ERR_HIP reports a launch
 *   that failed; launches of the same call made before it may already be
 *   enqueued.
 * - Tensors are dense and row-major.  Element (b, r, c) of a [batch][rows][cols]
 *   tensor is at offset (b*rows + r)*cols + c, in units of elements.
 * - Codes, scales and outputs must be 16-byte aligned; a tensor scale
 *   4-byte aligned.  A pointer may be NULL only when its tensor is empty.
 * - A tensor holds fewer than 2^34 elements and each of batch, rows, cols is
 *   below 2^31 (LP_ERR_SHAPE otherwise).
 * - In the products (lp_linear_bwd*, lp_grouped_bwd, lp_*_fwd) the token
 *   count M is below 2^30 and every other dimension (N, K) below 2^22
 *   (LP_ERR_SHAPE otherwise).
 * - The output of a product must have few enough tiles to count in 32 bits:
 *   R * (cols/128 + 1) <= 2^30 (LP_ERR_SHAPE otherwise), with R =
 *   rows/128 + G + 1 for grad_X and the forward (rows: tokens) and
 *   R = G * (N/128 + 1) for grad_W, G being the number of groups (1 for
 *   the dense calls).
 *
 * Formats (lp_fmt)
 * ----------------
 *   LP_BF16      bf16 values, 2 bytes each.  No scales.
 *   LP_MXFP4     E2M1 codes packed two per byte along cols (element 2j in
 *                the low nibble, 2j+1 in the high nibble), one E8M0 scale
 *                byte per 32 elements along cols: scales[batch][rows][cols/32].
 *   LP_NVFP4     E2M1 codes packed as LP_MXFP4; one E4M3 scale byte per 16
 *                along cols: scales[batch][rows][cols/16]; plus one fp32
 *                tensor scale (a decode multiplier, read from device memory).
 *   LP_FP8_B128  E4M3 codes, one byte each; fp32 inverse scales (decode
 *                multipliers) per 128x128 block:
 *                scales[batch][ceil(rows/128)][ceil(cols/128)], blocks cut at
 *                the tensor edge ("Train adapters on top of FP8 weights",
 *                _dequantize_fp8_weight).
 *   LP_MXFP8     E4M3 codes, one byte each; one E8M0 scale byte per 32
 *                elements along `scale_axis`: -1 -> scales[batch][rows][cols/32],
 *                -2 -> scales[batch][rows/32][cols] ("perf: defer mxfp8
 *                backward quantization", npu_dynamic_mx_quant axis argument
 *                and group_sizes [1, 1, 32]).
 *
 * *   LP_FP8T_E4M3 E4M3 codes, one byte each, with ONE fp32 scale for the
 *                whole tensor (tensor_scale: the decode multiplier, which is
 *                the quantization step); no block scales (`scales` and
 *                `scale_axis` are ignored).
 *   LP_FP8T_E5M2 E5M2 codes, one byte each, one fp32 tensor scale likewise.
 *                ("AstrAI fp8.py": per-tensor scaled FP8, E4M3 for the
 *                forward operands and E5M2 for gradients.)
 *
 * Element values: E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit:
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6), E4M3 (bias 7, max 448, no infinities,
 * S.1111.111 = NaN), E5M2 (bias 15, max 57344, S.11111.00 = infinity,
 * S.11111.01..11 = NaN), E8M0 (2^(byte-127), 0xFF = NaN).
 *
 * Decoded value: bf16_rne(fp32_rne(code_value * S)) where S is the fp32
 * block multiplier (NVFP4: S = fp32_rne(E4M3(block byte) * tensor_scale);
 * LP_FP8T_*: S = tensor_scale).
 * A NaN result is 0x7FC0 carrying the code's sign bit.
 */
#ifndef LP_H
#define LP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LP_OK = 0,
  LP_ERR_NULL = 1,    /* a required pointer is NULL                              */
  LP_ERR_SHAPE = 2,   /* negative size, operand sizes disagree, or a block or
                         packing divisibility rule is broken                    */
  LP_ERR_FORMAT = 3,  /* a format / scale-axis combination this call does not
                         support                                                */
  LP_ERR_ALIGN = 4,   /* a pointer breaks the alignment rule                     */
  LP_ERR_HIP = 5      /* the HIP runtime reported an error at launch             */
} lp_status;

typedef enum {
  LP_BF16 = 0,
  LP_MXFP4 = 1,
  LP_NVFP4 = 2,
  LP_FP8_B128 = 3,
  LP_MXFP8 = 4,
  LP_FP8T_E4M3 = 5,
  LP_FP8T_E5M2 = 6
} lp_fmt;

/* A (possibly block-scaled) tensor of logical shape [batch][rows][cols]. */
typedef struct {
  int32_t fmt;               /* lp_fmt                                          */
  int32_t scale_axis;        /* -1: scale blocks run along cols; -2: along rows
                                (LP_MXFP8 only; ignored for LP_BF16)            */
  int64_t batch;             /* groups for a grouped weight, else 1             */
  int64_t rows;
  int64_t cols;              /* logical elements (not packed bytes)             */
  const void* codes;         /* device pointer, layout per format above          */
  const void* scales;        /* device pointer, NULL for LP_BF16                 */
  const float* tensor_scale; /* device pointer to one fp32, LP_NVFP4 and
                                LP_FP8T_* only                                  */
} lp_qtensor;

/*
 * lp_dequant - decode a block-scaled tensor to bf16.
 *
 * Cites: "Add Autograd Backward Support for FP4 GEMM Custom Ops" (the backward
 * dequantizes the saved packed FP4 inputs to BF16); "Train adapters on top of
 * FP8 weights", _dequantize_fp8_weight (E4M3 times its 128x128-block inverse
 * scale).
 *
 * src       any format except LP_BF16.  Divisibility: cols % 32 == 0 for
 *           LP_MXFP4 and for LP_MXFP8 with scale_axis -1; rows % 32 == 0 and
 *           cols % 16 == 0 for LP_MXFP8 with scale_axis -2; cols % 16 == 0 for
 *           LP_NVFP4, LP_FP8_B128 and LP_FP8T_* (rows arbitrary; partial
 *           128-blocks are cut at the edge).
 * dst_bf16  device bf16 output [batch][rows][cols].
 * Result is bit-exact: the rule in the header comment above.
 */
lp_status lp_dequant(const lp_qtensor* src, void* dst_bf16, void* stream);

/*
 * lp_mx_quant - dynamic MX quantization of a bf16 tensor along one axis.
 *
 * Cites: "perf: defer mxfp8 backward quantization", MXFP8GMMFunction.op_dx and
 * MXFP8MatMul.backward (npu_dynamic_mx_quant of the gradient along -1 and of
 * the weight along its reduction axis; E8M0 scale per 32).
 *
 * src_bf16    device bf16 [batch][rows][cols].
 * axis        -1: blocks of 32 along cols (cols % 32 == 0);
 *             -2: blocks of 32 along rows (rows % 32 == 0, cols % 8 == 0).
 * dst_fmt     LP_MXFP8 (E4M3 elements) or LP_MXFP4 (E2M1, packed along cols;
 *             cols must be even).
 * dst_codes   device [batch][rows][cols] bytes (LP_MXFP8) or [batch][rows][cols/2].
 * dst_scales  device E8M0 bytes [batch][rows][cols/32] (axis -1) or
 *             [batch][rows/32][cols] (axis -2).
 * Per block: amax = max |v|; e = floor(log2 amax) - emax (8 for E4M3, 2 for
 * E2M1) clamped to [-127, 127]; scale byte = e + 127; each element is
 * v * 2^-e rounded to nearest (ties to even) on the element grid, saturated
 * to +-448 / +-6, sign kept.  A block holding a NaN or an infinity gets
 * scale 0xFF and NaN codes (E4M3 0x7F | sign; E2M1 codes 0); an all-zero
 * block gets scale 0 and signed-zero codes.  Bit-exact.
 */
lp_status lp_mx_quant(const void* src_bf16, int64_t batch, int64_t rows, int64_t cols,
                      int32_t axis, int32_t dst_fmt, void* dst_codes, void* dst_scales,
                      void* stream);

/*
 * lp_mx_quant_dual - dynamic MX quantization along both axes at once.
 *
 * Cites: "perf: defer mxfp8 backward quantization", MXFP8MatMul.backward
 * (npu_dynamic_mx_quant_with_dual_axis of the gradient: one copy scaled
 * along -1 for grad_X, one along -2 for grad_W).
 *
 * src_bf16     device bf16 [batch][rows][cols]; rows % 32 == 0, cols % 32 == 0.
 * dst_fmt      LP_MXFP8 or LP_MXFP4.
 * codes_cols, scales_cols   the copy with blocks along cols: exactly what
 *              lp_mx_quant(src, ..., axis -1, ...) writes.
 * codes_rows, scales_rows   the copy with blocks along rows: exactly what
 *              lp_mx_quant(src, ..., axis -2, ...) writes.
 * One read of src.  Bit-exact, with the rules of lp_mx_quant.
 */
lp_status lp_mx_quant_dual(const void* src_bf16, int64_t batch, int64_t rows, int64_t cols, int32_t dst_fmt,
                           void* codes_cols, void* scales_cols, void* codes_rows, void* scales_rows,
                           void* stream);

/*
 * lp_tensor_amax - amax of a bf16 tensor.
 *
 * Cites: "AstrAI fp8.py" (each quantization records the amax of its tensor,
 * max |x| over every element, into an amax history).
 *
 * src_bf16  device bf16, n elements; n % 8 == 0 and n < 2^34.
 * amax      device fp32: max |x| (exact), 0 when n == 0, NaN when any
 *           element is NaN.  It may point into an amax history ring.
 */
lp_status lp_tensor_amax(const void* src_bf16, int64_t n, float* amax, void* stream);

/*
 * lp_tensor_quant - per-tensor FP8 quantization of a bf16 tensor, recording
 * its amax in the same pass.
 *
 * Cites: "AstrAI fp8.py" (codes are the FP8 cast of x / scale with one scale
 * per tensor; FP8_MAX is 448 for E4M3 and 57344 for E5M2; the backward
 * quantizes the gradient once and returns its amax for the history).
 *
 * src_bf16   device bf16, n elements; n % 8 == 0 and n < 2^34.
 * dst_fmt    LP_FP8T_E4M3 or LP_FP8T_E5M2.
 * scale      device fp32: the quantization step (the decode multiplier of
 *            the result), e.g. written by lp_scale_from_history.
 * dst_codes  device bytes [n], 16-byte aligned.
 * amax       device fp32, or NULL: receives the input's amax as
 *            lp_tensor_amax computes it.  Must not be `scale`
 *            (LP_ERR_SHAPE).
 * Each code: t = x / scale in fp32 (IEEE division, nearest even); |t| above
 * FP8_MAX, infinity included, saturates to FP8_MAX with t's sign; otherwise
 * the nearest FP8 value, ties to the even code; NaN becomes 0x7F with x's
 * sign bit.  Bit-exact.
 */
lp_status lp_tensor_quant(const void* src_bf16, int64_t n, int32_t dst_fmt, const float* scale,
                          void* dst_codes, float* amax, void* stream);

/*
 * lp_scale_from_history - per-tensor scale from an amax history.
 *
 * Cites: "AstrAI fp8.py" (scale = (amax / FP8_MAX) / 2^margin, at least
 * 1e-12; delayed scaling takes the largest amax of the history ring,
 * dynamic scaling the current amax).
 *
 * history  device fp32 [len], 1 <= len <= 65536.  A history of one entry,
 *          the current amax, is dynamic scaling.
 * fmt      LP_FP8T_E4M3 (FP8_MAX 448) or LP_FP8T_E5M2 (FP8_MAX 57344).
 * margin   -64 <= margin <= 64.
 * scale    device fp32: s = fp32(max(history) / FP8_MAX), then
 *          fp32(s / 2^margin), raised to fp32(1e-12) when below it; NaN when
 *          any entry is NaN.
 */
lp_status lp_scale_from_history(const float* history, int32_t len, int32_t fmt, int32_t margin, float* scale,
                                void* stream);

/*
 * lp_tensor_quant_delayed - one delayed-scaling quantization step: the
 * scale from an amax history, quantization with it, and the input's amax
 * recorded into the history.
 *
 * Cites: "AstrAI fp8.py" (DelayedScaling: the scale of a step comes from the
 * largest amax of the ring; the step's amax is then recorded at the ring's
 * index; _LinearFp8.backward quantizes the gradient this way).
 *
 * src_bf16, n, dst_fmt, dst_codes: as lp_tensor_quant.
 * history  device fp32 [len], 1 <= len <= 65536; slot: 0 <= slot < len (the
 *          caller's ring index); margin: as lp_scale_from_history.
 * scale    device fp32, outside history: receives the step's scale.
 * Results are bit-identical to lp_scale_from_history(history, len, ...,
 * scale) followed by lp_tensor_quant(src, ..., scale, codes, history + slot):
 * the scale sees history[slot] before it is overwritten.  Two launches.
 */
lp_status lp_tensor_quant_delayed(const void* src_bf16, int64_t n, int32_t dst_fmt, float* history, int32_t len,
                                  int32_t slot, int32_t margin, void* dst_codes, float* scale, void* stream);

/*
 * lp_linear_bwd - backward of a linear layer y = x @ W^T with saved
 * block-scaled operands.
 *
 * Cites: "Add Autograd Backward Support for FP4 GEMM Custom Ops",
 * Implementation Method (grad_X = grad_output @ W_bf16, grad_W =
 * grad_output.T @ X_bf16); "Train adapters on top of FP8 weights",
 * FP8LinearFunction.backward (frozen weight: grad_X only); "AstrAI fp8.py",
 * _LinearFp8.backward (each output is computed only when it is needed).
 *
 * grad_out  [M][N]: LP_BF16; or LP_MXFP8 with scale_axis -1 (its scales run
 *           along the dX contraction; needs grad_w == NULL); or LP_MXFP8 with
 *           scale_axis -2 (along the dW contraction; needs grad_x == NULL and x
 *           LP_MXFP8 with scale_axis -2), as produced by lp_mx_quant_dual.
 *           ("perf: defer mxfp8 backward quantization", MXFP8MatMul.backward:
 *           the gradient is quantized along both axes, one copy per product.)
 *           Or LP_FP8T_E4M3 / LP_FP8T_E5M2, one copy for both products, with
 *           x and w LP_FP8T_* too ("AstrAI fp8.py", _LinearFp8.backward):
 *           per-tensor scaled operands pair only with each other.
 * x         [M][K] saved input, or NULL when grad_w == NULL.
 * w         [N][K] saved weight, or NULL when grad_x == NULL.
 *           x and w: LP_BF16, LP_MXFP4, LP_NVFP4 (scale_axis -1), LP_FP8_B128,
 *           or LP_MXFP8 (scale_axis -1 or -2) with a bf16 or MXFP8 grad_out;
 *           LP_FP8T_* with an LP_FP8T_* grad_out.
 * grad_x    device bf16 [M][K], or NULL to skip grad_X.
 * grad_w    device bf16 [N][K], or NULL to skip grad_W.
 * Sizes: M >= 0 arbitrary; N % 16 == 0, K % 16 == 0, plus each operand's
 * block rule (K % 32 for FP4 and MX along K; N % 32 for MXFP8 grad_out and
 * for MXFP8 w with scale_axis -2; M % 32 for MXFP8 x with scale_axis -2).
 * Accumulation is fp32; outputs are rounded to bf16 (nearest even).
 * When both operands of a product are MXFP8 with their scales along its
 * contraction (dX: grad_out -1, w -2; dW: grad_out -2, x -2), the product
 * runs on the block-scaled FP8 MFMA: each code product times its two E8M0
 * scales is exact, so the result equals the decode-then-bf16 route up to
 * fp32 summation order.  Per-tensor scaled operands run on the same MFMA
 * with unit block scales: the fp32 sum of exact code products is multiplied
 * by fp32(scale_grad * scale_other), then rounded to bf16.
 * A quantized x or w is decoded inside the contraction, once per output
 * tile that reads it.  Decoding it beforehand with lp_dequant and passing
 * the bf16 copy (fmt LP_BF16) gives bit-identical outputs; when many output
 * tiles share the operand (grad_X of many tokens against one weight) that
 * is faster, at the cost of the copy's memory.
 */
lp_status lp_linear_bwd(const lp_qtensor* grad_out, const lp_qtensor* x, const lp_qtensor* w,
                        void* grad_x, void* grad_w, void* stream);

/*
 * lp_linear_bwd_workspace - workspace bytes that lp_linear_bwd_ws can use to
 * split the contraction of this call across workgroups.
 *
 * Arguments as for lp_linear_bwd; grad_x and grad_w only say which outputs
 * are wanted (non-NULL) and are not dereferenced.  *bytes is 0 when the
 * call does not split (its 256 x 256 output tiles already fill the GPU, or
 * its contraction is short); otherwise it is the size of a workspace that
 * lets lp_linear_bwd_ws split it.  Checks and errors as for lp_linear_bwd.
 */
lp_status lp_linear_bwd_workspace(const lp_qtensor* grad_out, const lp_qtensor* x, const lp_qtensor* w,
                                  const void* grad_x, const void* grad_w, size_t* bytes);

/*
 * lp_linear_bwd_ws - lp_linear_bwd with a caller-owned workspace.
 *
 * Cites: as lp_linear_bwd (same operation, same results up to fp32
 * summation order).
 *
 * When a contraction has fewer 256 x 256 output tiles than the GPU has
 * compute units, the library splits its contraction over several
 * workgroups per tile: each writes an fp32 partial tile into the workspace,
 * and the last to finish sums the partials in a fixed order and writes the
 * bf16 output.  The result does not depend on which workgroup finishes
 * last.
 *
 * workspace        device memory, 256-byte aligned, or NULL (no splitting).
 * workspace_bytes  its size; if smaller than lp_linear_bwd_workspace
 *                  reports, the call does not split (still correct).
 * The workspace must be zero-filled before its first use; every completed
 * call leaves the part that must start at zero (per-tile counters) zero
 * again.  Two calls that may run at the same time (other streams, other
 * threads) must not share a workspace.  Other arguments, rules and errors
 * as for lp_linear_bwd; LP_ERR_ALIGN for a misaligned workspace.
 */
lp_status lp_linear_bwd_ws(const lp_qtensor* grad_out, const lp_qtensor* x, const lp_qtensor* w,
                           void* grad_x, void* grad_w, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * lp_linear_bwd_noalloc - lp_linear_bwd_ws for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).
 *
 * Same operation, arguments, results and errors as lp_linear_bwd_ws, with the
 * workspace taken from a device array inside the library instead of from the
 * caller: 64 MiB + 4 KiB per GPU, set aside when the library is loaded and
 * held until the process ends.  Every contraction that splits fits in it (a
 * split plan uses at most 256 partial tiles of 256 x 256 fp32); the call
 * returns LP_ERR_SHAPE if a plan ever needed more.  The call itself allocates
 * nothing: no hipMalloc, no hipFree, no allocating library routine.  The
 * array's address on the current device is looked up once (the first call on
 * that device); LP_ERR_HIP if that lookup fails.  Each call first clears the
 * array's per-tile counters with a small kernel on `stream` (no memset, so it
 * can be captured).
 *
 * All calls on one GPU share the array, which keeps the last call's partial
 * tiles: calls that may run at the same time on one GPU (other streams,
 * other threads) race and must be serialized by the caller.  `stream` must
 * belong to the current device.
 */
lp_status lp_linear_bwd_noalloc(const lp_qtensor* grad_out, const lp_qtensor* x, const lp_qtensor* w,
                                void* grad_x, void* grad_w, void* stream);

/*
 * lp_grouped_bwd - backward of a grouped (per-expert) matmul.
 *
 * Cites: "Train adapters on top of FP8 weights", FP8GroupedMatmulFunction.
 * backward ((S, output_dim) @ grouped (num_experts, output_dim, input_dim)
 * -> (S, input_dim)) and FP8GroupedLinear.forward (int32 cumulative end
 * offsets); the EP-sentinel comment of fp8_grouped_mm_experts_forward (rows
 * past offsets[G-1] are skipped and left unwritten); "perf: defer mxfp8
 * backward quantization", MXFP8GMMFunction.op_dx.
 *
 * offsets   device int32 [groups], cumulative END row of each group; group g
 *           owns rows [offsets[g-1], offsets[g]) with offsets[-1] = 0.  The
 *           caller guarantees 0 <= offsets[0] <= ... <= offsets[G-1] <= M.  The
 *           kernels use end_g = clamp(offsets[g], end_{g-1}, M) (end_{-1} = 0),
 *           which equals offsets[g] for a valid array and keeps a bad one from
 *           making them read or write out of bounds.  Offsets are never read
 *           on the host (no synchronisation).
 * grad_out  [M][N] as for lp_linear_bwd.
 * x         [M][K] (rows grouped like grad_out), or NULL when grad_w == NULL.
 * w         [groups][N][K] (batch == groups), or NULL when grad_x == NULL.
 * grad_x    device bf16 [M][K] or NULL.  Rows at or past offsets[G-1] are NOT
 *           written.
 * grad_w    device bf16 [groups][N][K] or NULL.  An empty group's slice is
 *           written with zeros (the empty sum).
 * Size and format rules as for lp_linear_bwd, except that grad_out scaled
 * along its rows (-2) is not accepted (its 32-row blocks would straddle
 * groups); 1 <= groups <= 1024.
 */
lp_status lp_grouped_bwd(const lp_qtensor* grad_out, const lp_qtensor* x, const lp_qtensor* w,
                         const int32_t* offsets, int64_t groups, void* grad_x, void* grad_w,
                         void* stream);

/*
 * lp_grouped_dx_deferred - grad_X of a grouped layer in the deferred MXFP8
 * recipe, with the bf16 weight quantized as part of the call.
 *
 * Cites: "perf: defer mxfp8 backward quantization", MXFP8GMMFunction.op_dx
 * (the weight is quantized in the backward along its reduction axis, one
 * E8M0 scale per 32, and contracted with the MXFP8 gradient; the page trades
 * this backward compute for saved memory).
 *
 * Computes exactly what lp_mx_quant(w, axis -2, LP_MXFP8) followed by
 * lp_grouped_bwd(grad_out, NULL, that weight, offsets, groups, grad_x, NULL)
 * computes, bit for bit.  A group of at most fuse_rows rows quantizes its
 * weight slices inside the product, which then reads the bf16 weight once
 * and never writes its quantized copy; the weights of larger groups are
 * quantized first into w_codes / w_scales, then contracted.
 *
 * grad_out   LP_MXFP8 with scales along -1, [M][N] (N % 32 == 0).
 * w          device bf16 [groups][N][K] (K % 16 == 0), 16-byte aligned.
 * offsets    device int32 [groups], cumulative end rows, as for
 *            lp_grouped_bwd (the group sizes that fuse_rows is compared with
 *            are taken from it on the device, with its clamping).
 * fuse_rows  >= 0; 0 quantizes every weight first, >= M none.  Weights are
 *            quantized inside the product only when N % 512 == 0 (the
 *            kernel reads the gradient's scale rows in 16-byte pieces) and
 *            K % 32 == 0; otherwise every weight is quantized first.
 * grad_x     device bf16 [M][K]; rows at or past offsets[groups-1] are not
 *            written.
 * w_codes    device u8 [groups][N][K] and w_scales u8 [groups][N/32][K]:
 * w_scales   caller-owned, written for the groups whose weight is quantized
 *            first (the others' slices are left as they are); may be NULL
 *            when fuse_rows >= M, N % 512 == 0 and K % 32 == 0.
 * Errors: LP_ERR_FORMAT unless grad_out is MXFP8 along -1; LP_ERR_SHAPE for
 * sizes outside the rules (groups 1..1024, fuse_rows < 0, K % 16, the size
 * limits of lp_grouped_bwd); LP_ERR_NULL / LP_ERR_ALIGN as usual; checked
 * before anything is enqueued.  LP_ERR_HIP: a launch failed (earlier
 * launches of the call may already be enqueued).
 */
lp_status lp_grouped_dx_deferred(const lp_qtensor* grad_out, const void* w, int64_t K, const int32_t* offsets,
                                 int64_t groups, int64_t fuse_rows, void* grad_x, void* w_codes, void* w_scales,
                                 void* stream);

/*
 * lp_linear_fwd - forward of a linear layer y = x @ W^T with quantized (or
 * bf16) operands.
 *
 * Cites: "Add Autograd Backward Support for FP4 GEMM Custom Ops" (the forward
 * ops that the backward pairs with multiply FP4 inputs by FP4 weights into
 * BF16); "perf: defer mxfp8 backward quantization", MXFP8MatMul.forward (x
 * quantized along its last axis, the weight along its reduction axis, one
 * E8M0 scale per 32); "Train adapters on top of FP8 weights",
 * FP8LinearFunction.forward (a bf16 input times an E4M3 weight with fp32
 * inverse scales per 128 x 128 block).
 *
 * x  [M][K], w [N][K], one of:
 *    - both LP_MXFP4 or both LP_MXFP8, scale_axis -1 (blocks of 32 along K);
 *      K % 128 == 0 (LP_MXFP4) or K % 64 == 0 (LP_MXFP8);
 *    - both LP_NVFP4 (E4M3 scales per 16 along K, each its own tensor
 *      scale); K % 32 == 0;
 *    - x LP_BF16 and w LP_BF16 or LP_FP8_B128 (K % 16 == 0) or LP_NVFP4
 *      (scale_axis -1, K % 32 == 0): an NVFP4 x decoded first with
 *      lp_dequant, which saves the per-tile decode of x.
 *    N % 16 == 0; M >= 0 arbitrary.
 * y  device bf16 [M][N].
 * MX operands: y[m][n] = sum_k dec(x)[m][k] * dec(w)[n][k] on the
 * block-scaled MFMA: each product code_x * code_w * 2^(sx + sw) is exact,
 * the sum is fp32, the result is rounded to bf16 (nearest even).
 * NVFP4 and block-FP8 operands are decoded to bf16 inside the contraction,
 * exactly as lp_dequant decodes them (so a NaN code or scale gives NaN
 * outputs in its row or column), then contracted on the bf16 MFMA with fp32
 * sums; decoding them first with lp_dequant and passing the bf16 copies
 * gives bit-identical results.
 * LP_ERR_FORMAT for other format combinations.
 */
lp_status lp_linear_fwd(const lp_qtensor* x, const lp_qtensor* w, void* y, void* stream);

/*
 * lp_grouped_fwd - forward of a grouped (per-expert) matmul.
 *
 * Cites: "Add Autograd Backward Support for FP4 GEMM Custom Ops" (grouped FP4
 * forward); "Train adapters on top of FP8 weights", FP8GroupedLinear.forward
 * and FP8GroupedMatmulFunction.forward (the kernel's grouped_matmul of a
 * bf16 input with block-FP8 expert weights over int32 cumulative end
 * offsets); the EP-sentinel comment of fp8_grouped_mm_experts_forward (rows
 * past the last offset are not written).
 *
 * x        [M][K] rows grouped by offsets; w [groups][N][K]; formats and sizes
 *          as lp_linear_fwd.  offsets as lp_grouped_bwd (read on the device,
 *          clamped the same way); 1 <= groups <= 1024.
 * y        device bf16 [M][N]: rows of group g are x[rows] @ w[g]^T; rows at or
 *          past offsets[G-1] are NOT written.
 */
lp_status lp_grouped_fwd(const lp_qtensor* x, const lp_qtensor* w, const int32_t* offsets, int64_t groups,
                         void* y, void* stream);

/* A static, human-readable name for a status code. */
const char* lp_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* LP_H */
