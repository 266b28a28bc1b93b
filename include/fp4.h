/*
 * fp4.h -- C ABI of the block-scaled FP4 (E2M1) library for AMD Instinct
 * MI355X (gfx950): quantize, dequantize and the W4A4 block-scaled GEMM.
 *
 * Formats (Ultralytics glossary page "FP4", section "Como funciona FP4"):
 *   E2M1 element: 1 sign, 2 exponent, 1 mantissa bit; magnitudes
 *                 {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *   MXFP4: 32 consecutive values share one 8-bit power-of-two scale (E8M0).
 *   NVFP4: 16 consecutive values share one FP8 E4M3 scale, under a second
 *          FP32 per-tensor scale.
 * Options (Hugging Face transformers page "Four Over Six", introduction):
 *   adaptive 4-or-6 block scaling for NVFP4, random Hadamard transform,
 *   2D block scaling, transposed inputs, stochastic rounding.
 *
 * Conventions common to every entry point
 *   - Every buffer pointer is a DEVICE pointer owned by the caller. The library
 *     never allocates, frees, or keeps a pointer after the call returns, and
 *     never writes its inputs.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and runs asynchronously; nothing synchronises the host.
 *   - Arguments are validated on the host before any HIP call. A call that
 *     returns anything but FP4_OK has enqueued nothing and written nothing.
 *   - A batch, row or column count of zero is a valid empty call: FP4_OK,
 *     nothing enqueued.
 *   - Non-finite inputs give unspecified (but in-bounds) outputs.
 *   - Calls that share an output buffer or workspace on one stream are
 *     ordered; on different streams they race, as with any HIP kernel.
 *
 * Packed layout
 *   codes:  [R, C/2] bytes, row stride ld_codes; element 2j of a row in bits
 *           3:0 of byte j, element 2j+1 in bits 7:4. Bit 3 of a code is the
 *           sign, bits 2:0 index the magnitude list above.
 *   scales: [R, C/blk] bytes, row stride ld_scales (blk = 32 MXFP4, 16 NVFP4).
 *           MXFP4: byte = e + 127 where the block's scale is 2^e.
 *           NVFP4: byte = E4M3 code (OCP "fn": bias 7, max 448).
 *           Under FP4_BLOCK2D each 16x16 tile's byte is stored on each of the
 *           tile's 16 rows, so dequantize and GEMM read the 1 x 16 layout.
 *   tensor_scale (NVFP4): one fp32 per batch item, S_t. The dequantized value
 *           of code c in a block with scale byte s is val(c) * (E4M3(s) * S_t).
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4_OK = 0,
  FP4_ERR_INVALID = -1,     /* null pointer, negative size, stride too small, bad opts->size */
  FP4_ERR_UNSUPPORTED = -2, /* option or shape combination the method does not define here */
  FP4_ERR_ALIGN = -3,       /* pointer or stride misaligned (see each entry point) */
  FP4_ERR_DEVICE = -4,      /* the current HIP device is not gfx950 */
  FP4_ERR_WORKSPACE = -5,   /* workspace missing or smaller than fp4_quantize_workspace() */
  FP4_ERR_HIP = -6,         /* the HIP runtime reported an error at launch */
  FP4_ERR_SCRATCH = -7      /* fp4_quantize_noalloc: the call needs more scratch than
                               FP4_NOALLOC_SCRATCH_BYTES, or the scratch could not be located */
} fp4_status;

typedef enum { FP4_MXFP4 = 0, FP4_NVFP4 = 1 } fp4_format;

typedef enum { FP4_F32 = 0, FP4_BF16 = 1 } fp4_dtype;

/* fp4_quant_opts.flags */
enum {
  /* NVFP4: each block is scaled so its max maps to 4 and to 6; the
   * candidate with the smaller sum of squared errors is kept (ties keep 6).
   * ("Four Over Six", introduction.) MXFP4: the same choice between the
   * power-of-two scales that put the block max in [4, 8) (the standard
   * exponent e, values above 6 clip) and in [2, 4) (e + 1); e + 1 is kept
   * iff its squared error is smaller. */
  FP4_FOUR_OVER_SIX = 1u,
  /* NVFP4 only. One scale per 16x16 tile instead of per 1x16 row slice.
   * ("Four Over Six", option list: 2D block scaling.) */
  FP4_BLOCK2D = 2u,
  /* Quantize X^T: blocks run along the rows of X^T, i.e. down the columns of
   * X; the output has shape [cols, rows]. ("Four Over Six": transposed
   * inputs.) */
  FP4_TRANSPOSE = 4u,
  /* Stochastic rounding of the elements, driven by Philox4x32-10 (seed,
   * offset). ("FP4", section "Inferencia e Treinamento FP4"; "Four Over
   * Six" option list.) */
  FP4_STOCHASTIC = 8u,
  /* Random Hadamard transform of every 16-slice along the block direction
   * before quantization: sign flip by rht_signs, 16-point Walsh-Hadamard,
   * times 1/4. The same signs applied to both GEMM operands cancel in the
   * product. ("FP4", "Inferencia e Treinamento FP4"; "Four Over Six".) */
  FP4_HADAMARD = 16u,
  /* NVFP4 only. The 4/6 choice widened to every E4M3 scale code from the
   * M = 6 candidate's to the M = 4 candidate's: the block max may map to
   * any representable point between 6 and 4; the smallest squared error
   * wins, ties keep the smaller code. Tensor scale as under 4/6 (D = 4 *
   * 448); takes precedence over FP4_FOUR_OVER_SIX. (The pages' theme of
   * choosing the scale by error, "Four Over Six", introduction.) */
  FP4_SCALE_SEARCH = 32u,
  /* NVFP4 layout with one scale for the whole tensor: every block-scale byte
   * is 0x38 (E4M3 1.0) and S_t = T / 6, so each value is quantized against
   * T / 6 alone, the whole-tensor scaling of the worked example ("FP4",
   * "Como funciona FP4": the block is the whole tensor, its max maps to 6).
   * Dequantize and fp4_gemm read it as any NVFP4 tensor. Not with
   * FP4_FOUR_OVER_SIX, FP4_SCALE_SEARCH or FP4_BLOCK2D (FP4_ERR_UNSUPPORTED). */
  FP4_TENSOR_SCALE = 64u
};

typedef struct fp4_quant_opts {
  uint32_t size;        /* must equal sizeof(fp4_quant_opts) */
  int32_t format;       /* fp4_format */
  uint32_t flags;       /* FP4_* bits above; unknown bits -> FP4_ERR_INVALID */
  uint32_t rht_signs;   /* FP4_HADAMARD: bit i negates element i of each 16-slice */
  uint64_t seed;        /* FP4_STOCHASTIC: Philox key (low, high words) */
  uint64_t offset;      /* FP4_STOCHASTIC: Philox counter words 2 and 3 */
  const float* amax_in; /* NVFP4: optional device array [batch] of tensor amax
                           values (after the transform, if any); NULL = the
                           library computes it in a pre-pass */
} fp4_quant_opts;

/*
 * Bytes of device workspace fp4_quantize needs for these sizes and options
 * (0 when none: MXFP4, or NVFP4 with amax_in supplied). Returns 0 for
 * arguments fp4_quantize would reject.
 */
size_t fp4_quantize_workspace(int64_t batch, int64_t rows, int64_t cols, const fp4_quant_opts* opts);

/*
 * fp4_quantize -- quantize `batch` matrices X_b [rows, cols] to FP4.
 *
 *   x            device, fp32 or bf16 (x_dtype); element (b, r, c) at
 *                x[b * batch_stride_x + r * ld_x + c] (strides in elements).
 *                16-byte aligned; ld_x and batch_stride_x multiples of
 *                16 bytes' worth of elements.
 *   opts         host pointer, see fp4_quant_opts.
 *   codes        device, output [batch][R, C/2] bytes with (R, C) = (rows,
 *                cols), or (cols, rows) under FP4_TRANSPOSE; 8-byte aligned,
 *                ld_codes >= C/2 and a multiple of 8, batch_stride_codes a
 *                multiple of 8.
 *   scales       device, output [batch][R, C/blk] bytes; ld_scales >= C/blk.
 *   tensor_scale NVFP4: device float[batch], receives S_t; MXFP4: ignored.
 *   workspace    device scratch of at least fp4_quantize_workspace() bytes,
 *                16-byte aligned; may be NULL when that is 0. Its contents on
 *                entry do not matter; it must not be shared by calls running
 *                concurrently.
 *
 * Shape rules (else FP4_ERR_INVALID): C % blk == 0; under FP4_TRANSPOSE the
 * source column count (= R) is a multiple of 8; under FP4_BLOCK2D also
 * R % 16 == 0.
 * FP4_BLOCK2D or FP4_SCALE_SEARCH with MXFP4 -> FP4_ERR_UNSUPPORTED.
 *
 * NVFP4 tensor scale: T = max |x| over the batch item (after the Hadamard
 * transform, if on) or amax_in[b]; S_t = T / (6 * 448), or T / (4 * 448)
 * under FP4_FOUR_OVER_SIX or FP4_SCALE_SEARCH, or T / 6 under
 * FP4_TENSOR_SCALE; S_t = 1 when that is zero, denormal or not finite.
 */
fp4_status fp4_quantize(const void* x, int32_t x_dtype, int64_t batch, int64_t rows, int64_t cols,
                        int64_t ld_x, int64_t batch_stride_x, const fp4_quant_opts* opts,
                        uint8_t* codes, int64_t ld_codes, int64_t batch_stride_codes,
                        uint8_t* scales, int64_t ld_scales, int64_t batch_stride_scales,
                        float* tensor_scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp4_quantize_noalloc -- fp4_quantize for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc. Same arguments, results and errors as
 * fp4_quantize, without the workspace: the NVFP4 tensor-amax partials go to
 * a scratch array inside the library, FP4_NOALLOC_SCRATCH_BYTES per GPU,
 * held by each GPU the library runs on until the process ends. Nothing is
 * allocated or freed and no allocating routine is called.
 *   Limit: a call whose fp4_quantize_workspace() would exceed
 *   FP4_NOALLOC_SCRATCH_BYTES returns FP4_ERR_SCRATCH with nothing enqueued
 *   (one NVFP4 item without amax_in needs at most 4100 bytes, so up to 63
 *   batch items always fit). MXFP4, and NVFP4 with amax_in, need none.
 *   The first call on a device looks up that device's copy of the array
 *   (FP4_ERR_SCRATCH if the runtime cannot); later calls reuse the address.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (different streams, or different host threads without ordering)
 *   race and may produce wrong tensor scales. Calls ordered on one stream
 *   are safe. The array keeps the last call's contents; no word of it needs
 *   to start at zero (the pre-pass writes every word the quantizer reads).
 */
#define FP4_NOALLOC_SCRATCH_BYTES 262144
fp4_status fp4_quantize_noalloc(const void* x, int32_t x_dtype, int64_t batch, int64_t rows, int64_t cols,
                                int64_t ld_x, int64_t batch_stride_x, const fp4_quant_opts* opts,
                                uint8_t* codes, int64_t ld_codes, int64_t batch_stride_codes,
                                uint8_t* scales, int64_t ld_scales, int64_t batch_stride_scales,
                                float* tensor_scale, void* stream);

/*
 * fp4_dequantize -- y = val(code) * scale, per element ("FP4", section "Como
 * funciona FP4": dequantized value = grid value * sign * scale).
 * MXFP4: val * 2^(byte - 127). NVFP4: val * (E4M3(byte) * tensor_scale[b]).
 * Shapes as produced by fp4_quantize: codes [batch][rows, cols/2], scales
 * [batch][rows, cols/blk]; y [batch][rows, cols] of y_dtype (fp32 or bf16,
 * round-to-nearest-even), strides in elements, 16-byte aligned with 16-byte
 * row pitch. cols % blk == 0. codes 8-byte aligned, ld_codes a multiple of 8.
 * The Hadamard transform, if one was applied, is not undone.
 */
fp4_status fp4_dequantize(int32_t format, int64_t batch, int64_t rows, int64_t cols,
                          const uint8_t* codes, int64_t ld_codes, int64_t batch_stride_codes,
                          const uint8_t* scales, int64_t ld_scales, int64_t batch_stride_scales,
                          const float* tensor_scale, void* y, int32_t y_dtype, int64_t ld_y,
                          int64_t batch_stride_y, void* stream);

/*
 * fp4_gemm -- W4A4 block-scaled GEMM ("FP4", section "Inferencia e
 * Treinamento FP4": matrix products in FP4 with higher-precision
 * accumulation):
 *   C_g[m, n] = sum_k deq(A_g)[m, k] * deq(B_g)[n, k],  g < groups,
 * accumulated in fp32, written as fp32 or bf16 (c_dtype, round-to-nearest-
 * even). A_g is [M, K] and B_g is [N, K] (an nn.Linear weight [out, in]),
 * both K-major codes+scales as fp4_quantize writes them (quantize a [K, N]
 * weight with FP4_TRANSPOSE). MXFP4 runs on the gfx950 block-scaled FP4
 * matrix cores; NVFP4 is dequantized exactly to fp16 in registers and
 * multiplied on the fp16 matrix cores, with S_a * S_b applied in the
 * epilogue. a_tensor_scale / b_tensor_scale: NVFP4 device float[groups].
 *   Strides: lda, ldb in bytes (>= K/2, multiples of 16); lda_scales,
 *   ldb_scales in bytes (>= K/blk, multiples of 16); ldc and group strides
 *   of C in elements; group strides of codes/scales in bytes (multiples of
 *   16). K % 64 == 0; M and N arbitrary (>= 0). Code and scale pointers
 *   16-byte aligned; c 4-byte aligned (2 for bf16).
 *   Scale rows are read in 16-byte pieces up to the next multiple of 16 of
 *   K/blk, so every scale row must be readable up to that length (true for
 *   any [rows, ld] buffer with ld a multiple of 16): give fp4_quantize a
 *   scale pitch rounded up to 16 bytes when its output feeds fp4_gemm.
 *   Each group's code and scale panels must span less than 2 GiB, and
 *   every row pitch (lda, ldb, lda_scales, ldb_scales) must be below 8 MiB
 *   (else FP4_ERR_UNSUPPORTED).
 * Errors: FP4_ERR_INVALID for bad sizes, strides or NULL operands,
 * FP4_ERR_ALIGN for misaligned pointers or pitches, FP4_ERR_DEVICE off
 * gfx950, FP4_ERR_HIP if the launch fails. Nothing is written on error.
 */
fp4_status fp4_gemm(int32_t format, int64_t groups, int64_t M, int64_t N, int64_t K,
                    const uint8_t* a_codes, int64_t lda, int64_t a_group_stride,
                    const uint8_t* a_scales, int64_t lda_scales, int64_t a_scales_group_stride,
                    const float* a_tensor_scale,
                    const uint8_t* b_codes, int64_t ldb, int64_t b_group_stride,
                    const uint8_t* b_scales, int64_t ldb_scales, int64_t b_scales_group_stride,
                    const float* b_tensor_scale,
                    void* c, int32_t c_dtype, int64_t ldc, int64_t c_group_stride, void* stream);

/*
 * fp4_gemm_quantize_output -- fp4_gemm whose epilogue quantizes the product
 * instead of storing it, so that a W4A4 layer hands the next one FP4
 * activations without a round trip of C through HBM ("FP4", section
 * "Inferencia e Treinamento FP4": activations quantized to FP4 for FP4
 * matrix products). Operands, groups, strides and their errors as for
 * fp4_gemm. Each C_g [M, N], as fp4_gemm computes it in fp32 (after the
 * tensor scales), is quantized along its rows exactly as fp4_quantize
 * quantizes a row-major [M, N] fp32 matrix with out_opts:
 *   out_opts     format MXFP4 or NVFP4 (either, whatever the operands'
 *                format); flags FP4_FOUR_OVER_SIX, FP4_SCALE_SEARCH
 *                (NVFP4), FP4_STOCHASTIC
 *                (index of element (m, n) of group g: (g M + m) N + n, as in
 *                a batched fp4_quantize), FP4_HADAMARD; FP4_BLOCK2D and
 *                FP4_TRANSPOSE -> FP4_ERR_UNSUPPORTED. NVFP4 needs amax_in:
 *                device float[groups], the tensor amax to derive S_t from
 *                (the amax of C is only known once C is complete, so the
 *                caller supplies it, e.g. from a previous step or a
 *                calibration; values above it saturate).
 *   out_codes    device [groups][M, N/2] bytes, row pitch ld_out_codes
 *                (>= N/2, a multiple of 8; 8-byte aligned base and group
 *                stride).
 *   out_scales   device [groups][M, N/blk] bytes, row pitch ld_out_scales.
 *   out_tensor_scale  NVFP4: device float[groups], receives S_t.
 * N must be a multiple of the output block (16 or 32), else
 * FP4_ERR_INVALID.
 */
fp4_status fp4_gemm_quantize_output(int32_t format, int64_t groups, int64_t M, int64_t N, int64_t K,
                                    const uint8_t* a_codes, int64_t lda, int64_t a_group_stride,
                                    const uint8_t* a_scales, int64_t lda_scales, int64_t a_scales_group_stride,
                                    const float* a_tensor_scale,
                                    const uint8_t* b_codes, int64_t ldb, int64_t b_group_stride,
                                    const uint8_t* b_scales, int64_t ldb_scales, int64_t b_scales_group_stride,
                                    const float* b_tensor_scale, const fp4_quant_opts* out_opts,
                                    uint8_t* out_codes, int64_t ld_out_codes, int64_t out_codes_group_stride,
                                    uint8_t* out_scales, int64_t ld_out_scales, int64_t out_scales_group_stride,
                                    float* out_tensor_scale, void* stream);

/*
 * fp4_gemm_grouped -- the grouped GEMM of a mixture-of-experts layer, where
 * a router decides how many rows (tokens) each group (expert) gets ("FP4",
 * section "Inferencia e Treinamento FP4": MoE weights in MXFP4, FP4 matrix
 * products with higher-precision accumulation):
 *   C[m, n] = sum_k deq(A)[m, k] * deq(B_g)[n, k]
 *             for offsets[g] <= m < offsets[g + 1], g < groups.
 * A [M, K] holds every group's rows back to back, as one fp4_quantize call
 * writes them (one NVFP4 tensor scale, a_tensor_scale: device float[1]);
 * B_g [N, K] at b_group_stride (b_tensor_scale: NVFP4 device float[groups]);
 * C [M, N], row pitch ldc in elements. Rows of C outside every group are not
 * written. Formats, strides, alignment and the 2 GiB / 8 MiB limits are as
 * for fp4_gemm, with A and C taken as one group of M rows.
 *   group_offsets: DEVICE int32[groups + 1], read by the kernel (stream-
 *   ordered), so counts that a router computed on the device need no host
 *   round trip. Meant to be nondecreasing from 0 to M; the kernel clamps
 *   each offset into [0, M] and each group's end to at least its start, so
 *   no offsets make it access memory outside A, B and C (but overlapping
 *   groups write the same rows in an unspecified order).
 *   Work per tile grows with groups / 64; groups > 4096 ->
 *   FP4_ERR_UNSUPPORTED. Errors as for fp4_gemm.
 */
fp4_status fp4_gemm_grouped(int32_t format, int64_t groups, const int32_t* group_offsets, int64_t M, int64_t N,
                            int64_t K, const uint8_t* a_codes, int64_t lda, const uint8_t* a_scales,
                            int64_t lda_scales, const float* a_tensor_scale,
                            const uint8_t* b_codes, int64_t ldb, int64_t b_group_stride,
                            const uint8_t* b_scales, int64_t ldb_scales, int64_t b_scales_group_stride,
                            const float* b_tensor_scale, void* c, int32_t c_dtype, int64_t ldc, void* stream);

/* Static string naming a status code; never NULL. */
const char* fp4_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H */
