/*
 * fp4_oracle.c -- plain, slow, single-threaded CPU oracle for block-scaled FP4
 * (E2M1) quantization, dequantization and the W4A4 GEMM reference.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library may include, link,
 * load or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header, table or constant with the
 * HIP kernels: every table below is written out here on its own.
 *
 * Arithmetic: IEEE binary32, round-to-nearest-even, one rounding per written
 * operation. Build with -ffp-contract=off so that no multiply-add is fused
 * unless fmaf() is written explicitly. Denormals are honoured.
 *
 * Sources (the pages):
 *   [FP4]   Ultralytics glossary page "FP4": section "Como funciona FP4" gives
 *           the E2M1 value set, the per-block scale that maps the block's
 *           largest magnitude near 6, MXFP4 (32 values under an 8-bit
 *           power-of-two E8M0 scale, per the OCP MX spec) and NVFP4 (16 values
 *           under an FP8 E4M3 scale plus a second per-tensor FP32 scale), and
 *           the worked example (whole-tensor / 32 / 16 block MAE).
 *           Section "Inferencia e Treinamento FP4": FP4 matmul with
 *           higher-precision accumulation; random Hadamard transforms to spread
 *           outliers and stochastic rounding for gradients.
 *   [4o6]   Hugging Face transformers page "Four Over Six" (Quatro sobre seis),
 *           introduction: NVFP4 blocks scaled adaptively so their max maps to
 *           4 or to 6; options random Hadamard transform, 2D block scaling,
 *           transposed inputs, stochastic rounding; an FP32-simulated matmul
 *           fallback (dequantize, then multiply in FP32).
 *
 * Where the pages leave a step open, the reading taken is stated at the step.
 * Parity status of each function is listed in the header comment of
 * oracle.py (the Python wrapper).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>

/* ------------------------------------------------------------------------ */
/* E2M1 element format                                                        */
/* ------------------------------------------------------------------------ */

/* [FP4] "Como funciona FP4": the eight non-negative E2M1 magnitudes; bit 3 of
 * a code is the sign, bits 2:0 index this table. */
static const float E2M1_MAGNITUDE[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float or_e2m1_value(uint8_t code) {
  float m = E2M1_MAGNITUDE[code & 7];
  return (code & 8) ? -m : m;
}

/* Nearest E2M1 value to q, ties to the even code (round-to-nearest-even in the
 * 1-bit mantissa), saturating at +-6. The pages' snippet takes the nearest grid
 * value; the tie rule is a reading (the snippet's argmin would take the lower
 * value). Each threshold is the midpoint between neighbouring magnitudes; the
 * comparison is strict where the lower neighbour has the even code and
 * inclusive where the upper one has. The sign bit is copied from q, so -0 and
 * small negatives give code 0x8. */
uint8_t or_e2m1_rne(float q) {
  uint8_t sign = signbit(q) ? 8 : 0;
  float a = fabsf(q);
  uint8_t m = (uint8_t)((a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                        (a > 2.5f) + (a >= 3.5f) + (a > 5.0f));
  return sign | m;
}

/* Stochastic rounding of q onto the E2M1 grid ([FP4] "Inferencia e
 * Treinamento FP4" names stochastic rounding for gradients; the rule is a
 * reading). With a = |q| < 6, lo the largest magnitude <= a and hi the next,
 * f = (a - lo) / (hi - lo) is exact (Sterbenz, and a power-of-two divisor).
 * The 16-bit random integer r rounds up iff r < f * 2^16, so
 * P(up) = ceil(f * 2^16) / 2^16 and grid values are never moved. a >= 6
 * saturates to 6. */
uint8_t or_e2m1_sr(float q, uint32_t r16) {
  uint8_t sign = signbit(q) ? 8 : 0;
  float a = fabsf(q);
  if (a >= 6.0f) return sign | 7;
  int lo = 0;
  while (lo < 6 && E2M1_MAGNITUDE[lo + 1] <= a) lo++;
  float step = E2M1_MAGNITUDE[lo + 1] - E2M1_MAGNITUDE[lo];
  float f = (a - E2M1_MAGNITUDE[lo]) / step;
  int up = (float)r16 < f * 65536.0f;
  return sign | (uint8_t)(lo + up);
}

/* ------------------------------------------------------------------------ */
/* Scale formats                                                              */
/* ------------------------------------------------------------------------ */

/* OCP FP8 E4M3 ("fn" variant): bias 7, no infinities, 0x7F/0xFF are NaN, max
 * finite 448, subnormal step 2^-9. [FP4] names E4M3 as the NVFP4 block-scale
 * format. */
float or_e4m3_value(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  float v = (e == 0) ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return (c & 0x80) ? -v : v;
}

/* Nearest E4M3 value to s in [0, 448], ties to the even code, found by
 * exhaustive search over the 127 non-negative finite codes. */
uint8_t or_e4m3_rne(float s) {
  uint8_t best = 0;
  double best_d = INFINITY;
  for (int c = 0; c <= 126; c++) {
    double d = fabs((double)or_e4m3_value((uint8_t)c) - (double)s);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = (uint8_t)c;
      best_d = d;
    }
  }
  return best;
}

/* E8M0 block exponent for MXFP4 ([FP4]: 32 values under an 8-bit power-of-two
 * scale per the OCP MX spec). Reading: e = floor(log2(amax)) - 2, the MX
 * convention that puts the block max in [4, 8) so that values above 6
 * saturate; clamped to the E8M0 range [-127, 127]; amax = 0 gives -127. The
 * stored byte is e + 127. */
int or_e8m0_exponent(float amax) {
  if (amax == 0.0f) return -127;
  int E;
  (void)frexpf(amax, &E); /* amax = m * 2^E, m in [0.5, 1): floor(log2) = E-1 */
  int e = (E - 1) - 2;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as     */
/* easy as 1, 2, 3", SC'11): 10 rounds of the Philox S-box on a 128-bit        */
/* counter under a 64-bit key, with the Weyl key schedule.                     */
/* ------------------------------------------------------------------------ */
void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; round++) {
    uint64_t p0 = (uint64_t)M0 * c0;
    uint64_t p1 = (uint64_t)M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += W0;
    k1 += W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 16-bit random integer for the element whose linear index (row-major over
 * the whole, possibly batched, output) is L. Reading: one Philox call per 8
 * consecutive elements, counter = (n_lo, n_hi, offset_lo, offset_hi) with
 * n = L / 8, key = (seed_lo, seed_hi); the call's four 32-bit words are split
 * into halves, word (L / 2) % 4, low half for even L, high half for odd L. */
uint32_t or_sr_random16(uint64_t seed, uint64_t offset, uint64_t L) {
  uint64_t n = L >> 3;
  uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  or_philox4x32_10(ctr, key, out);
  uint32_t w = out[(L >> 1) & 3];
  return (L & 1) ? (w >> 16) : (w & 0xFFFFu);
}

/* ------------------------------------------------------------------------ */
/* Random Hadamard transform on one 16-slice ([4o6] option list; [FP4]        */
/* "Inferencia e Treinamento FP4": RHT spreads outliers).                     */
/* Reading: negate v_i where bit i of `signs` is set, apply the fast           */
/* Walsh-Hadamard transform (Sylvester order) in stages h = 1, 2, 4, 8, each   */
/* butterfly (a, b) -> (a + b, a - b), then multiply by 1/4 so the transform   */
/* is orthonormal.                                                            */
/* ------------------------------------------------------------------------ */
void or_rht16(float v[16], uint32_t signs) {
  for (int i = 0; i < 16; i++)
    if ((signs >> i) & 1u) v[i] = -v[i];
  for (int h = 1; h < 16; h <<= 1) {
    for (int j = 0; j < 16; j++) {
      if (j & h) continue;
      float a = v[j], b = v[j + h];
      v[j] = a + b;
      v[j + h] = a - b;
    }
  }
  for (int i = 0; i < 16; i++) v[i] = v[i] * 0.25f;
}

/* ------------------------------------------------------------------------ */
/* Quantizer                                                                  */
/* ------------------------------------------------------------------------ */

enum { OR_MXFP4 = 0, OR_NVFP4 = 1 };
enum { OR_F32 = 0, OR_BF16 = 1 };
enum {
  OR_FOUR_OVER_SIX = 1u,
  OR_BLOCK2D = 2u,
  OR_TRANSPOSE = 4u,
  OR_STOCHASTIC = 8u,
  OR_HADAMARD = 16u,
  OR_SCALE_SEARCH = 32u,
  OR_TENSOR_SCALE = 64u
};

static float load_elem(const void* x, int dtype, int64_t idx) {
  if (dtype == OR_BF16) {
    uint32_t bits = (uint32_t)((const uint16_t*)x)[idx] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
  }
  return ((const float*)x)[idx];
}

/* Materialise the working matrix W [rows_out, cols_out] in fp32: the input,
 * transposed when OR_TRANSPOSE is set ([4o6] option list: transposed
 * inputs; quantize X^T, blocks running along the rows of X^T), then the RHT on every 16-slice
 * of each row when OR_HADAMARD is set. Returns malloc'd memory. */
static float* working_matrix(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                             unsigned flags, uint32_t signs, int64_t* rows_out, int64_t* cols_out) {
  int tr = (flags & OR_TRANSPOSE) != 0;
  int64_t R = tr ? cols : rows, C = tr ? rows : cols;
  float* w = (float*)malloc((size_t)(R * C) * sizeof(float));
  if (!w) return NULL;
  for (int64_t r = 0; r < R; r++)
    for (int64_t c = 0; c < C; c++)
      w[r * C + c] = tr ? load_elem(x, dtype, c * ld + r) : load_elem(x, dtype, r * ld + c);
  if (flags & OR_HADAMARD)
    for (int64_t r = 0; r < R; r++)
      for (int64_t c = 0; c < C; c += 16) or_rht16(&w[r * C + c], signs);
  *rows_out = R;
  *cols_out = C;
  return w;
}

/* Tensor amax T = max |w| over the working matrix (after the RHT). */
float or_tensor_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                     unsigned flags, uint32_t signs) {
  int64_t R, C;
  float* w = working_matrix(x, dtype, rows, cols, ld, flags, signs, &R, &C);
  if (!w) return NAN;
  float t = 0.0f;
  for (int64_t i = 0; i < R * C; i++) {
    float a = fabsf(w[i]);
    if (a > t) t = a;
  }
  free(w);
  return t;
}

/* NVFP4 per-tensor FP32 scale ([FP4] "Como funciona FP4": NVFP4 puts one
 * FP32 scale per tensor on top of its E4M3 block scales). Reading: amax-based, S_t = T / D with D = 6 * 448 so that the block holding
 * the tensor max gets the largest E4M3 scale; under 4/6, D = 4 * 448 so the
 * M = 4 candidate of that block does not saturate. If S_t is zero, denormal or
 * not finite, S_t = 1 (the tensor then quantizes to zeros). */
float or_nvfp4_tensor_scale(float amax, int four_over_six) {
  /* four_over_six = 2: the whole-tensor mode below, D = 6 */
  float D = four_over_six == 2 ? 6.0f : (four_over_six ? 1792.0f : 2688.0f);
  float s = amax / D;
  if (!(s >= FLT_MIN) || !(s <= FLT_MAX)) s = 1.0f;
  return s;
}

/* One NVFP4 scale candidate for a block whose amax is `a`: the block max maps
 * to M (6, or 4 under 4/6). s = a * k_M with k_M = 1 / (M * S_t) formed once
 * per tensor; the E4M3 code is the nearest to min(s, 448); eff = dec * S_t is
 * the effective scale, r = 1 / eff its reciprocal. A block whose eff is below
 * FLT_MIN (including eff = 0) is a zero block: every code keeps only its sign. */
typedef struct {
  uint8_t code;
  float eff, r;
  int zero;
} nv_cand;

static nv_cand nv_candidate(float a, float M, float S_t) {
  nv_cand c;
  float k = 1.0f / (M * S_t);
  float s = a * k;
  if (s > 448.0f) s = 448.0f;
  c.code = or_e4m3_rne(s);
  c.eff = or_e4m3_value(c.code) * S_t;
  c.zero = !(c.eff >= FLT_MIN);
  c.r = c.zero ? 0.0f : 1.0f / c.eff;
  return c;
}

/* The candidate whose E4M3 code is `code` (the scale search below). */
static nv_cand nv_code_candidate(uint8_t code, float S_t) {
  nv_cand c;
  c.code = code;
  c.eff = or_e4m3_value(code) * S_t;
  c.zero = !(c.eff >= FLT_MIN);
  c.r = c.zero ? 0.0f : 1.0f / c.eff;
  return c;
}

static uint8_t quant_rne_nv(float x, const nv_cand* c) {
  if (c->zero) return signbit(x) ? 8 : 0;
  return or_e2m1_rne(x * c->r);
}

/* Squared error of one 16-value row under a candidate, in the scaled domain:
 * with q = x * r and d = val(code(q)) - q (exact, by Sterbenz), the sum of d^2
 * is taken as two fused-multiply-add chains, over elements 0..7 and over
 * elements 8..15 in order, then added. `stride` steps between the elements. */
static float row16_sq_err(const float* x, int64_t stride, const nv_cand* c) {
  float half[2];
  for (int hf = 0; hf < 2; hf++) {
    float acc = 0.0f;
    for (int i = 8 * hf; i < 8 * hf + 8; i++) {
      float q = x[i * stride] * c->r;
      float d = or_e2m1_value(or_e2m1_rne(q)) - q;
      acc = fmaf(d, d, acc);
    }
    half[hf] = acc;
  }
  return half[0] + half[1];
}

/* The 4/6 error of one candidate for the block at (r0, c0): eff^2 times the
 * row16_sq_err sum, over the 16 source rows of a 16x16 tile combined by a
 * pairwise tree over adjacent rows; infinite for a zero-block candidate. */
static float nv_block_sse(const float* w, int64_t C, int64_t r0, int64_t c0, int b2d, int tr, const nv_cand* c) {
  if (c->zero) return INFINITY;
  float part[16];
  if (!b2d) {
    part[0] = row16_sq_err(&w[r0 * C + c0], 1, c);
  } else {
    for (int s = 0; s < 16; s++)
      part[s] = tr ? row16_sq_err(&w[r0 * C + c0 + s], C, c) : row16_sq_err(&w[(r0 + s) * C + c0], 1, c);
    for (int width = 1; width < 16; width <<= 1)
      for (int s = 0; s < 16; s += 2 * width) part[s] = part[s] + part[s + width];
  }
  return (c->eff * c->eff) * part[0];
}

typedef struct {
  int format;
  unsigned flags;
  uint64_t seed, offset;
  uint32_t rht_signs;
  int has_amax;
  float amax;
} or_opts;

/*
 * or_quantize: quantize X [rows, cols] (row stride ld elements, fp32 or bf16).
 * Output (dense): codes [R, C/2] bytes, element 2j in bits 3:0 and 2j+1 in
 * bits 7:4 of byte j; scales [R, C/blk] bytes (E8M0 exponent + 127 for MXFP4,
 * E4M3 code for NVFP4; under OR_BLOCK2D each 16x16 tile's byte is written on
 * all 16 of its rows). (R, C) = (rows, cols), or (cols, rows) under
 * OR_TRANSPOSE. For NVFP4, *tensor_scale receives S_t and *amax_out T.
 * `L0` is the linear index of element (0, 0) of this output inside the whole
 * batched output; it only feeds the stochastic-rounding counter.
 * Returns 0, or -1 on a shape the method does not define.
 */
int or_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, const or_opts* o,
                uint64_t L0, uint8_t* codes, uint8_t* scales, float* tensor_scale, float* amax_out) {
  int nv = o->format == OR_NVFP4;
  int blk = nv ? 16 : 32;
  int search = nv && (o->flags & OR_SCALE_SEARCH);
  int fos = nv && (o->flags & OR_FOUR_OVER_SIX);
  int b2d = nv && (o->flags & OR_BLOCK2D);
  int sr = (o->flags & OR_STOCHASTIC) != 0;
  /* Whole-tensor scale ([FP4] "Como funciona FP4": the worked example's
   * first mode, one scale for the whole tensor that maps its max to 6): kept
   * in the NVFP4 layout with every block's E4M3 scale at 1.0, and S_t = T / 6
   * (a reading: the pages store no format for it). */
  int whole = nv && (o->flags & OR_TENSOR_SCALE);
  if (!nv && (o->flags & (OR_BLOCK2D | OR_SCALE_SEARCH | OR_TENSOR_SCALE))) return -1;
  if (whole && (o->flags & (OR_FOUR_OVER_SIX | OR_SCALE_SEARCH | OR_BLOCK2D))) return -1;
  int64_t R, C;
  float* w = working_matrix(x, dtype, rows, cols, ld, o->flags, o->rht_signs, &R, &C);
  if (!w) return -1;
  if (C % blk != 0 || (b2d && R % 16 != 0)) {
    free(w);
    return -1;
  }
  int64_t nb = C / blk;
  memset(codes, 0, (size_t)(R * C / 2));

  if (!nv) {
    /* MXFP4: e = E8M0 exponent of the block amax; q = x * 2^-e, exact barring
     * underflow (ldexpf rounds it correctly); dequantized value val * 2^e. */
    for (int64_t r = 0; r < R; r++) {
      for (int64_t b = 0; b < nb; b++) {
        const float* v = &w[r * C + b * blk];
        float a = 0.0f;
        for (int i = 0; i < blk; i++)
          if (fabsf(v[i]) > a) a = fabsf(v[i]);
        int e = or_e8m0_exponent(a);
        if ((o->flags & OR_FOUR_OVER_SIX) && e < 127) {
          /* 4/6 carried over to power-of-two scales (a reading; the pages
           * define 4/6 for NVFP4 only): the block max lands in [4, 8) under
           * e, in [2, 4) under e + 1, which clips nothing. Keep the exponent
           * with the smaller squared error SSE_e = 4^e * S_e, S_e the sum of
           * (val - q)^2 over the block with q = x * 2^-e, taken per 16-value
           * half as in row16_sq_err and the halves added; e + 1 wins iff
           * 4 * S_{e+1} < S_e (the 4^e factor cancels exactly). */
          float S[2];
          for (int k = 0; k < 2; k++) {
            float half[2];
            for (int hf = 0; hf < 2; hf++) {
              float part[2];
              for (int p8 = 0; p8 < 2; p8++) {
                float acc = 0.0f;
                for (int i = 16 * hf + 8 * p8; i < 16 * hf + 8 * p8 + 8; i++) {
                  float q = ldexpf(v[i], -(e + k));
                  float d = or_e2m1_value(or_e2m1_rne(q)) - q;
                  acc = fmaf(d, d, acc);
                }
                part[p8] = acc;
              }
              half[hf] = part[0] + part[1];
            }
            S[k] = half[0] + half[1];
          }
          if (4.0f * S[1] < S[0]) e = e + 1;
        }
        scales[r * nb + b] = (uint8_t)(e + 127);
        for (int i = 0; i < blk; i++) {
          int64_t col = b * blk + i;
          float q = ldexpf(v[i], -e);
          uint8_t cd = sr ? or_e2m1_sr(q, or_sr_random16(o->seed, o->offset, L0 + (uint64_t)(r * C + col)))
                          : or_e2m1_rne(q);
          codes[r * (C / 2) + col / 2] |= (uint8_t)(cd << ((col & 1) * 4));
        }
      }
    }
    free(w);
    return 0;
  }

  /* NVFP4 */
  float T;
  if (o->has_amax) {
    T = o->amax;
  } else {
    T = 0.0f;
    for (int64_t i = 0; i < R * C; i++)
      if (fabsf(w[i]) > T) T = fabsf(w[i]);
  }
  float S_t = or_nvfp4_tensor_scale(T, whole ? 2 : (fos || search));
  if (tensor_scale) *tensor_scale = S_t;
  if (amax_out) *amax_out = T;

  /* block geometry: 1 x 16, or 16 x 16 tiles under OR_BLOCK2D */
  int64_t tile_rows = b2d ? 16 : 1;
  for (int64_t r0 = 0; r0 < R; r0 += tile_rows) {
    for (int64_t b = 0; b < nb; b++) {
      int64_t c0 = b * 16;
      float a = 0.0f;
      for (int64_t r = r0; r < r0 + tile_rows; r++)
        for (int i = 0; i < 16; i++)
          if (fabsf(w[r * C + c0 + i]) > a) a = fabsf(w[r * C + c0 + i]);

      nv_cand c6 = nv_candidate(a, 6.0f, S_t);
      nv_cand chosen = c6;
      if (whole) {
        chosen = nv_code_candidate(0x38, S_t); /* E4M3 1.0: eff = S_t = T / 6 */
      } else if (search) {
        /* The 4/6 choice widened to every E4M3 scale between the two: the
         * candidates are the codes from the M = 6 candidate's up to the
         * M = 4 candidate's, so the block max maps to each representable
         * point between 6 and 4 (a reading of trying more candidate maxima; the
         * tensor scale is the 4/6 one). Each candidate's error is the 4/6
         * error below; the smallest wins, ties keep the smaller code. */
        uint8_t hi = nv_candidate(a, 4.0f, S_t).code;
        float best = nv_block_sse(w, C, r0, c0, b2d, (o->flags & OR_TRANSPOSE) != 0, &c6);
        for (int code = c6.code + 1; code <= hi; code++) {
          nv_cand c = nv_code_candidate((uint8_t)code, S_t);
          float e = nv_block_sse(w, C, r0, c0, b2d, (o->flags & OR_TRANSPOSE) != 0, &c);
          if (e < best) {
            best = e;
            chosen = c;
          }
        }
      } else if (fos) {
        /* [4o6] introduction: each block's max maps to 4 or to 6, keeping the
         * lower-error choice. Reading: error = sum of squared errors,
         * SSE_M = eff_M^2 * sum_i (val_i - q_i)^2 with q_i = x_i * r_M, the
         * sum over one 16-value row as in row16_sq_err; in a 16x16 tile the
         * 16 row sums (rows in the orientation of the *source* matrix, so a
         * transposed input gives the same choice) are combined by a pairwise
         * tree over adjacent rows. Pick 4 iff SSE_4 < SSE_6 (ties keep 6). A
         * zero-block candidate has infinite error. */
        nv_cand c4 = nv_candidate(a, 4.0f, S_t);
        int tr = (o->flags & OR_TRANSPOSE) != 0;
        float sse[2] = {nv_block_sse(w, C, r0, c0, b2d, tr, &c6), nv_block_sse(w, C, r0, c0, b2d, tr, &c4)};
        if (sse[1] < sse[0]) chosen = c4;
      }

      for (int64_t r = r0; r < r0 + tile_rows; r++) {
        scales[r * nb + b] = chosen.code;
        for (int i = 0; i < 16; i++) {
          int64_t col = c0 + i;
          float xv = w[r * C + col];
          uint8_t cd;
          if (chosen.zero) {
            cd = signbit(xv) ? 8 : 0;
          } else if (sr) {
            cd = or_e2m1_sr(xv * chosen.r, or_sr_random16(o->seed, o->offset, L0 + (uint64_t)(r * C + col)));
          } else {
            cd = quant_rne_nv(xv, &chosen);
          }
          codes[r * (C / 2) + col / 2] |= (uint8_t)(cd << ((col & 1) * 4));
        }
      }
    }
  }
  free(w);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantizer                                                                */
/* ------------------------------------------------------------------------ */

/* MXFP4: val * 2^e (exact). NVFP4: val * eff with eff = dec(E4M3) * S_t, one
 * rounding each, as in the quantizer. Output fp32 [R, C] dense. */
int or_dequantize(int format, int64_t R, int64_t C, const uint8_t* codes, const uint8_t* scales,
                  float tensor_scale, float* y) {
  int nv = format == OR_NVFP4;
  int blk = nv ? 16 : 32;
  if (C % blk != 0) return -1;
  int64_t nb = C / blk;
  for (int64_t r = 0; r < R; r++) {
    for (int64_t c = 0; c < C; c++) {
      uint8_t byte = codes[r * (C / 2) + c / 2];
      uint8_t cd = (c & 1) ? (byte >> 4) : (byte & 15);
      uint8_t s = scales[r * nb + c / blk];
      float val = or_e2m1_value(cd);
      if (nv) {
        float eff = or_e4m3_value(s) * tensor_scale;
        y[r * C + c] = val * eff;
      } else {
        y[r * C + c] = ldexpf(val, (int)s - 127);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Float-scale mode of the worked example ([FP4] "Como funciona FP4"): the    */
/* plain block scaling the page measures its MAE with, before any scale       */
/* format. Each block's scale is its largest magnitude over 6, in fp32, so    */
/* that the block max lands on 6; every value becomes the E2M1 magnitude      */
/* nearest to t = fl(|x| / scale), carrying the sign of x (zero stays zero),  */
/* times the scale. Where two magnitudes are equally near, the example keeps  */
/* the smaller one. That nearest magnitude is found as the number of          */
/* midpoints between neighbouring magnitudes that t exceeds (strictly, so     */
/* that a tie keeps the smaller one). Writes the dequantized tensor.          */
/* ------------------------------------------------------------------------ */
int or_float_scale_dequant(const float* x, int64_t n, int64_t block, float* deq) {
  static const float MIDPOINT[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  if (block <= 0 || n % block != 0) return -1;
  for (int64_t start = 0; start < n; start += block) {
    float largest = 0.0f;
    for (int64_t i = start; i < start + block; i++) largest = fmaxf(largest, fabsf(x[i]));
    const float scale = largest / 6.0f;
    for (int64_t i = start; i < start + block; i++) {
      const float t = fabsf(x[i]) / scale;
      int m = 0;
      while (m < 7 && t > MIDPOINT[m]) m++;
      const float mag = E2M1_MAGNITUDE[m] * scale;
      deq[i] = x[i] > 0.0f ? mag : (x[i] < 0.0f ? -mag : 0.0f);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the element codecs, for the tests' exhaustive sweeps.       */
/* ------------------------------------------------------------------------ */
void or_e2m1_rne_n(const float* q, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = or_e2m1_rne(q[i]);
}
void or_e4m3_rne_n(const float* s, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = or_e4m3_rne(s[i]);
}
void or_e2m1_sr_n(const float* q, const uint32_t* r16, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = or_e2m1_sr(q[i], r16[i]);
}
void or_e8m0_exponent_n(const float* a, int64_t n, int32_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = or_e8m0_exponent(a[i]);
}
