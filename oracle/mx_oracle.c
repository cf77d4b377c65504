/*
 * mx_oracle.c -- plain CPU reference for microscaling quantization and the
 * block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library. Shares no code with
 * it. Written for a reader checking it against the pages by eye: values come
 * from the formats' bit-field definitions, rounding is a nearest-value search
 * over the representable set, and sums are plain loops in double.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared.
 * Contraction must stay off: the NVFP4 sequence is specified in fp32 with one
 * rounding per operation.
 *
 * Parity status, per function (what pins each one is listed in the tests):
 *  - format decoders, element encoders, MX scale rule, MX quantize,
 *    dequantize, GEMM: pinned (printed value sets and formulas, invariants,
 *    brute force, library cross-checks).
 *  - NVFP4 quantize: the element and scale roundings are pinned, but the
 *    tensor-scale rule s_t = amax / (6 * 448) and the fp32 operation order are
 *    a reading; no page prints an NVFP4 worked example, so the composed
 *    sequence is pinned only by invariants.
 */
#include "mx_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Element and scale formats                                                  */
/* ------------------------------------------------------------------------ */

/* bf16 = the high 16 bits of an IEEE binary32. */
double mxo_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* E2M1 ("Fundamentos matematicos do formato MXFP4 e E8M0"): 1 sign bit,
 * 2 exponent bits with bias 1, 1 explicit mantissa bit. Exponent field 0 is
 * subnormal. */
double mxo_e2m1_value(uint8_t code) {
  int s = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double v;
  if (e == 0)
    v = ldexp(m / 2.0, 1 - 1); /* 2^(1-bias) * 0.m */
  else
    v = ldexp(1.0 + m / 2.0, e - 1); /* 2^(e-bias) * 1.m */
  return s ? -v : v;
}

/* FP8 E4M3 (OCP "fn" variant: no Inf, S.1111.111 is NaN, max 448 as in the
 * format table): exponent bias 7, 3 mantissa bits, field 0 is subnormal. */
double mxo_e4m3_value(uint8_t code) {
  int s = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, 1 - 7);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* FP8 E5M2 (OCP): exponent bias 15, 2 mantissa bits, field 0 subnormal,
 * field 31 is Inf (mantissa 0) or NaN; largest finite 1.75 * 2^15 = 57344. */
double mxo_e5m2_value(uint8_t code) {
  int s = (code >> 7) & 1;
  int e = (code >> 2) & 31;
  int m = code & 3;
  double v;
  if (e == 31) v = (m == 0) ? INFINITY : NAN;
  else if (e == 0)
    v = ldexp((double)m / 4.0, 1 - 15);
  else
    v = ldexp(1.0 + m / 4.0, e - 15);
  return s ? -v : v;
}

/* FP6 E3M2 (OCP MX): exponent bias 3, 2 mantissa bits, field 0 subnormal, no
 * Inf or NaN; largest 1.75 * 2^4 = 28. */
double mxo_e3m2_value(uint8_t code) {
  int s = (code >> 5) & 1;
  int e = (code >> 2) & 7;
  int m = code & 3;
  double v;
  if (e == 0)
    v = ldexp((double)m / 4.0, 1 - 3);
  else
    v = ldexp(1.0 + m / 4.0, e - 3);
  return s ? -v : v;
}

/* E8M0: an unsigned power of two, 2^(E-127). E = 255 is the format's NaN
 * (2^128 is not finite in fp32 either). */
double mxo_e8m0_value(uint8_t e) {
  if (e == 255) return NAN;
  return ldexp(1.0, (int)e - 127);
}

/* Nearest magnitude in a sorted code table, ties to the code with a clear LSB
 * (the even mantissa), saturating at the top code. Codes 0..ncodes-1 are the
 * non-negative values in increasing order. */
static int nearest_code(double a, double (*value)(uint8_t), int ncodes) {
  double top = value((uint8_t)(ncodes - 1));
  if (a >= top) return ncodes - 1; /* includes +Inf: saturate */
  int best = 0;
  double bestd = fabs(a - value(0));
  for (int c = 1; c < ncodes; c++) {
    double d = fabs(a - value((uint8_t)c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

uint8_t mxo_encode_e2m1(double v) {
  int neg = signbit(v) ? 1 : 0;
  int c = nearest_code(fabs(v), mxo_e2m1_value, 8);
  return (uint8_t)((neg << 3) | c);
}

uint8_t mxo_encode_e4m3(double v) {
  int neg = signbit(v) ? 1 : 0;
  int c = nearest_code(fabs(v), mxo_e4m3_value, 127); /* 0x00..0x7E finite */
  return (uint8_t)((neg << 7) | c);
}

uint8_t mxo_encode_e5m2(double v) {
  int neg = signbit(v) ? 1 : 0;
  int c = nearest_code(fabs(v), mxo_e5m2_value, 124); /* 0x00..0x7B finite */
  return (uint8_t)((neg << 7) | c);
}

uint8_t mxo_encode_e3m2(double v) {
  int neg = signbit(v) ? 1 : 0;
  int c = nearest_code(fabs(v), mxo_e3m2_value, 32);
  return (uint8_t)((neg << 5) | c);
}

/* bf16 nearest-even: keep the high half, adding half an ulp plus the LSB of
 * the kept part so that exact halves go to the even neighbour. */
uint16_t mxo_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Shared-exponent rule (FAQ, "Como o formato E8M0 calcula o expoente"):
 * E = ceil(log2(amax / emax)) + 127, i.e. 127 + the smallest integer n with
 * amax <= emax * 2^n, so no element of the block exceeds the element format's
 * ceiling after scaling. amax = 0 has no such smallest n (log2 -> -inf); the
 * clamp to the format's range [0, 254] gives E = 0. Evaluated by search, with
 * exact power-of-two products, not with a logarithm. */
int mxo_mx_scale_exponent(double amax, double emax) {
  if (!isfinite(amax)) return 255;
  if (amax == 0.0) return 0;
  int n = -300;
  while (!(amax <= ldexp(emax, n))) n++;
  int E = n + 127;
  if (E < 0) E = 0;
  if (E > 254) E = 254;
  return E;
}

static int elem_bits(int fmt) {
  if (fmt == MXO_FMT_MXFP8 || fmt == MXO_FMT_MXFP8_E5M2) return 8;
  return (fmt == MXO_FMT_MXFP6_E3M2) ? 6 : 4;
}

static int is_mx(int fmt) {
  return fmt == MXO_FMT_MXFP4 || fmt == MXO_FMT_MXFP8 || fmt == MXO_FMT_MXFP8_E5M2 ||
         fmt == MXO_FMT_MXFP6_E3M2;
}

/* Largest element value: what the MX scale rule maps the block amax onto. */
static double elem_max(int fmt) {
  switch (fmt) {
    case MXO_FMT_MXFP8: return 448.0;
    case MXO_FMT_MXFP8_E5M2: return 57344.0;
    case MXO_FMT_MXFP6_E3M2: return 28.0;
    default: return 6.0;
  }
}

static double elem_value(int fmt, uint8_t code) {
  switch (fmt) {
    case MXO_FMT_MXFP8: return mxo_e4m3_value(code);
    case MXO_FMT_MXFP8_E5M2: return mxo_e5m2_value(code);
    case MXO_FMT_MXFP6_E3M2: return mxo_e3m2_value(code);
    default: return mxo_e2m1_value(code);
  }
}

static uint8_t elem_encode(int fmt, double v) {
  switch (fmt) {
    case MXO_FMT_MXFP8: return mxo_encode_e4m3(v);
    case MXO_FMT_MXFP8_E5M2: return mxo_encode_e5m2(v);
    case MXO_FMT_MXFP6_E3M2: return mxo_encode_e3m2(v);
    default: return mxo_encode_e2m1(v);
  }
}

static int fmt_block(int fmt) {
  return (fmt == MXO_FMT_NVFP4 || fmt == MXO_FMT_MXFP4_MBS16) ? 16 : 32;
}

static int is_mbs(int fmt) { return fmt == MXO_FMT_MXFP4_MBS || fmt == MXO_FMT_MXFP4_MBS16; }

/* Elements per row must be a multiple of this: the block, or the 128-element
 * macro block of MXFP4-MBS. */
static int fmt_granule(int fmt) {
  return is_mbs(fmt) ? 128 : fmt_block(fmt);
}

/* 4 bits per element plus 8 bits per 32-element block is the page's
 * "4 + 8/32 = 4.25 bits per element". */
int64_t mxo_storage_bytes(int fmt, int64_t rows, int64_t cols) {
  if (fmt < MXO_FMT_MXFP4 || fmt > MXO_FMT_MXFP4_MBS16) return -1;
  int64_t n = rows * cols;
  int64_t code_bytes = n * elem_bits(fmt) / 8;
  int64_t scale_bytes = n / fmt_block(fmt);
  int64_t extra = (fmt == MXO_FMT_NVFP4) ? 4 : is_mbs(fmt) ? n / 128 : 0;
  return code_bytes + scale_bytes + extra;
}

/* ------------------------------------------------------------------------ */
/* Quantize                                                                   */
/* ------------------------------------------------------------------------ */

static void put_code(uint8_t* codes, int fmt, int64_t idx, uint8_t code) {
  const int w = elem_bits(fmt);
  if (w == 8) {
    codes[idx] = code;
    return;
  }
  /* bit b of the code goes to bit (w idx + b) of the byte string */
  for (int b = 0; b < w; b++) {
    int64_t bit = (int64_t)w * idx + b;
    uint8_t* byte = &codes[bit / 8];
    if ((code >> b) & 1)
      *byte = (uint8_t)(*byte | (1u << (bit % 8)));
    else
      *byte = (uint8_t)(*byte & ~(1u << (bit % 8)));
  }
}

static uint8_t get_code(const uint8_t* codes, int fmt, int64_t idx) {
  const int w = elem_bits(fmt);
  if (w == 8) return codes[idx];
  uint8_t code = 0;
  for (int b = 0; b < w; b++) {
    int64_t bit = (int64_t)w * idx + b;
    code = (uint8_t)(code | (((codes[bit / 8] >> (bit % 8)) & 1u) << b));
  }
  return code;
}

static int bf16_is_finite(uint16_t bits) {
  return ((bits >> 7) & 0xFF) != 0xFF;
}

/* MXFP4 / MXFP8: per 32-element block, E from the block amax, then each
 * element divided by 2^(E-127) (exact in double) and rounded to the nearest
 * element value. A block holding Inf or NaN gets the NaN scale and zero codes.
 * emax is the value the scale rule maps the amax onto: the element format's
 * largest value (6 or 448), or 7 for MXFP4 under OAS. */
static void quantize_mx(int fmt, int64_t rows, int64_t cols, const uint16_t* x,
                        uint8_t* codes, uint8_t* scales, double emax) {
  const int B = 32;
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t b = 0; b < cols / B; b++) {
      const uint16_t* xb = x + r * cols + b * B;
      int64_t first = r * cols + b * B;
      int finite = 1;
      double amax = 0.0;
      for (int i = 0; i < B; i++) {
        if (!bf16_is_finite(xb[i])) finite = 0;
        double a = fabs(mxo_bf16_value(xb[i]));
        if (a > amax) amax = a;
      }
      if (!finite) {
        scales[r * (cols / B) + b] = 255;
        for (int i = 0; i < B; i++) put_code(codes, fmt, first + i, 0);
        continue;
      }
      int E = mxo_mx_scale_exponent(amax, emax);
      scales[r * (cols / B) + b] = (uint8_t)E;
      for (int i = 0; i < B; i++) {
        double v = ldexp(mxo_bf16_value(xb[i]), 127 - E); /* x / 2^(E-127) */
        uint8_t c = elem_encode(fmt, v);
        put_code(codes, fmt, first + i, c);
      }
    }
  }
}

/* Nearest-even E2M1 code of x / D for D > 0 without forming the quotient:
 * |x| is compared with each midpoint times D, all exact in double. */
static uint8_t e2m1_nearest_scaled(double x, double D) {
  double a = fabs(x);
  int c = 0;
  for (int k = 0; k < 7; k++) {
    double mid = (mxo_e2m1_value((uint8_t)k) + mxo_e2m1_value((uint8_t)(k + 1))) / 2.0 * D;
    if (a > mid || (a == mid && ((k + 1) & 1) == 0))
      c = k + 1;
    else
      break;
  }
  return (uint8_t)((signbit(x) ? 8 : 0) | c);
}

/* MBS-static macro mantissa (gist.science summary, section 2.B: a factor
 * 1 + m with 8 mantissa bits per macro block, computed directly from the
 * block maximum so that the outlier is normalised before the standard
 * quantization). n is found by search with exact products, as in the MX
 * rule; rho = alpha / 2^n is exact; m by search over the 8-bit grid. */
int mxo_mbs_macro_mantissa(double alpha) {
  if (!isfinite(alpha) || alpha == 0.0) return 0;
  int n = -300;
  while (!(alpha <= ldexp(6.0, n))) n++;
  const double rho = ldexp(alpha, -n);
  for (int m = 0; m < 256; m++)
    if (3.0 * (1.0 + m / 256.0) >= rho) return m;
  return 0; /* rho in (3 (1 + 255/256), 6]: already at the top of the grid */
}

/* MXFP4-MBS: per macro block of 128, the factor f from the macro amax; then
 * each base block of B elements (16, the summary's "1 x 16"; or 32, MXFP4's
 * own block) quantizes x / f by the MX rule with its own E8M0 exponent. The
 * scale search compares amax_b with (6 f) 2^n and the codes compare |x| with
 * midpoint * f * 2^(E-127): every product is exact in double, so x / f is
 * never rounded. */
static void quantize_mbs(int64_t rows, int64_t cols, int B, const uint16_t* x, uint8_t* codes,
                         uint8_t* scales) {
  const int64_t nb = cols / B, nm = cols / 128;
  uint8_t* macro = scales + rows * nb;
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t q = 0; q < nm; q++) {
      const uint16_t* xm = x + r * cols + q * 128;
      int finite = 1;
      double alpha = 0.0;
      for (int i = 0; i < 128; i++) {
        if (!bf16_is_finite(xm[i])) finite = 0;
        double a = fabs(mxo_bf16_value(xm[i]));
        if (a > alpha) alpha = a;
      }
      const int m = finite ? mxo_mbs_macro_mantissa(alpha) : 0;
      macro[r * nm + q] = (uint8_t)m;
      const double f = 1.0 + m / 256.0;
      for (int b = 0; b < 128 / B; b++) {
        const uint16_t* xb = xm + B * b;
        const int64_t first = r * cols + q * 128 + B * b;
        const int64_t sidx = r * nb + q * (128 / B) + b;
        int bfinite = 1;
        double amax = 0.0;
        for (int i = 0; i < B; i++) {
          if (!bf16_is_finite(xb[i])) bfinite = 0;
          double a = fabs(mxo_bf16_value(xb[i]));
          if (a > amax) amax = a;
        }
        if (!bfinite) {
          scales[sidx] = 255;
          for (int i = 0; i < B; i++) put_code(codes, MXO_FMT_MXFP4, first + i, 0);
          continue;
        }
        const int E = mxo_mx_scale_exponent(amax, 6.0 * f);
        scales[sidx] = (uint8_t)E;
        const double D = ldexp(f, E - 127);
        for (int i = 0; i < B; i++)
          put_code(codes, MXO_FMT_MXFP4, first + i, e2m1_nearest_scaled(mxo_bf16_value(xb[i]), D));
      }
    }
  }
}

/* NVFP4. The scales in fp32, one rounding per operation; the codes from the
 * exact quotient:
 *  1. T = max |x| over the tensor.
 *  2. s_t = T / 2688 (2688 = 6 * 448 maps T onto the largest E2M1 value times
 *     the largest E4M3 scale); T = 0 gives s_t = 1.
 *  3. per 16-block: s_b = E4M3 nearest-even, saturating, of amax_b / (6 s_t).
 *  4. s_b = 0 gives sign-only zero codes for the block.
 *  5. code = E2M1 nearest-even, saturating, of the exact quotient
 *     x / (s_b s_t) (the product is exact in double, and so is each midpoint
 *     times it); x = +-0 gives +-0.
 * A non-finite T gives s_t = NaN, NaN block scales and zero codes.
 * reciprocal != 0 replaces steps 4-5 by the fp32 sequence D = fl(s_b s_t),
 * D = 0 -> sign-only zeros, code = E2M1 of fl(x * fl(1 / D)) (information:
 * how often that cheaper form decides a code differently). */
static void quantize_nvfp4(int64_t rows, int64_t cols, const uint16_t* x,
                           uint8_t* codes, uint8_t* scales, float* tensor_scale,
                           int reciprocal) {
  const int B = 16;
  const int64_t n = rows * cols;
  float T = 0.0f;
  int finite = 1;
  for (int64_t i = 0; i < n; i++) {
    if (!bf16_is_finite(x[i])) finite = 0;
    float a = fabsf((float)mxo_bf16_value(x[i]));
    if (a > T) T = a;
  }
  if (!finite) {
    if (tensor_scale) *tensor_scale = NAN;
    for (int64_t b = 0; b < n / B; b++) scales[b] = 0x7F;
    for (int64_t i = 0; i < n; i++) put_code(codes, MXO_FMT_NVFP4, i, 0);
    return;
  }
  const float s_t = (T == 0.0f) ? 1.0f : T / 2688.0f;
  const float d6 = 6.0f * s_t;
  if (tensor_scale) *tensor_scale = s_t;
  for (int64_t b = 0; b < n / B; b++) {
    const uint16_t* xb = x + b * B;
    float bamax = 0.0f;
    for (int i = 0; i < B; i++) {
      float a = fabsf((float)mxo_bf16_value(xb[i]));
      if (a > bamax) bamax = a;
    }
    float r = bamax / d6;
    uint8_t sb = mxo_encode_e4m3((double)r);
    scales[b] = sb;
    const double sbv = mxo_e4m3_value(sb);
    const float D = (float)sbv * s_t;
    const float R = 1.0f / D;
    for (int i = 0; i < B; i++) {
      float xi = (float)mxo_bf16_value(xb[i]);
      uint8_t c;
      if (xi == 0.0f || (reciprocal ? D == 0.0f : sbv == 0.0)) {
        c = signbit(xi) ? 0x8 : 0x0;
      } else if (!reciprocal) {
        c = e2m1_nearest_scaled((double)xi, sbv * (double)s_t);
      } else {
        float q = xi * R;
        c = mxo_encode_e2m1((double)q);
      }
      put_code(codes, MXO_FMT_NVFP4, b * B + i, c);
    }
  }
}

int mxo_quantize(int fmt, int block, int64_t rows, int64_t cols,
                 const uint16_t* x, uint8_t* codes, uint8_t* scales,
                 float* tensor_scale) {
  if (rows <= 0 || cols <= 0 || !x || !codes || !scales) return MXO_ERR_ARG;
  if (fmt < MXO_FMT_MXFP4 || fmt > MXO_FMT_MXFP4_MBS16) return MXO_ERR_ARG;
  if (block != fmt_block(fmt) || cols % fmt_granule(fmt) != 0) return MXO_ERR_ARG;
  if (is_mbs(fmt)) {
    quantize_mbs(rows, cols, fmt_block(fmt), x, codes, scales);
    if (tensor_scale) *tensor_scale = 1.0f;
  } else if (is_mx(fmt)) {
    quantize_mx(fmt, rows, cols, x, codes, scales, elem_max(fmt));
    if (tensor_scale) *tensor_scale = 1.0f;
  } else {
    quantize_nvfp4(rows, cols, x, codes, scales, tensor_scale, 0);
  }
  return MXO_OK;
}

int mxo_quantize_nvfp4_reciprocal(int64_t rows, int64_t cols,
                                  const uint16_t* x, uint8_t* codes,
                                  uint8_t* scales, float* tensor_scale) {
  if (rows <= 0 || cols <= 0 || cols % 16 != 0 || !x || !codes || !scales)
    return MXO_ERR_ARG;
  quantize_nvfp4(rows, cols, x, codes, scales, tensor_scale, 1);
  return MXO_OK;
}

/* ------------------------------------------------------------------------ */
/* Dequantize                                                                 */
/* ------------------------------------------------------------------------ */

/* Exact dequantized value of element idx (row-major), in double.
 * MX: element value * 2^(E-127) (x_real = S * x_elem). NVFP4: e * s_b * s_t,
 * which needs at most 2 + 4 + 24 significant bits, so it is exact. MXFP4-MBS
 * (base block 32 or 16): e * 2^(E-127) * (1 + m / 256), m from the macro plane
 * `macro` ([rows][cols/128]; NULL for the other formats). */
static double exact_value(int fmt, const uint8_t* codes, const uint8_t* scales,
                          const uint8_t* macro, float ts, int64_t cols, int64_t idx) {
  int block = fmt_block(fmt);
  int64_t r = idx / cols, c = idx % cols;
  uint8_t sc = scales[r * (cols / block) + c / block];
  uint8_t code = get_code(codes, fmt, idx);
  double e = elem_value(fmt, code);
  if (fmt == MXO_FMT_NVFP4) return e * mxo_e4m3_value(sc) * (double)ts;
  if (is_mbs(fmt))
    return e * mxo_e8m0_value(sc) * (1.0 + macro[r * (cols / 128) + c / 128] / 256.0);
  return e * mxo_e8m0_value(sc);
}

int mxo_dequantize(int fmt, int block, int64_t rows, int64_t cols,
                   const uint8_t* codes, const uint8_t* scales,
                   float tensor_scale, int out_dtype, void* y) {
  if (rows <= 0 || cols <= 0 || !codes || !scales || !y) return MXO_ERR_ARG;
  if (fmt < MXO_FMT_MXFP4 || fmt > MXO_FMT_MXFP4_MBS16) return MXO_ERR_ARG;
  if (block != fmt_block(fmt) || cols % fmt_granule(fmt) != 0) return MXO_ERR_ARG;
  if (out_dtype != MXO_OUT_F32 && out_dtype != MXO_OUT_BF16) return MXO_ERR_ARG;
  const uint8_t* macro = is_mbs(fmt) ? scales + rows * (cols / fmt_block(fmt)) : NULL;
  for (int64_t i = 0; i < rows * cols; i++) {
    float f;
    if (fmt == MXO_FMT_NVFP4) {
      /* y = fl32(fl32(e * s_b) * s_t); the inner product is exact. */
      int64_t r = i / cols, c = i % cols;
      uint8_t sc = scales[r * (cols / block) + c / block];
      float es = (float)(mxo_e2m1_value(get_code(codes, fmt, i)) * mxo_e4m3_value(sc));
      f = es * tensor_scale;
    } else {
      f = (float)exact_value(fmt, codes, scales, macro, 1.0f, cols, i);
    }
    if (out_dtype == MXO_OUT_F32)
      ((float*)y)[i] = f;
    else
      ((uint16_t*)y)[i] = mxo_f32_to_bf16(f);
  }
  return MXO_OK;
}

/* ------------------------------------------------------------------------ */
/* GEMM over exactly dequantized operands                                     */
/* ------------------------------------------------------------------------ */

static void dequant_row(int fmt, const void* data, const uint8_t* scales,
                        const uint8_t* macro, float ts, int64_t K, int64_t row, double* out) {
  if (fmt == MXO_FMT_BF16) {
    const uint16_t* x = (const uint16_t*)data + row * K;
    for (int64_t k = 0; k < K; k++) out[k] = mxo_bf16_value(x[k]);
    return;
  }
  /* exact_value indexes the whole matrix; pass the row's element index. */
  for (int64_t k = 0; k < K; k++)
    out[k] = exact_value(fmt, (const uint8_t*)data, scales, macro, ts, K, row * K + k);
}

static int gemm_args_ok(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K,
                        const void* a, const uint8_t* a_scales, const void* b,
                        const uint8_t* b_scales) {
  if (M <= 0 || N <= 0 || K <= 0 || !a || !b) return 0;
  if (fmt_a < MXO_FMT_BF16 || fmt_a > MXO_FMT_MXFP4_MBS16) return 0;
  if (fmt_b < MXO_FMT_MXFP4 || fmt_b > MXO_FMT_MXFP4_MBS16) return 0;
  if (fmt_a != MXO_FMT_BF16 && (!a_scales || K % fmt_granule(fmt_a) != 0)) return 0;
  if (!b_scales || K % fmt_granule(fmt_b) != 0) return 0;
  return 1;
}

/* The macro plane of an MXFP4-MBS operand with `rows` rows, else NULL. */
static const uint8_t* macro_plane(int fmt, const uint8_t* scales, int64_t rows, int64_t K) {
  return is_mbs(fmt) ? scales + rows * (K / fmt_block(fmt)) : NULL;
}

static void dot_abs(const double* x, const double* y, int64_t K, double* c,
                    double* s) {
  double acc = 0.0, accabs = 0.0;
  for (int64_t k = 0; k < K; k++) {
    double p = x[k] * y[k];
    acc += p;
    accabs += fabs(p);
  }
  *c = acc;
  *s = accabs;
}

int mxo_gemm(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K,
             const void* a, const uint8_t* a_scales, float a_ts,
             const void* b, const uint8_t* b_scales, float b_ts,
             double* C, double* S) {
  if (!gemm_args_ok(fmt_a, fmt_b, M, N, K, a, a_scales, b, b_scales) || !C || !S)
    return MXO_ERR_ARG;
  double* bt = (double*)malloc(sizeof(double) * (size_t)(N * K));
  if (!bt) return MXO_ERR_ARG;
  const uint8_t* ma = macro_plane(fmt_a, a_scales, M, K);
  const uint8_t* mb = macro_plane(fmt_b, b_scales, N, K);
  int failed = 0;
  /* Rows are independent: each output entry is one sequential dot product,
   * whichever thread computes it, so the result does not depend on the
   * thread count. */
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < N; j++) dequant_row(fmt_b, b, b_scales, mb, b_ts, K, j, bt + j * K);
#pragma omp parallel reduction(| : failed)
  {
    double* ar = (double*)malloc(sizeof(double) * (size_t)K);
    if (!ar) failed = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; i++) {
      if (!ar) continue;
      dequant_row(fmt_a, a, a_scales, ma, a_ts, K, i, ar);
      for (int64_t j = 0; j < N; j++) dot_abs(ar, bt + j * K, K, &C[i * N + j], &S[i * N + j]);
    }
    free(ar);
  }
  free(bt);
  return failed ? MXO_ERR_ARG : MXO_OK;
}

int mxo_gemm_entries(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K,
                     const void* a, const uint8_t* a_scales, float a_ts,
                     const void* b, const uint8_t* b_scales, float b_ts,
                     int64_t n_entries, const int64_t* ii, const int64_t* jj,
                     double* C, double* S) {
  if (!gemm_args_ok(fmt_a, fmt_b, M, N, K, a, a_scales, b, b_scales) || !C || !S ||
      n_entries < 0 || (n_entries > 0 && (!ii || !jj)))
    return MXO_ERR_ARG;
  for (int64_t t = 0; t < n_entries; t++)
    if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N) return MXO_ERR_ARG;
  const uint8_t* ma = macro_plane(fmt_a, a_scales, M, K);
  const uint8_t* mb = macro_plane(fmt_b, b_scales, N, K);
  int failed = 0;
#pragma omp parallel reduction(| : failed)
  {
    double* ar = (double*)malloc(sizeof(double) * (size_t)K);
    double* br = (double*)malloc(sizeof(double) * (size_t)K);
    if (!ar || !br) failed = 1;
#pragma omp for schedule(dynamic, 16)
    for (int64_t t = 0; t < n_entries; t++) {
      if (!ar || !br) continue;
      dequant_row(fmt_a, a, a_scales, ma, a_ts, K, ii[t], ar);
      dequant_row(fmt_b, b, b_scales, mb, b_ts, K, jj[t], br);
      dot_abs(ar, br, K, &C[t], &S[t]);
    }
    free(ar);
    free(br);
  }
  return failed ? MXO_ERR_ARG : MXO_OK;
}

/* Threads the GEMM routines use (OpenMP's limit; 1 in a build without it). */
int mxo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Variants: overflow-aware scaling and the 32-point Walsh-Hadamard rotation */
/* ------------------------------------------------------------------------ */

int mxo_wht32(int64_t rows, int64_t cols, const uint16_t* x, uint16_t* y) {
  if (rows <= 0 || cols <= 0 || cols % 32 != 0 || !x || !y) return MXO_ERR_ARG;
  const float c = (float)(1.0 / sqrt(32.0));
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t b = 0; b < cols / 32; b++) {
      float v[32];
      for (int i = 0; i < 32; i++) v[i] = (float)mxo_bf16_value(x[r * cols + b * 32 + i]);
      for (int h = 1; h < 32; h *= 2) {
        for (int i = 0; i < 32; i++) {
          if (i & h) continue;
          const float a = v[i], d = v[i + h];
          v[i] = a + d;
          v[i + h] = a - d;
        }
      }
      for (int i = 0; i < 32; i++) {
        const float t = v[i] * c;
        y[r * cols + b * 32 + i] = mxo_f32_to_bf16(t);
      }
    }
  }
  return MXO_OK;
}

int mxo_quantize_ex(int fmt, int block, int rule, int rot, int64_t rows, int64_t cols,
                    const uint16_t* x, uint8_t* codes, uint8_t* scales) {
  if (rows <= 0 || cols <= 0 || !x || !codes || !scales) return MXO_ERR_ARG;
  if (fmt != MXO_FMT_MXFP4 && fmt != MXO_FMT_MXFP8) return MXO_ERR_ARG;
  if (block != 32 || cols % 32 != 0) return MXO_ERR_ARG;
  if (rule != MXO_RULE_CEIL && !(rule == MXO_RULE_OAS && fmt == MXO_FMT_MXFP4)) return MXO_ERR_ARG;
  if (rot != MXO_ROT_NONE && rot != MXO_ROT_WHT32) return MXO_ERR_ARG;
  const double emax = (fmt == MXO_FMT_MXFP8) ? 448.0 : (rule == MXO_RULE_OAS ? 7.0 : 6.0);
  if (rot == MXO_ROT_NONE) {
    quantize_mx(fmt, rows, cols, x, codes, scales, emax);
    return MXO_OK;
  }
  uint16_t* t = (uint16_t*)malloc((size_t)(rows * cols) * sizeof(uint16_t));
  if (!t) return MXO_ERR_ARG;
  mxo_wht32(rows, cols, x, t);
  quantize_mx(fmt, rows, cols, t, codes, scales, emax);
  free(t);
  return MXO_OK;
}
