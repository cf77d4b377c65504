/*
 * mx_oracle.h -- plain CPU reference ("oracle") for microscaling block
 * quantization (MXFP4, MXFP8, NVFP4) and the block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this library. The GPU
 * library shares no code, header, table or constant with it, and never calls it.
 *
 * Every routine works on host memory, computes in double unless a reading
 * fixes fp32 (the NVFP4 tensor and block scales), and is written for
 * clarity, not speed.
 *
 * Sources (web pages on microscaling formats):
 *  - "Microscaling MXFP4/NVFP4 on Blackwell for reasoning LLMs"
 *    (produtoramaxvision.com.br), sections "Fundamentos matematicos do formato
 *    MXFP4 e E8M0" (E2M1 layout and value set, E8M0 = 2^(E-127),
 *    x_real = S * x_elem, 4.25 effective bits), the format table (FP8 E4M3
 *    range +-448, NVFP4 row) and the FAQ answer on the shared exponent
 *    (E = ceil(log2(max|x| / max_E2M1)) + 127).
 *  - zubnet.ai news summary: NVFP4 = E2M1 in 16-element blocks; MXFP8 =
 *    E4M3/E5M2 in 32-element blocks (the OCP FP8 formats).
 *  - produtoramaxvision format table: MXFP6 = E3M2 elements with an E8M0
 *    scale per 32, 6.25 bits per element.
 *  - gist.science summary of "Unveiling the Potential of Quantization with
 *    MXFP4", section 2.A: the standard MX rule maps the block amax into (3, 6];
 *    NVFP4 scales carry a mantissa; overflow-aware scaling (OAS) widens the
 *    scaled-amax range to (3.5, 7].
 *  - the same gist.science summary, section 2.B: macro-block scaling (MBS)
 *    adds a scale factor 1 + m with an 8-bit mantissa per 1 x 128 macro
 *    block, computed in the static variant directly from the block maximum
 *    to normalise outliers before the standard quantization.
 *  - produtoramaxvision page, section "Tecnicas de preservacao de acuracia:
 *    QuaRot, SpinQuant e ReSET": Hadamard / Walsh-Hadamard rotations spread
 *    a block's energy evenly over its 32 elements.
 */
#ifndef MX_ORACLE_H
#define MX_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Format identifiers (numbered like the GPU library's, but defined here
 * independently). */
enum {
  MXO_FMT_BF16 = 0,  /* plain bf16, no scales (activation side of W4A16) */
  MXO_FMT_MXFP4 = 1, /* E2M1 codes, one E8M0 scale per 32 elements */
  MXO_FMT_MXFP8 = 2, /* E4M3 codes, one E8M0 scale per 32 elements */
  MXO_FMT_NVFP4 = 3, /* E2M1 codes, one E4M3 scale per 16, fp32 tensor scale */
  MXO_FMT_MXFP8_E5M2 = 4, /* E5M2 codes, one E8M0 scale per 32 */
  MXO_FMT_MXFP6_E3M2 = 5, /* E3M2 codes (6 bits, packed), one E8M0 scale per 32 */
  MXO_FMT_MXFP4_MBS = 6,  /* MBS-static over MXFP4's 32-element E8M0 blocks (a
                             reading: base block 32) */
  MXO_FMT_MXFP4_MBS16 = 7 /* MBS-static as the gist.science summary prints it:
                             E2M1 codes, one E8M0 per 16-element base block,
                             one 8-bit macro mantissa per 128 */
};
enum { MXO_OUT_F32 = 0, MXO_OUT_BF16 = 1 };
enum { MXO_OK = 0, MXO_ERR_ARG = 1 };

/* ---- element and scale formats (decoded from their bit-field definitions) */
double mxo_bf16_value(uint16_t bits);
double mxo_e2m1_value(uint8_t code);  /* low 4 bits used */
double mxo_e4m3_value(uint8_t code);  /* 0x7F / 0xFF -> NaN */
double mxo_e8m0_value(uint8_t e);     /* 255 -> NaN */
double mxo_e5m2_value(uint8_t code);  /* exponent 31: Inf (mantissa 0) or NaN */
double mxo_e3m2_value(uint8_t code);  /* low 6 bits used; no Inf or NaN */

/* Nearest representable value, ties to the even code, saturating at the
 * largest magnitude; the sign bit of v is copied (so -0 encodes as -0). */
uint8_t mxo_encode_e2m1(double v);
uint8_t mxo_encode_e4m3(double v);
uint8_t mxo_encode_e5m2(double v);
uint8_t mxo_encode_e3m2(double v);

/* Round a float to bf16, nearest-even (NaN stays NaN, overflow goes to Inf). */
uint16_t mxo_f32_to_bf16(float f);

/* MX shared exponent for a block amax: the smallest integer n with
 * amax <= emax * 2^n, biased by 127 and clamped to [0, 254]; 255 (NaN) for a
 * non-finite amax. emax = 6 (E2M1) or 448 (E4M3). */
int mxo_mx_scale_exponent(double amax, double emax);

/* MBS-static macro mantissa m (0..255, factor f = 1 + m / 256) of a macro
 * block with amax alpha: with n the smallest integer such that
 * alpha <= 6 * 2^n and rho = alpha / 2^n (in (3, 6]), m is the smallest
 * integer >= 0 with 3 f >= rho, so that alpha / f lies in
 * (6 (1 - 2^-8), 6] * 2^(n-1), the top of the E2M1 grid one binade down;
 * m = 256 (rho within 2^-8 of 6 already) becomes 0. alpha = 0 or non-finite
 * gives 0. */
int mxo_mbs_macro_mantissa(double alpha);

/* Bytes of codes + scales (+4 for the NVFP4 tensor scale, + one macro byte
 * per 128 elements for MXFP4-MBS and MXFP4-MBS16). */
int64_t mxo_storage_bytes(int fmt, int64_t rows, int64_t cols);

/* ---- tensor operations, row-major, blocks along cols ------------------- */
/* x: bf16 bits [rows][cols]; codes: [rows][cols/2] (FP4, even element in the
 * low nibble), [rows][cols] (FP8) or [rows][3 cols/4] (FP6: element i of a row
 * in bits 6i .. 6i+5 of the row's bytes, little-endian); scales: [rows][cols/block] bytes;
 * tensor_scale: NVFP4 only (written), may be NULL otherwise.
 * NVFP4 (block 16): s_t = fl(T / 2688) for the tensor amax T (T = 0 -> 1);
 * s_b = E4M3 nearest-even, saturating, of fl(amax_b / fl(6 s_t)); each code
 * the nearest-even E2M1 value of the exact quotient x / (s_b s_t),
 * saturating, sign copied (s_b = 0: sign-only zeros); a non-finite T gives
 * s_t = NaN, every scale 0x7F and every code 0.
 * MXFP4-MBS16 (block 16) and MXFP4-MBS (block 32), cols a multiple of 128:
 * codes as MXFP4; scales holds two planes, the E8M0 bytes [rows][cols/block]
 * followed by the macro mantissas [rows][cols/128]. Per macro block of 128:
 * m = mxo_mbs_macro_mantissa(amax) (0 if the macro block holds Inf or NaN),
 * f = 1 + m / 256; per base block: E = smallest n with amax_b <= 6 f 2^n, plus
 * 127, clamped to [0, 254], and each code the nearest-even E2M1 value of
 * x / (f 2^(E-127)), saturating, sign copied; a base block holding Inf or NaN
 * gets E = 255 and zero codes. The dequantized value is e * 2^(E-127) * f. */
int mxo_quantize(int fmt, int block, int64_t rows, int64_t cols,
                 const uint16_t* x, uint8_t* codes, uint8_t* scales,
                 float* tensor_scale);

/* Variants of MX quantization (MXFP4 / MXFP8, block 32):
 *  rule: MXO_RULE_CEIL -- the standard rule above;
 *        MXO_RULE_OAS  -- MXFP4 only: E = smallest n with amax <= 7 * 2^n
 *                         (+127, clamped), so the scaled amax lies in
 *                         (3.5, 7] and values in (6, 7] saturate to 6.
 *  rot:  MXO_ROT_NONE, or MXO_ROT_WHT32 -- every 32-block is first replaced by
 *        bf16(fl32(fl32(H x) * fl32(1/sqrt(32)))), see mxo_wht32. */
enum { MXO_RULE_CEIL = 0, MXO_RULE_OAS = 1 };
enum { MXO_ROT_NONE = 0, MXO_ROT_WHT32 = 1 };
int mxo_quantize_ex(int fmt, int block, int rule, int rot, int64_t rows, int64_t cols,
                    const uint16_t* x, uint8_t* codes, uint8_t* scales);

/* 32-point Walsh-Hadamard rotation of every 32-element block of bf16 rows:
 * y = bf16(fl32(fl32(H32 x) * c)), c = fl32(1/sqrt(32)), H32 the Sylvester
 * matrix (H[i][j] = (-1)^popcount(i & j)), computed in fp32 by the radix-2
 * butterfly with spans 1, 2, 4, 8, 16, each pair (i, i + h) becoming
 * (x_i + x_{i+h}, x_i - x_{i+h}). */
int mxo_wht32(int64_t rows, int64_t cols, const uint16_t* x, uint16_t* y);

/* NVFP4 only, information: codes from the fp32 sequence D = fl(s_b * s_t),
 * code = E2M1(fl(x * fl(1 / D))) instead of the exact quotient
 * x / (s_b * s_t); scales are as mxo_quantize's. */
int mxo_quantize_nvfp4_reciprocal(int64_t rows, int64_t cols,
                                  const uint16_t* x, uint8_t* codes,
                                  uint8_t* scales, float* tensor_scale);

/* y: float [rows][cols] (MXO_OUT_F32) or bf16 bits (MXO_OUT_BF16). */
int mxo_dequantize(int fmt, int block, int64_t rows, int64_t cols,
                   const uint8_t* codes, const uint8_t* scales,
                   float tensor_scale, int out_dtype, void* y);

/* C[i][j] = sum_k a[i][k] * b[j][k] and S[i][j] = sum_k |a[i][k] * b[j][k]|,
 * both in double, over exactly dequantized operands. A is M x K (fmt_a;
 * MXO_FMT_BF16 means bf16 bits, no scales), B is stored N x K (fmt_b). */
int mxo_gemm(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K,
             const void* a, const uint8_t* a_scales, float a_ts,
             const void* b, const uint8_t* b_scales, float b_ts,
             double* C, double* S);

/* Same definition, only for the listed (ii[t], jj[t]) output entries. */
int mxo_gemm_entries(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K,
                     const void* a, const uint8_t* a_scales, float a_ts,
                     const void* b, const uint8_t* b_scales, float b_ts,
                     int64_t n_entries, const int64_t* ii, const int64_t* jj,
                     double* C, double* S);

/* Threads the two GEMM routines above run on (OpenMP over output rows or
 * entries; every entry is still one sequential double-precision loop, so the
 * results do not depend on the count). */
int mxo_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif /* MX_ORACLE_H */
