/*
 * mx.h -- C ABI of libmx: microscaling (MX / NVFP4) block quantization and the
 * block-scaled GEMM on AMD Instinct MI355X (gfx950).
 *
 * Formats (pages: "Microscaling MXFP4/NVFP4 on Blackwell for reasoning LLMs",
 * section "Fundamentos matematicos do formato MXFP4 e E8M0" and its format
 * table; zubnet.ai summary, opening paragraph):
 *   MXFP4  E2M1 element codes, one E8M0 scale 2^(E-127) per 32 elements.
 *   MXFP8  E4M3 (OCP, max 448) element codes, one E8M0 scale per 32.
 *   NVFP4  E2M1 element codes, one E4M3 scale per 16 elements, plus one fp32
 *          scale for the whole tensor (x ~ e * s_b * s_t).
 *
 * Layouts (all row-major, blocks run along the contiguous "cols"/K axis):
 *   x       bf16 [rows][cols]
 *   codes   FP4: uint8 [rows][cols/2], element 2j in bits 3:0 of byte j and
 *                element 2j+1 in bits 7:4;   FP8: uint8 [rows][cols]
 *   scales  uint8 [rows][cols/block]: E8M0 exponent byte (MX) or E4M3 code
 *           (NVFP4)
 *   GEMM    A is M x K, B is stored N x K (the Linear weight layout, K
 *           contiguous), C is M x N with leading dimension ldc.
 *
 * Ownership and threading: every pointer is a device pointer owned by the
 * caller, unless stated otherwise. The library never allocates or frees
 * memory and never synchronizes. Work is enqueued on `stream` (a hipStream_t;
 * NULL is the default stream) and the call returns at once. Calls keep no state
 * between them and may be made from several threads at once.
 *
 * Errors: every argument is checked before anything is launched.
 *   MX_ERR_INVALID_ARG  null pointer, a size <= 0, cols or K not a multiple of
 *                       the block (of 128 for MXFP4_MBS), a pointer not
 *                       16-byte aligned, ldc < N, or
 *                       workspace_bytes below the size the call needs.
 *   MX_ERR_UNSUPPORTED  a format/block pair or format combination outside the
 *                       list below, a rounding mode other than MX_ROUND_RNE,
 *                       an unknown output dtype.
 *   MX_ERR_HIP          a HIP launch failed; mx_last_hip_error() returns the
 *                       hipError_t (per calling thread).
 * Nothing is printed and no C++ exception crosses this interface.
 */
#ifndef MX_H
#define MX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_FMT_BF16 = 0,  /* plain bf16 (only as the A operand of a W4A16 GEMM) */
  MX_FMT_MXFP4 = 1, /* E2M1 + E8M0 per 32 */
  MX_FMT_MXFP8 = 2, /* E4M3 + E8M0 per 32 */
  MX_FMT_NVFP4 = 3, /* E2M1 + E4M3 per 16 + fp32 tensor scale */
  MX_FMT_MXFP8_E5M2 = 4, /* E5M2 + E8M0 per 32 (the OCP MXFP8 alternative) */
  MX_FMT_MXFP6_E3M2 = 5, /* E3M2 + E8M0 per 32; 6-bit codes, element i of a row
                            in bits 6i .. 6i+5 of the row's bytes (little-endian),
                            3 cols / 4 bytes per row */
  MX_FMT_MXFP4_MBS = 6,  /* MXFP4 with static macro-block scaling over MXFP4's
                            own 32-element blocks (a reading: base block 32):
                            E2M1 + E8M0 per 32, plus one 8-bit macro mantissa
                            m per 128 (factor 1 + m/256); cols must be a
                            multiple of 128. scales = two planes in one
                            buffer: the E8M0 bytes [rows][cols/32], then the
                            macro bytes [rows][cols/128] */
  MX_FMT_MXFP4_MBS16 = 7 /* static macro-block scaling as the gist.science
                            summary prints it (section 2.B): E2M1 codes, one
                            E8M0 scale per 1 x 16 base block, one 8-bit macro
                            mantissa per 1 x 128 (block 16, cols a multiple of
                            128). scales = the E8M0 bytes [rows][cols/16],
                            then the macro bytes [rows][cols/128] */
} mx_format;

typedef enum { MX_ROUND_RNE = 0 } mx_round; /* nearest, ties to even */

typedef enum { MX_OUT_F32 = 0, MX_OUT_BF16 = 1 } mx_dtype;

typedef enum {
  MX_OK = 0,
  MX_ERR_INVALID_ARG = 1,
  MX_ERR_UNSUPPORTED = 2,
  MX_ERR_HIP = 3
} mx_status;

/*
 * Block quantization (the shared-exponent rule of the FAQ on the
 * produtoramaxvision page; x_real = 2^(E-127) * x_elem).
 *   MXFP4/MXFP8/MXFP6 (block 32): per block, E = ceil(log2(amax / emax))
 *     + 127 clamped to [0, 254] with emax = 6 (E2M1), 448 (E4M3), 57344
 *     (E5M2) or 28 (E3M2; E5M2 and E3M2 as named by the zubnet.ai summary and
 *     the produtoramaxvision format table, fields as in the OCP formats), evaluated
 *     exactly from the bf16 bits of amax; each element is x / 2^(E-127)
 *     rounded to nearest-even with saturation, sign copied (-0 stays -0).
 *     A block holding Inf/NaN gets scale 255 (E8M0 NaN) and zero codes.
 *   MXFP4_MBS (block 32; the static macro-block scaling of the gist.science
 *     summary of "Unveiling the Potential of Quantization with MXFP4",
 *     section 2.B): per macro block of 128 with amax alpha, n = the smallest
 *     integer with alpha <= 6 * 2^n, rho = alpha / 2^n, and m = the smallest
 *     integer >= 0 with 3 (1 + m/256) >= rho (m = 256 becomes 0; a zero or
 *     non-finite alpha gives 0); f = 1 + m/256. Each 32-block then gets
 *     E = the smallest n with amax_b <= 6 f 2^n, plus 127, clamped to [0, 254],
 *     and codes = nearest-even E2M1 of x / (f 2^(E-127)) with saturation, the
 *     sign copied; a 32-block holding Inf/NaN gets 255 and zero codes. The
 *     element's value is e * 2^(E-127) * f.
 *   NVFP4 (block 16), the scales in fp32 with one rounding per step:
 *     T = max|x| over the tensor; s_t = T / 2688 (1 if T = 0);
 *     s_b = E4M3(amax_b / (6 s_t)) nearest-even, saturating at 448;
 *     code = the E2M1 value nearest the exact quotient x / (s_b * s_t), ties
 *     to the even code, saturating; a zero x or s_b = 0 gives a signed zero
 *     code. Non-finite T: s_t = NaN, every block scale 0x7F (E4M3 NaN),
 *     every code 0.
 * x: bf16 [rows][cols]; codes, scales: outputs as in the layout above.
 * tensor_scale: NVFP4 only, one device fp32 written with s_t; NULL otherwise.
 * workspace: NVFP4 only, device scratch of at least
 *   mx_quantize_workspace_bytes(...) bytes (contents need no initialization);
 *   may be NULL with workspace_bytes 0 for MX formats.
 */
mx_status mx_quantize(mx_format fmt, int block, mx_round rnd, int64_t rows, int64_t cols,
                      const void* x, void* codes, void* scales, float* tensor_scale,
                      void* workspace, size_t workspace_bytes, void* stream);

size_t mx_quantize_workspace_bytes(mx_format fmt, int64_t rows, int64_t cols);

/* Scale rule and rotation variants of MX quantization (MXFP4 / MXFP8). */
typedef enum {
  MX_SCALE_CEIL = 0, /* the rule above: scaled block amax in (3, 6] for E2M1 */
  MX_SCALE_OAS = 1   /* overflow-aware scaling, MXFP4 only (gist.science
                        summary of "Unveiling the Potential of Quantization
                        with MXFP4", section 2.A): E = ceil(log2(amax / 7))
                        + 127, so the scaled amax lies in (3.5, 7] and
                        elements in (6, 7] saturate to 6 */
} mx_scale_rule;

typedef enum {
  MX_ROTATE_NONE = 0,
  MX_ROTATE_WHT32 = 1 /* each 32-block x is first replaced by
                         bf16(fl32(fl32(H32 x) * fl32(1/sqrt(32)))), H32 the
                         Sylvester Walsh-Hadamard matrix, H x by the fp32
                         radix-2 butterfly with spans 1, 2, 4, 8, 16 (pair
                         (i, i+h) -> (x_i + x_{i+h}, x_i - x_{i+h})); the
                         Hadamard rotation of the produtoramaxvision page,
                         section "Tecnicas de preservacao de acuracia: QuaRot,
                         SpinQuant e ReSET". Rotating both GEMM operands along
                         K leaves A * B^T unchanged up to rounding, since
                         (H/sqrt 32)(H/sqrt 32)^T = I. */
} mx_rotation;

/*
 * Operand layout for the GEMMs. The pages fix no memory layout; this one is
 * for HBM and cache locality on MI355X. MX_LAYOUT_ROWS is mx_quantize's:
 * codes [rows][cols * bits / 8], scales [rows][cols / block].
 * MX_LAYOUT_KPANEL cuts K into panels of W elements, W = 256 for MXFP4 and
 * W = 64 for MXFP8, MXFP8_E5M2, MXFP6_E3M2 and NVFP4 (one K step of that
 * format's GEMM), and stores each panel's rows back to back. With
 * wb = W * bits / 8 code bytes (MXFP4 128, MXFP8 and E5M2 64, E3M2 48,
 * NVFP4 32) and sb = W / block scale bytes (MXFP4 8, MXFP8, E5M2 and E3M2 2,
 * NVFP4 4) per row and panel:
 *   codes   [cols/W][rows][wb]: the code bytes of row r in panel p (elements
 *           W p .. W p + W - 1, packed as in MX_LAYOUT_ROWS) at byte
 *           (p * rows + r) * wb;
 *   scales  [cols/W][rows][sb]: byte (p * rows + r) * sb + j is the scale of
 *           block (W / block) p + j of row r.
 * The NVFP4 tensor scale is the same in both layouts. A GEMM step then reads
 * one contiguous range per operand tile instead of one short piece per row
 * spread over the whole matrix: on the MXFP4 MLP-down shape the GEMM runs
 * ~10% faster with K-panel weights, ~3% more with K-panel activations; the
 * MXFP8 / NVFP4 / E5M2 / E3M2 GEMMs of the QKV and MLP-up shapes 6-12%
 * faster with both operands in K panels. mx_pack re-lays a tensor;
 * mx_quantize_layout (any of these formats) and mx_quantize_ex (MXFP4,
 * MXFP8) write one directly.
 */
typedef enum {
  MX_LAYOUT_ROWS = 0,
  MX_LAYOUT_KPANEL = 1
} mx_layout;

/*
 * mx_quantize with a scale rule, a rotation and an output layout: MXFP4 and
 * MXFP8 (block 32) only; MX_SCALE_OAS with MXFP8, or another format, returns
 * MX_ERR_UNSUPPORTED. layout MX_LAYOUT_ROWS gives mx_quantize's layout;
 * MX_LAYOUT_KPANEL writes the same codes and scales in K panels and needs
 * cols a multiple of the panel width W, cols / W <= 65535 and
 * rows * (code bytes of a row) < 2^31 (MX_ERR_INVALID_ARG otherwise).
 * tensor_scale is not taken and no workspace is used. (MX_SCALE_CEIL,
 * MX_ROTATE_NONE, MX_LAYOUT_ROWS) is mx_quantize.
 */
mx_status mx_quantize_ex(mx_format fmt, int block, mx_round rnd, mx_scale_rule rule,
                         mx_rotation rot, int64_t rows, int64_t cols, const void* x,
                         void* codes, void* scales, void* stream, mx_layout layout);

/*
 * mx_quantize with an output layout: the same arguments, results and errors
 * as mx_quantize, with the codes and scales written in `layout`.
 * MX_LAYOUT_KPANEL (MXFP4, MXFP8, MXFP8_E5M2, MXFP6_E3M2 and NVFP4; the MBS
 * formats return MX_ERR_UNSUPPORTED) needs cols a multiple of the panel width
 * W, cols / W <= 65535 and rows * (code bytes of a row) < 2^31
 * (MX_ERR_INVALID_ARG otherwise); the codes, scales and NVFP4 tensor scale
 * are mx_quantize's, re-laid (mx_pack of mx_quantize's output gives the same
 * bytes). MX_LAYOUT_ROWS is mx_quantize.
 */
mx_status mx_quantize_layout(mx_format fmt, int block, mx_round rnd, int64_t rows, int64_t cols,
                             const void* x, void* codes, void* scales, float* tensor_scale,
                             void* workspace, size_t workspace_bytes, void* stream,
                             mx_layout layout);

/*
 * Dequantization (x_real = S * x_elem on the produtoramaxvision page): MX
 * y = val(code) * 2^(E-127); MXFP4_MBS y = val(code) * 2^(E-127) * (1 + m/256);
 * NVFP4 y = fl32(fl32(val(code) * s_b) * s_t).
 * The fp32 value is the output for MX_OUT_F32; MX_OUT_BF16 rounds it to bf16,
 * nearest-even (overflow gives Inf; E = 255 or an E4M3 NaN scale gives NaN).
 * tensor_scale: NVFP4 only, device pointer to one fp32; NULL otherwise.
 * y: [rows][cols] fp32 or bf16.
 */
mx_status mx_dequantize(mx_format fmt, int block, mx_round rnd, int64_t rows, int64_t cols,
                        const void* codes, const void* scales, const float* tensor_scale,
                        mx_dtype out_dtype, void* y, void* stream);

/*
 * Block-scaled GEMM, C = A * B^T over the dequantized operands, fp32
 * accumulation (the block-scaled dot product of the produtoramaxvision page,
 * section "Arquitetura Blackwell SM100 e aceleracao nativa de NVFP4": scales
 * are applied during FP32 accumulation, with no up-conversion of the operands).
 * Supported (fmt_a, fmt_b, block):
 *   (MXFP4, MXFP4, 32)  W4A4 on the FP4 scaled MFMA (codes and E8M0 scales go
 *                       to the matrix core as stored)
 *   (MXFP8, MXFP8, 32)  W8A8: e * 2^(E-127) is exact in bf16 and runs on the
 *                       bf16 MFMA (the FP8 scaled MFMA truncates block sums
 *                       beyond the accuracy bound below)
 *   (NVFP4, NVFP4, 16)  W4A4 with E4M3 block scales; e * s_b is exact in bf16,
 *                       so the product runs on bf16 MFMA and s_t^A * s_t^B is
 *                       applied to the fp32 result
 *   (MXFP8_E5M2, MXFP8_E5M2, 32) and (MXFP6_E3M2, MXFP6_E3M2, 32): exact
 *                       bf16 expansion on the bf16 MFMA, as for MXFP8 (these
 *                       need 256 * (bytes per code row) < 2^31, else
 *                       MX_ERR_INVALID_ARG)
 *   (MXFP4_MBS, MXFP4_MBS, 32) and (MXFP4_MBS16, MXFP4_MBS16, 16)  K a
 *                       multiple of 128: per macro block the FP4 scaled MFMA
 *                       gives the E8M0-scaled partial sum P (for 16-element
 *                       base blocks two MFMAs per 32 K, one per half) and the
 *                       vector ALU adds P * f_A * f_B (f_A f_B exact in fp32)
 *                       to the accumulator
 *   (BF16,  MXFP4, 32)  W4A16: bf16 activations times MXFP4 weights expanded
 *                       exactly to bf16 (weight-only quantization)
 * a: codes (or bf16 for MX_FMT_BF16) [M][...]; a_scales [M][K/block] (NULL for
 * BF16; for MXFP4_MBS / MBS16 the two-plane buffer of mx_quantize); a_ts,
 * b_ts: NVFP4 tensor scales (device fp32), NULL otherwise.
 * b: codes [N][...]; b_scales [N][K/block] (two planes for MXFP4_MBS / MBS16).
 * c: [M][ldc] fp32 or bf16 (rnd rounds the bf16 epilogue).
 * workspace: device scratch of at least mx_gemm_workspace_bytes(...) bytes
 * (may be NULL when that is 0).
 * K must be a multiple of 32 for every pair, and at most 65536 for W4A16;
 * other shapes return MX_ERR_INVALID_ARG.
 * Accuracy. With S_ij = sum_k |a_ik b_jk| over the dequantized operands, an
 * fp32 output errs from the exact sum by at most (L + c + n - 1) * 2^-24 *
 * S_ij: every fp32 step rounds once, the output's K is cut into n
 * accumulator chains of at most L = 48 steps (matrix instructions; macro
 * blocks for MBS; L = 32 and n = the K-splits of 2048 for W4A16) added in a
 * fixed order, and c <= 4 counts the roundings inside one step (the partial
 * sum of an MBS macro block; the NVFP4 tensor-scale product; W4A16's two
 * chains per split). That is within 2^-18 * S_ij, the bound of the pages'
 * target, even when every rounding goes the same way, for K <= 52224
 * (MXFP4: chains of 3072 K), 13056 (MXFP8, E5M2, MXFP6: 768 K), 12288
 * (NVFP4), 92160 (MBS: 6144 K), 79872 (MBS16) and 65536 (W4A16).
 * A bf16 output rounds an fp32 value once more (within 2^-8 * |C_ij|); on the
 * 256 x 256-tile kernels that value is one chain over all of K (K / 64 steps
 * for MXFP4, K / 16 for the 16-bit paths, K / 128 for MBS), so before that
 * rounding it errs by at most (steps + c) * 2^-24 * S_ij. Conditions: no
 * product or partial sum leaves fp32's range; below 2^-126 each fp32 step may
 * lose up to 2^-150 (K * 2^-149 in all); and for MXFP8 / E5M2 / MXFP6
 * operands whose E8M0 byte is at most 2, e * 2^(E-127) must lie on the bf16
 * grid (multiples of 2^-133) to be expanded exactly -- every code mx_quantize
 * writes from bf16 input does.
 */
mx_status mx_gemm(mx_format fmt_a, mx_format fmt_b, int block, mx_round rnd,
                  int64_t M, int64_t N, int64_t K,
                  const void* a, const void* a_scales, const float* a_ts,
                  const void* b, const void* b_scales, const float* b_ts,
                  mx_dtype out_dtype, void* c, int64_t ldc,
                  void* workspace, size_t workspace_bytes, void* stream);

size_t mx_gemm_workspace_bytes(mx_format fmt_a, mx_format fmt_b, int64_t M, int64_t N, int64_t K);

/*
 * Re-lays a quantized tensor from MX_LAYOUT_ROWS into MX_LAYOUT_KPANEL: a
 * byte permutation, no arithmetic. fmt must be MXFP4, MXFP8, MXFP8_E5M2,
 * MXFP6_E3M2 (block 32) or NVFP4 (block 16) (MX_ERR_UNSUPPORTED otherwise);
 * rows > 0 and cols a positive multiple of the panel width W with
 * cols / W <= 65535 and rows * (code bytes of a row) < 2^31
 * (MX_ERR_INVALID_ARG otherwise). The NVFP4 tensor scale needs no re-laying.
 * codes / scales
 * are the input (sizes as in mx_quantize), packed_codes / packed_scales the
 * output of the same sizes; input and output must not overlap. All pointers
 * 16-byte aligned device pointers.
 */
mx_status mx_pack(mx_format fmt, int block, int64_t rows, int64_t cols, const void* codes,
                  const void* scales, void* packed_codes, void* packed_scales, void* stream);

/*
 * mx_gemm with the layouts of the operands given. (MX_LAYOUT_ROWS,
 * MX_LAYOUT_ROWS) is exactly mx_gemm. MX_LAYOUT_KPANEL (codes and scales as
 * written by mx_pack, mx_quantize_layout or mx_quantize_ex) is supported
 * for A and / or B of (MXFP4, MXFP4, 32) on the 256 x 256-tile kernel: K a
 * multiple of 256, (M + 256) * K / 2 and (N + 256) * K / 2 below 2^31, and
 * K / 256 <= 65535; and for both A and B of (MXFP8, MXFP8, 32),
 * (MXFP8_E5M2, MXFP8_E5M2, 32), (MXFP6_E3M2, MXFP6_E3M2, 32) and
 * (NVFP4, NVFP4, 16) on the large-tile 16-bit kernel: K a multiple of 64,
 * K / 64 <= 65535, M and N times the code bytes of a row below 2^31 and
 * 256 times them below 2^31 (MX_ERR_UNSUPPORTED for other pairs or a single
 * K-panel operand of those, MX_ERR_INVALID_ARG for other shapes). The results
 * are bit-identical to mx_gemm on the same operands in MX_LAYOUT_ROWS.
 */
mx_status mx_gemm_ex(mx_format fmt_a, mx_format fmt_b, int block, mx_round rnd,
                     int64_t M, int64_t N, int64_t K,
                     const void* a, const void* a_scales, const float* a_ts,
                     const void* b, const void* b_scales, const float* b_ts,
                     mx_dtype out_dtype, void* c, int64_t ldc,
                     void* workspace, size_t workspace_bytes, void* stream,
                     mx_layout a_layout, mx_layout b_layout);

/*
 * mx_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments and results as mx_gemm without the workspace. Where mx_gemm
 * needs one (mx_gemm_workspace_bytes > 0: the W4A16 pair's split-K partials),
 * this call uses the library's own scratch instead: a fixed array of
 * 8 MiB (8388608 bytes) of device memory per GPU, which each GPU the library
 * runs on holds until the process ends (its address is looked up once per
 * device, on the first call with that device current). A shape that would
 * need more returns MX_ERR_INVALID_ARG; for the W4A16 pair that is
 * 4 * M * N * ceil(K / 2048) > 8388608, so the 16-token decode shape with
 * N = 28672 and K = 8192 (7.34 MB) fits. The call makes no hipMalloc, hipFree
 * or other allocating call. Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (several streams or threads at once) race and
 * must be serialized by the caller; the scratch needs no clearing, since each
 * call writes every partial it reads.
 */
mx_status mx_gemm_noalloc(mx_format fmt_a, mx_format fmt_b, int block, mx_round rnd,
                          int64_t M, int64_t N, int64_t K,
                          const void* a, const void* a_scales, const float* a_ts,
                          const void* b, const void* b_scales, const float* b_ts,
                          mx_dtype out_dtype, void* c, int64_t ldc, void* stream);

/* hipError_t saved by the last MX_ERR_HIP returned on the calling thread. */
int mx_last_hip_error(void);

/* Static, human-readable name of a status. */
const char* mx_status_string(mx_status s);

#ifdef __cplusplus
}
#endif
#endif /* MX_H */
