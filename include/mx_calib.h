/*
 * mx_calib.h -- roofline calibration for libmx's measurements (library
 * libmx_calib.so, built beside libmx.so; not part of the quantize / GEMM path).
 *
 * The published MI355X peaks (FP4 10.1 PFLOP/s, bf16 and fp16 2.5 PFLOP/s,
 * dense) assume the top clock. Under a steady stream of matrix instructions
 * the chip lowers its clock to stay within its power limit, so a kernel that
 * does nothing else sets the ceiling any real kernel can reach. This call
 * measures it. Likewise the published HBM bandwidth (8 TB/s) is more than
 * plain streams of loads and stores sustain; mx_calib_stream measures those.
 */
#ifndef MX_CALIB_H
#define MX_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* mx_calib_mfma: on the current device, launch `workgroups` workgroups that
 * issue only back-to-back matrix instructions of one kind on register
 * operands filled with pseudo-random bits, `iters` rounds each, `reps` times in
 * a row on a stream of its own (at most 256), and report the steady state:
 * the median launch time of the second half, after the clock has settled.
 *   kind 0: v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands and E8M0
 *           scales, 4 waves per workgroup, 16 independent 32x32 tiles per
 *           wave (the MXFP4 GEMM's shape); 131072 FLOP per instruction.
 *   kind 1: v_mfma_f32_32x32x16_bf16, 8 waves per workgroup, 8 tiles per
 *           wave (the bf16-expansion GEMM's shape); 32768 FLOP each.
 *   kind 2: v_mfma_f32_32x32x16_f16, as kind 1.
 * steady_ms: that launch time in milliseconds; flop: FLOP per launch (both
 * host pointers, written on success). The call allocates and frees its own
 * device buffer and synchronizes; it is meant for measurement runs, not for
 * a serving path. Returns 0, or the hipError_t of the first failing HIP call
 * (-1 for an unknown kind or a non-positive count).
 */
int mx_calib_mfma(int kind, int workgroups, int iters, int reps, float* steady_ms, double* flop);

/* mx_calib_stream: on the current device, stream `bytes` of device memory
 * in 16-byte chunks (consecutive lanes on consecutive chunks) with
 * workgroups of 256 threads, each thread issuing `unroll` (1, 2, 4 or 8)
 * chunks' loads before their stores; `reps` launches in a row on a stream of
 * its own (at most 256); report the steady state as mx_calib_mfma does.
 *   kind 0: read `bytes` (folded into a value that no store depends on in
 *           practice);
 *   kind 1: write `bytes`;
 *   kind 2: copy `bytes` (read `bytes`, write `bytes`);
 *   kind 3: read `bytes`, write bytes / 4: one 4-byte store per 16-byte
 *           chunk read, the access pattern of a 4-bit quantizer of bf16.
 * workgroups > 0: that many workgroups loop over the data (grid stride);
 * workgroups = 0: one pass, each workgroup a contiguous run of 256 * unroll
 * chunks. nontemporal = 1: non-temporal loads and stores (0: plain).
 * Buffers of at least four times the 256 MB last-level cache measure HBM.
 * steady_ms: that launch time in ms; moved: bytes read plus written per
 * launch (both host pointers, written on success). bytes: a multiple of 64,
 * 4096 .. 2^36. The call allocates and frees its own device buffers (their
 * contents are never initialised: only their traffic counts) and
 * synchronizes. Returns 0, the hipError_t of the first failing HIP call, or
 * -1 for an unknown kind or an argument out of range.
 */
int mx_calib_stream(int kind, int64_t bytes, int workgroups, int unroll, int nontemporal, int reps,
                    float* steady_ms, double* moved);

#ifdef __cplusplus
}
#endif
#endif /* MX_CALIB_H */
