// Roofline calibration: matrix instructions alone, on register operands, at
// the tile shapes of the library's GEMMs (declared in include/mx_calib.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "mx_calib.h"

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Four waves, 4 x 4 tiles of 32 x 32 per wave, K = 64 per instruction: every
// E2M1 code random (both signs, all magnitudes), scales 2^0.
__global__ __launch_bounds__(256, 1) void mfma_fp4_only(float* out, int iters) {
  const uint32_t t = blockIdx.x * 256 + threadIdx.x;
  i32x8 a[4], b[4];
  for (int i = 0; i < 4; i++)
    for (int k = 0; k < 8; k++) {
      a[i][k] = k < 4 ? (int)mix(t * 64 + i * 8 + k) : 0;
      b[i][k] = k < 4 ? (int)mix(t * 64 + 32 + i * 8 + k) : 0;
    }
  f32x16 acc[4][4];
  for (int i = 0; i < 4; i++)
    for (int j = 0; j < 4; j++) acc[i][j] = f32x16{};
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, 127, 0, 127);
  }
  float s = 0.0f;
  for (int i = 0; i < 4; i++)
    for (int j = 0; j < 4; j++)
      for (int k = 0; k < 16; k++) s += acc[i][j][k];
  out[t] = s;
}

// Eight waves, 4 x 2 tiles per wave, K = 16 per instruction: bf16 or fp16
// operands with random mantissas and signs, exponents kept near 1.
template <bool F16>
__global__ __launch_bounds__(512, 1) void mfma_16bit_only(float* out, int iters) {
  const uint32_t t = blockIdx.x * 512 + threadIdx.x;
  u32x4 a[4], b[2];
  const uint32_t keep = F16 ? 0x83FF83FFu : 0x807F807Fu;  // sign and mantissa
  const uint32_t one = F16 ? 0x38003800u : 0x3F003F00u;   // exponent of 0.5 .. 1
  for (int i = 0; i < 4; i++)
    for (int k = 0; k < 4; k++) a[i][k] = (mix(t * 31 + i * 4 + k) & keep) | one;
  for (int i = 0; i < 2; i++)
    for (int k = 0; k < 4; k++) b[i][k] = (mix(t * 37 + 100 + i * 4 + k) & keep) | one;
  f32x16 acc[4][2];
  for (int i = 0; i < 4; i++)
    for (int j = 0; j < 2; j++) acc[i][j] = f32x16{};
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 2; j++) {
        if (F16)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[i]),
                                                            __builtin_bit_cast(f16x8, b[j]), acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                             __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
      }
  }
  float s = 0.0f;
  for (int i = 0; i < 4; i++)
    for (int j = 0; j < 2; j++)
      for (int k = 0; k < 16; k++) s += acc[i][j][k];
  out[t] = s;
}

}  // namespace

extern "C" int mx_calib_mfma(int kind, int workgroups, int iters, int reps, float* steady_ms, double* flop) {
  if (kind < 0 || kind > 2 || workgroups <= 0 || iters <= 0 || reps <= 0 || !steady_ms || !flop) return -1;
  const int threads = kind == 0 ? 256 : 512;
  float* out = nullptr;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipMalloc(&out, (size_t)workgroups * threads * sizeof(float));
  if (err == hipSuccess) err = hipStreamCreate(&s);
  if (err == hipSuccess) err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  float ms_all[256];
  reps = std::min(reps, 256);
  for (int r = 0; r < reps && err == hipSuccess; r++) {
    err = hipEventRecord(e0, s);
    if (err != hipSuccess) break;
    void* args[] = {&out, &iters};
    const void* f = kind == 0   ? (const void*)&mfma_fp4_only
                    : kind == 1 ? (const void*)&mfma_16bit_only<false>
                                : (const void*)&mfma_16bit_only<true>;
    err = hipLaunchKernel(f, dim3((unsigned)workgroups), dim3((unsigned)threads), args, 0, s);
    if (err == hipSuccess) err = hipEventRecord(e1, s);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    ms_all[r] = ms;
  }
  if (e1) (void)hipEventDestroy(e1);
  if (e0) (void)hipEventDestroy(e0);
  if (s) (void)hipStreamDestroy(s);
  if (out) (void)hipFree(out);
  if (err != hipSuccess) return (int)err;
  const double per_wave = kind == 0 ? 16.0 * 131072.0 : 8.0 * 32768.0;
  // steady state: the median of the second half of the launches
  std::sort(ms_all + reps / 2, ms_all + reps);
  *steady_ms = ms_all[reps / 2 + (reps - reps / 2) / 2];
  *flop = (double)workgroups * (threads / 64) * (double)iters * per_wave;
  return 0;
}
