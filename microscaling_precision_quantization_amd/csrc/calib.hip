// Roofline calibration (declared in include/mx_calib.h): matrix instructions
// alone, on register operands, at the tile shapes of the library's GEMMs; and
// plain HBM streams of 16-byte loads and stores.
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

// HBM streams of 16-byte chunks, consecutive lanes on consecutive chunks,
// each thread issuing U chunks' loads before their stores.
//  KIND 0: read n chunks of src and XOR-fold them (a store that depends on
//          the folded value and practically never fires keeps the loads);
//  KIND 1: write n chunks of dst;
//  KIND 2: copy n chunks from src to dst;
//  KIND 3: read n chunks of src, write n dwords of dst (each the XOR of its
//          chunk): 4 bytes read per byte written, one 4-byte store per
//          16-byte load, as a 4-bit quantizer of bf16 input does.
// BLOCKED: one pass, workgroup w taking chunks 256 U w .. 256 U (w + 1) - 1;
// otherwise a grid-stride loop over the fixed grid. NT: non-temporal loads
// and stores.
template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}
template <bool NT, typename T>
__device__ __forceinline__ void st(T* p, T v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

template <int KIND, bool NT>
__device__ __forceinline__ void stream_put(u32x4* __restrict__ dst, int64_t i, const u32x4& x, u32x4& acc) {
  if (KIND == 0)
    acc ^= x;
  else if (KIND == 3)
    st<NT>((uint32_t*)dst + i, x.x ^ x.y ^ x.z ^ x.w);
  else
    st<NT>(dst + i, x);
}

template <int KIND, int U, bool NT, bool BLOCKED>
__global__ __launch_bounds__(256) void stream_only(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   uint32_t* __restrict__ sink, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  auto get = [&](int64_t i) -> u32x4 {
    if (KIND == 1) {
      const uint32_t v = (uint32_t)i;
      return u32x4{v, v + 1, v + 2, v + 3};
    }
    return ld<NT>(src + i);
  };
  if (BLOCKED) {
    const int64_t base = (int64_t)blockIdx.x * (256 * U) + threadIdx.x;
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; u++) x[u] = base + u * 256 < n ? get(base + u * 256) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < U; u++)
      if (base + u * 256 < n) stream_put<KIND, NT>(dst, base + u * 256, x[u], acc);
  } else {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = t;
    for (; i + (U - 1) * stride < n; i += U * stride) {
      u32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; u++) x[u] = get(i + u * stride);
#pragma unroll
      for (int u = 0; u < U; u++) stream_put<KIND, NT>(dst, i + u * stride, x[u], acc);
    }
    for (; i < n; i += stride) stream_put<KIND, NT>(dst, i, get(i), acc);
  }
  if (KIND == 0 && (acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x6A09E667u) sink[t & 255] = acc.x;
}

template <int KIND, int U>
const void* stream_kernel_nt(bool nt, bool blocked) {
  if (blocked)
    return nt ? (const void*)&stream_only<KIND, U, true, true> : (const void*)&stream_only<KIND, U, false, true>;
  return nt ? (const void*)&stream_only<KIND, U, true, false> : (const void*)&stream_only<KIND, U, false, false>;
}

template <int KIND>
const void* stream_kernel(int unroll, bool nt, bool blocked) {
  return unroll == 1   ? stream_kernel_nt<KIND, 1>(nt, blocked)
         : unroll == 2 ? stream_kernel_nt<KIND, 2>(nt, blocked)
         : unroll == 4 ? stream_kernel_nt<KIND, 4>(nt, blocked)
                       : stream_kernel_nt<KIND, 8>(nt, blocked);
}

// Median of the second half of `reps` launch times (the clock and the
// caches have settled by then).
float steady(float* ms_all, int reps) {
  std::sort(ms_all + reps / 2, ms_all + reps);
  return ms_all[reps / 2 + (reps - reps / 2) / 2];
}

}  // namespace

extern "C" int mx_calib_stream(int kind, int64_t bytes, int workgroups, int unroll, int nontemporal,
                               int reps, float* steady_ms, double* moved) {
  if (kind < 0 || kind > 3 || bytes < 4096 || bytes % 64 != 0 || bytes > ((int64_t)1 << 36) ||
      workgroups < 0 || workgroups > 65535 || (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) ||
      (nontemporal != 0 && nontemporal != 1) || reps <= 0 || !steady_ms || !moved)
    return -1;
  reps = std::min(reps, 256);
  const int64_t n = bytes / 16;  // 16-byte chunks read (kind 1: written)
  const size_t src_bytes = kind == 1 ? 0 : (size_t)bytes;
  const size_t dst_bytes = kind == 0 ? 0 : kind == 3 ? (size_t)bytes / 4 : (size_t)bytes;
  // One pass (workgroups == 0): as many workgroups as the chunks need, at
  // most 2^31 - 1 of them.
  const bool blocked = workgroups == 0;
  const int64_t grid = blocked ? (n + 256LL * unroll - 1) / (256LL * unroll) : workgroups;
  if (grid > 0x7FFFFFFF) return -1;
  void *src = nullptr, *dst = nullptr, *sink = nullptr;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipMalloc(&sink, 1024);
  if (err == hipSuccess && src_bytes) err = hipMalloc(&src, src_bytes);
  if (err == hipSuccess && dst_bytes) err = hipMalloc(&dst, dst_bytes);
  if (err == hipSuccess) err = hipStreamCreate(&s);
  if (err == hipSuccess) err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  float ms_all[256];
  const bool nt = nontemporal == 1;
  const void* f = kind == 0   ? stream_kernel<0>(unroll, nt, blocked)
                  : kind == 1 ? stream_kernel<1>(unroll, nt, blocked)
                  : kind == 2 ? stream_kernel<2>(unroll, nt, blocked)
                              : stream_kernel<3>(unroll, nt, blocked);
  for (int r = 0; r < reps && err == hipSuccess; r++) {
    err = hipEventRecord(e0, s);
    if (err != hipSuccess) break;
    int64_t nn = n;
    void* args[] = {&src, &dst, &sink, &nn};
    err = hipLaunchKernel(f, dim3((unsigned)grid), dim3(256), args, 0, s);
    if (err == hipSuccess) err = hipEventRecord(e1, s);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    ms_all[r] = ms;
  }
  if (e1) (void)hipEventDestroy(e1);
  if (e0) (void)hipEventDestroy(e0);
  if (s) (void)hipStreamDestroy(s);
  if (dst) (void)hipFree(dst);
  if (src) (void)hipFree(src);
  if (sink) (void)hipFree(sink);
  if (err != hipSuccess) return (int)err;
  *steady_ms = steady(ms_all, reps);
  *moved = (double)(src_bytes + dst_bytes);
  return 0;
}

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
  *steady_ms = steady(ms_all, reps);
  *flop = (double)workgroups * (threads / 64) * (double)iters * per_wave;
  return 0;
}
