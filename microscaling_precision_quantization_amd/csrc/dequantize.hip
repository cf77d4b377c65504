// Dequantization kernels for gfx950: x_real = S * x_elem ("Fundamentos
// matematicos do formato MXFP4 e E8M0" on the produtoramaxvision page). MX
// (MXFP4, MXFP8 E4M3 / E5M2, MXFP6 E3M2):
// y = val(code) * 2^(E-127); NVFP4: y = fl32(fl32(val * s_b) * s_t); MXFP4
// with macro-block scaling: y = val(code) * 2^(E-127) * (1 + m / 256), exact in
// fp32 (the product has at most 11 significant bits) unless it overflows.
//
// One thread expands one 16-byte group of 8 outputs' codes. The scaled decodes
// v_cvt_scalef32_pk_{f32,bf16}_fp4 and v_cvt_scalef32_pk_f32_fp8 multiply by a
// power-of-two scale exactly and round once to the output type.
#include "bf16.h"
#include "mx_internal.h"

namespace mx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr uint32_t kNaNf = 0x7FC00000u;

__device__ __forceinline__ float e8m0_to_float(uint32_t E) {
  return __builtin_bit_cast(float, E == 0 ? 0x00400000u : E << 23);
}


template <int OUT>
__device__ __forceinline__ void store8(void* y, int64_t c, const float (&o)[8]) {
  if (OUT == kOutF32) {
    f32x4* p = (f32x4*)y + 2 * c;
    __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, p);
    __builtin_nontemporal_store(f32x4{o[4], o[5], o[6], o[7]}, p + 1);
  } else {
    u32x4 w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
    __builtin_nontemporal_store(w, (u32x4*)y + c);
  }
}

template <int OUT>
__global__ __launch_bounds__(kThreads) void dequant_mxfp4_kernel(const uint32_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales,
                                                                 void* __restrict__ y, int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= nchunks) return;
  const uint32_t q = codes[c];
  const uint32_t E = scales[c >> 2];
  if (OUT == kOutBF16 && E != 255) {
    const float s = e8m0_to_float(E);
    u32x4 w;
    w.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 0));
    w.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 1));
    w.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 2));
    w.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 3));
    __builtin_nontemporal_store(w, (u32x4*)y + c);
    return;
  }
  float o[8];
  if (E == 255) {
    for (int i = 0; i < 8; i++) o[i] = __builtin_bit_cast(float, kNaNf);
  } else {
    const float s = e8m0_to_float(E);
    f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 0);
    f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 1);
    f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 2);
    f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 3);
    o[0] = p0.x; o[1] = p0.y; o[2] = p1.x; o[3] = p1.y;
    o[4] = p2.x; o[5] = p2.y; o[6] = p3.x; o[7] = p3.y;
  }
  store8<OUT>(y, c, o);
}

template <int OUT, bool E5M2>
__global__ __launch_bounds__(kThreads) void dequant_mxfp8_kernel(const u32x2* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales,
                                                                 void* __restrict__ y, int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= nchunks) return;
  const u32x2 q = codes[c];
  const uint32_t E = scales[c >> 2];
  float o[8];
  if (E == 255) {
    for (int i = 0; i < 8; i++) o[i] = __builtin_bit_cast(float, kNaNf);
  } else {
    const float s = e8m0_to_float(E);
    f32x2 p0, p1, p2, p3;
    if (E5M2) {
      p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(q.x, s, false);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(q.x, s, true);
      p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(q.y, s, false);
      p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(q.y, s, true);
    } else {
      p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q.x, s, false);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q.x, s, true);
      p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q.y, s, false);
      p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q.y, s, true);
    }
    o[0] = p0.x; o[1] = p0.y; o[2] = p1.x; o[3] = p1.y;
    o[4] = p2.x; o[5] = p2.y; o[6] = p3.x; o[7] = p3.y;
  }
  store8<OUT>(y, c, o);
}

// MXFP4-MBS: the MXFP4 value times the macro factor of its 128-element block.
template <int OUT, int BASE>
__global__ __launch_bounds__(kThreads) void dequant_mbs_kernel(const uint32_t* __restrict__ codes,
                                                               const uint8_t* __restrict__ scales,
                                                               const uint8_t* __restrict__ macro,
                                                               void* __restrict__ y, int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= nchunks) return;
  const uint32_t q = codes[c];
  // chunk c (8 elements) lies in base block c / 4 (BASE 32) or c / 2 (BASE 16)
  const uint32_t E = scales[BASE == 32 ? (c >> 2) : (c >> 1)];
  const float f = (float)(256u + macro[c >> 4]) * 0x1p-8f;
  float o[8];
  if (E == 255) {
    for (int i = 0; i < 8; i++) o[i] = __builtin_bit_cast(float, kNaNf);
  } else {
    const float s = e8m0_to_float(E);
    const f32x2 p[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 0),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 1),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 2),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 3)};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      o[2 * k] = p[k].x * f;
      o[2 * k + 1] = p[k].y * f;
    }
  }
  store8<OUT>(y, c, o);
}

typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
typedef float f32x32 __attribute__((ext_vector_type(32)));

// MXFP6 (E3M2): one thread per 32-block (24 code bytes).
template <int OUT>
__global__ __launch_bounds__(kThreads) void dequant_mxfp6_kernel(const u32x2* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales,
                                                                 void* __restrict__ y, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nblocks) return;
  const u32x2 q0 = codes[3 * b], q1 = codes[3 * b + 1], q2 = codes[3 * b + 2];
  const uint32_t E = scales[b];
  f32x32 v;
  if (E == 255) {
#pragma unroll
    for (int i = 0; i < 32; i++) v[i] = __builtin_bit_cast(float, kNaNf);
  } else {
    v = __builtin_amdgcn_cvt_scalef32_pk32_f32_bf6(u32x6{q0.x, q0.y, q1.x, q1.y, q2.x, q2.y}, e8m0_to_float(E));
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const float o[8] = {v[8 * j], v[8 * j + 1], v[8 * j + 2], v[8 * j + 3],
                        v[8 * j + 4], v[8 * j + 5], v[8 * j + 6], v[8 * j + 7]};
    store8<OUT>(y, 4 * b + j, o);
  }
}

template <int OUT>
__global__ __launch_bounds__(kThreads) void dequant_nvfp4_kernel(const uint32_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales,
                                                                 const float* __restrict__ tensor_scale,
                                                                 void* __restrict__ y, int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= nchunks) return;
  const float st = tensor_scale[0];
  const uint32_t q = codes[c];
  const float sb = __builtin_amdgcn_cvt_f32_fp8((int)scales[c >> 1], 0);
  const f32x2 e[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0),
                       __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1),
                       __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2),
                       __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3)};
  float o[8];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    o[2 * j] = (e[j].x * sb) * st;  // e * s_b is exact; one rounding by s_t
    o[2 * j + 1] = (e[j].y * sb) * st;
  }
  store8<OUT>(y, c, o);
}

}  // namespace

hipError_t dequant(int fmt, int64_t rows, int64_t cols, const void* codes, const void* scales,
                   const float* tensor_scale, int out_dtype, void* y, hipStream_t s) {
  const int64_t nchunks = rows * cols / 8;
  const dim3 grid((unsigned)((nchunks + kThreads - 1) / kThreads));
  const uint8_t* sc = (const uint8_t*)scales;
  if (fmt == kMXFP4) {
    if (out_dtype == kOutF32)
      MX_TRY(launch_kernel(&dequant_mxfp4_kernel<kOutF32>, grid, kThreads, 0, s, (const uint32_t*)codes, sc, y, nchunks));
    else
      MX_TRY(launch_kernel(&dequant_mxfp4_kernel<kOutBF16>, grid, kThreads, 0, s, (const uint32_t*)codes, sc, y, nchunks));
  } else if (fmt == kMXFP8) {
    if (out_dtype == kOutF32)
      MX_TRY(launch_kernel(&dequant_mxfp8_kernel<kOutF32, false>, grid, kThreads, 0, s, (const u32x2*)codes, sc, y, nchunks));
    else
      MX_TRY(launch_kernel(&dequant_mxfp8_kernel<kOutBF16, false>, grid, kThreads, 0, s, (const u32x2*)codes, sc, y, nchunks));
  } else if (fmt == kMXFP8E5M2) {
    if (out_dtype == kOutF32)
      MX_TRY(launch_kernel(&dequant_mxfp8_kernel<kOutF32, true>, grid, kThreads, 0, s, (const u32x2*)codes, sc, y, nchunks));
    else
      MX_TRY(launch_kernel(&dequant_mxfp8_kernel<kOutBF16, true>, grid, kThreads, 0, s, (const u32x2*)codes, sc, y, nchunks));
  } else if (fmt == kMXFP4MBS) {
    const uint8_t* mac = sc + rows * (cols / 32);
    if (out_dtype == kOutF32)
      MX_TRY(launch_kernel(&dequant_mbs_kernel<kOutF32, 32>, grid, kThreads, 0, s, (const uint32_t*)codes, sc, mac, y, nchunks));
    else
      MX_TRY(launch_kernel(&dequant_mbs_kernel<kOutBF16, 32>, grid, kThreads, 0, s, (const uint32_t*)codes, sc, mac, y, nchunks));
  } else if (fmt == kMXFP4MBS16) {
    const uint8_t* mac = sc + rows * (cols / 16);
    if (out_dtype == kOutF32)
      MX_TRY(launch_kernel(&dequant_mbs_kernel<kOutF32, 16>, grid, kThreads, 0, s, (const uint32_t*)codes, sc, mac, y, nchunks));
    else
      MX_TRY(launch_kernel(&dequant_mbs_kernel<kOutBF16, 16>, grid, kThreads, 0, s, (const uint32_t*)codes, sc, mac, y, nchunks));
  } else if (fmt == kMXFP6) {
    const int64_t nblocks = rows * cols / 32;
    const dim3 g6((unsigned)((nblocks + kThreads - 1) / kThreads));
    if (out_dtype == kOutF32)
      MX_TRY(launch_kernel(&dequant_mxfp6_kernel<kOutF32>, g6, kThreads, 0, s, (const u32x2*)codes, sc, y, nblocks));
    else
      MX_TRY(launch_kernel(&dequant_mxfp6_kernel<kOutBF16>, g6, kThreads, 0, s, (const u32x2*)codes, sc, y, nblocks));
  } else {
    if (out_dtype == kOutF32)
      MX_TRY(launch_kernel(&dequant_nvfp4_kernel<kOutF32>, grid, kThreads, 0, s, (const uint32_t*)codes, sc, tensor_scale, y, nchunks));
    else
      MX_TRY(launch_kernel(&dequant_nvfp4_kernel<kOutBF16>, grid, kThreads, 0, s, (const uint32_t*)codes, sc, tensor_scale, y, nchunks));
  }
  return hipSuccess;
}

}  // namespace mx
