// Block-scaled GEMM for MXFP8 x MXFP8 and NVFP4 x NVFP4 on gfx950's bf16 MFMA
// (v_mfma_f32_16x16x32_bf16), with every operand expanded exactly to bf16.
//
// Why not the matrix core's own FP8 / scaled path:
//  * NVFP4 scales are E4M3 per 16 elements (zubnet.ai summary; gist.science
//    summary, section 1: NVFP4 scale factors carry a mantissa) while the
//    scaled MFMA takes one E8M0 power of two per 32 elements.
//  * For MXFP8, gfx950's FP8 scaled MFMA does not sum a block exactly: small
//    products are truncated against the block's largest one (measured: with
//    unit scales, 256 + 2^-9 returns 256, and random E4M3 operands err by
//    ~2^-13 of sum|a*b|), which is outside the 2^-18 * sum|a*b| acceptance
//    bound. The bf16 MFMA returns fl32 of the exact sum on the same probes.
// Both expansions are exact in bf16:
//  * MXFP8: e * 2^(E-127) has the 4 significant bits of E4M3
//    (v_cvt_scalef32_pk_bf16_fp8 rounds it once, exactly when representable);
//  * NVFP4: e * s_b has at most 6 significant bits and lies in [2^-10, 2688];
//    s_t^A * s_t^B then scales the fp32 result:
//    C_ij = (s_t^A s_t^B) * sum_k (e^A s^A_b)(e^B s^B_b).
//
// Expansion happens once per tile while staging global -> LDS. bf16 MFMA
// layout (measured): lane l = r + 16 g holds K elements [8g, 8g + 8) of row r;
// the output lane l holds column l % 16, rows 4 (l / 16) + 0..3.
#include "bf16.h"
#include "mx_internal.h"

namespace mx {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 64;  // elements
constexpr int kStride = BK * 2 + 16;         // bytes per LDS row of bf16 (padded)
constexpr int kSegSteps = 24;                // K steps per accumulation chain (2 MFMAs each)

__device__ __forceinline__ float e8m0_to_float(uint32_t E) {
  return __builtin_bit_cast(float, E == 0 ? 0x00400000u : E << 23);
}

// NVFP4: the 8 codes of one dword times an E4M3 block scale, as 8 bf16. The
// products are exact in bf16, so keeping the high half of each fp32 is exact.
__device__ __forceinline__ u32x4 expand_nvfp4_dword(uint32_t q, float sb) {
  const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
  const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
  const f32x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
  const f32x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
  auto pk = [sb](f32x2 e) {
    return (__builtin_bit_cast(uint32_t, e.x * sb) >> 16) |
           (__builtin_bit_cast(uint32_t, e.y * sb) & 0xFFFF0000u);
  };
  return u32x4{pk(e0), pk(e1), pk(e2), pk(e3)};
}

// MXFP8: the 8 codes of two dwords times 2^(E-127), as 8 bf16.
__device__ __forceinline__ u32x4 expand_mxfp8_2dwords(uint32_t q0, uint32_t q1, float s) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q0, s, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q0, s, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q1, s, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q1, s, true))};
}

// Staging: thread t owns row t / 2 and the 32-element half (t % 2) of the
// 64-element K step, for A and for B.
template <int FMT>
struct Stage {
  static constexpr int kCodeBytes = (FMT == kMXFP8) ? 32 : 16;  // codes per thread
  u32x4 q[2];
  uint32_t e0, e1;  // scale bytes (NVFP4: two 16-blocks; MXFP8: e0 only)

  __device__ __forceinline__ void load(const uint8_t* __restrict__ X, const uint8_t* __restrict__ S,
                                       int grow, int glim, int K, int kt, int half) {
    const int64_t rowbytes = (FMT == kMXFP8) ? K : K / 2;
    const int k0 = kt * BK + half * 32;  // first element
    const bool ok = grow < glim && k0 < K;
    const uint8_t* src = X + (int64_t)grow * rowbytes + ((FMT == kMXFP8) ? k0 : k0 / 2);
    q[0] = ok ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
    if (FMT == kMXFP8) q[1] = ok ? *(const u32x4*)(src + 16) : u32x4{0, 0, 0, 0};
    if (FMT == kMXFP8) {
      e0 = ok ? S[(int64_t)grow * (K / 32) + k0 / 32] : 127u;
      e1 = 0;
    } else {
      const int64_t sb = (int64_t)grow * (K / 16) + k0 / 16;
      e0 = ok ? S[sb] : 0x38u;  // E4M3 1.0 for padding
      e1 = ok ? S[sb + 1] : 0x38u;
    }
  }

  __device__ __forceinline__ void expand_store(uint8_t* dst) const {
    if (FMT == kMXFP8) {
      const float s = e8m0_to_float(e0);
      // A NaN scale (255) makes the whole block NaN, as in the oracle.
      const bool nan = e0 == 255u;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        u32x4 o0 = expand_mxfp8_2dwords(q[h].x, q[h].y, s);
        u32x4 o1 = expand_mxfp8_2dwords(q[h].z, q[h].w, s);
        if (nan) o0 = o1 = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
        *(u32x4*)(dst + h * 32) = o0;
        *(u32x4*)(dst + h * 32 + 16) = o1;
      }
    } else {
      const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)e0, 0);
      const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)e1, 0);
      *(u32x4*)(dst + 0) = expand_nvfp4_dword(q[0].x, s0);
      *(u32x4*)(dst + 16) = expand_nvfp4_dword(q[0].y, s0);
      *(u32x4*)(dst + 32) = expand_nvfp4_dword(q[0].z, s1);
      *(u32x4*)(dst + 48) = expand_nvfp4_dword(q[0].w, s1);
    }
  }
};

template <int FMT, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_bf16x_kernel(const uint8_t* __restrict__ A,
                                                              const uint8_t* __restrict__ SA,
                                                              const float* __restrict__ TA,
                                                              const uint8_t* __restrict__ B,
                                                              const uint8_t* __restrict__ SB,
                                                              const float* __restrict__ TB,
                                                              void* __restrict__ C, int64_t ldc,
                                                              int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[BM * kStride];
  __shared__ __attribute__((aligned(16))) uint8_t lB[BN * kStride];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int nk = (K + BK - 1) / BK;
  const int srow = tid >> 1, shalf = tid & 1;

  Stage<FMT> sa, sb;
  f32x4 acc[4][4], tot[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = tot[i][j] = f32x4{0, 0, 0, 0};

  const int r = lane & 15, g = lane >> 4;
  sa.load(A, SA, m0 + srow, M, K, 0, shalf);
  sb.load(B, SB, n0 + srow, N, K, 0, shalf);
  for (int kt = 0; kt < nk; kt++) {
    __syncthreads();
    sa.expand_store(lA + srow * kStride + shalf * 64);
    sb.expand_store(lB + srow * kStride + shalf * 64);
    __syncthreads();
    if (kt + 1 < nk) {
      sa.load(A, SA, m0 + srow, M, K, kt + 1, shalf);
      sb.load(B, SB, n0 + srow, N, K, kt + 1, shalf);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ks++) {
      bf16x8 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        af[i] = *(const bf16x8*)(lA + (wm * 64 + i * 16 + r) * kStride + ks * 64 + g * 16);
        bf[i] = *(const bf16x8*)(lB + (wn * 64 + i * 16 + r) * kStride + ks * 64 + g * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    // Accumulation chains of at most kSegSteps K steps (48 MFMAs), added
    // into a running total (one fp32 rounding per segment).
    if ((kt + 1) % kSegSteps == 0 && kt + 1 < nk) {
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          tot[i][j] += acc[i][j];
          acc[i][j] = f32x4{0, 0, 0, 0};
        }
    }
  }
  if (nk > kSegSteps) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] += tot[i][j];
  }

  const float ts = (FMT == kNVFP4) ? TA[0] * TB[0] : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int col = n0 + wn * 64 + j * 16 + r;
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const int row = m0 + wm * 64 + i * 16 + 4 * g + t;
        if (row < M && col < N) {
          const float v = (FMT == kNVFP4) ? acc[i][j][t] * ts : acc[i][j][t];
          if (OUT == kOutF32)
            ((float*)C)[(int64_t)row * ldc + col] = v;
          else
            ((uint16_t*)C)[(int64_t)row * ldc + col] = bf16_bits(v);
        }
      }
    }
}

template <int FMT>
hipError_t launch(const dim3& grid, hipStream_t s, const uint8_t* A, const uint8_t* SA, const float* TA,
            const uint8_t* B, const uint8_t* SB, const float* TB, int out_dtype, void* c, int64_t ldc,
            int M, int N, int K) {
  if (out_dtype == kOutF32)
    MX_TRY(launch_kernel(&gemm_bf16x_kernel<FMT, kOutF32>, grid, kThreads, 0, s, A, SA, TA, B, SB, TB, c, ldc, M, N, K));
  else
    MX_TRY(launch_kernel(&gemm_bf16x_kernel<FMT, kOutBF16>, grid, kThreads, 0, s, A, SA, TA, B, SB, TB, c, ldc, M, N, K));
  return hipSuccess;
}

}  // namespace

hipError_t gemm_bf16x(int fmt, int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                      const float* ta, const void* b, const void* sb, const float* tb,
                      int out_dtype, void* c, int64_t ldc, hipStream_t s) {
  if (gemm_bf16x_large_fits(fmt, M, N, K))
    return gemm_bf16x_large(fmt, M, N, K, a, sa, ta, b, sb, tb, out_dtype, c, ldc, s);
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  if (fmt == kMXFP8)
    return launch<kMXFP8>(grid, s, A, SA, ta, B, SB, tb, out_dtype, c, ldc, (int)M, (int)N, (int)K);
  return launch<kNVFP4>(grid, s, A, SA, ta, B, SB, tb, out_dtype, c, ldc, (int)M, (int)N, (int)K);
}

}  // namespace mx
