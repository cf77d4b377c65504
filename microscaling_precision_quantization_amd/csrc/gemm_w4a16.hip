// W4A16 GEMM on gfx950: bf16 activations (M x K, few rows: decode) times MXFP4
// weights (stored N x K) with fp32 accumulation. Weight-only quantization saves
// memory traffic rather than compute (noticiai.com.br page on Nunchaku W4A4:
// dequantizing weights at compute time mainly saves memory), so this kernel is
// built to stream the weight codes once from HBM:
//  * each lane loads 16 bytes (32 codes, exactly one E8M0 block) per step and
//    expands them to bf16 with v_cvt_scalef32_pk_bf16_fp4, which multiplies by
//    the power-of-two scale exactly;
//  * the 32 codes feed four v_mfma_f32_16x16x32_bf16 in a row. The K order
//    inside a 128-element step is permuted the same way for both operands:
//    MFMA j uses elements 32g + 8j .. 32g + 8j + 7 in lane group g, so a lane's
//    codes, its one scale and its activation slice stay contiguous;
//  * activations for the workgroup's K range are staged once in LDS;
//  * K is split across workgroups; partial sums go to a workspace and a second
//    kernel adds them in a fixed order (deterministic, no float atomics).
#include "bf16.h"
#include "mx_internal.h"

namespace mx {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int TN = 64;    // output columns per workgroup (16 per wave)
constexpr int TM = 16;    // activation rows per workgroup
constexpr int KC = 512;   // K elements of activations staged in LDS at once
constexpr int kAStride = KC * 2 + 16;  // bytes per LDS activation row (padded)
constexpr uint32_t kUnitScale = 127u;

__device__ __forceinline__ float e8m0_to_float(uint32_t E) {
  return __builtin_bit_cast(float, E == 0 ? 0x00400000u : E << 23);
}

// 8 codes (one dword) -> 8 bf16 times 2^(E-127).
__device__ __forceinline__ bf16x8 expand8(uint32_t q, float s) {
  u32x4 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 0));
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 1));
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 2));
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 3));
  return __builtin_bit_cast(bf16x8, o);
}

// grid: x = N tiles, y = M tiles, z = K splits. Each split covers kper
// elements (a multiple of 128) starting at z * kper.
template <bool DIRECT, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_w4a16_kernel(const uint16_t* __restrict__ A,
                                                              const uint8_t* __restrict__ B,
                                                              const uint8_t* __restrict__ SB,
                                                              void* __restrict__ out, int64_t ldc,
                                                              int M, int N, int K, int kper) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[TM * kAStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.y * TM;
  const int n = blockIdx.x * TN + wave * 16 + r;  // this lane's weight row
  const int kbeg = blockIdx.z * kper;
  const int kend = min(K, kbeg + kper);
  const int64_t rowbytes = K / 2;
  const int kblocks = K / 32;

  // Four accumulators, one per MFMA of a 128-element step: independent chains
  // keep the matrix pipeline busy and each chain at most K/128 steps long.
  f32x4 acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  for (int kc = kbeg; kc < kend; kc += KC) {
    __syncthreads();
    // Stage activations [m0, m0+16) x [kc, kc+KC) as bf16, zero-padded.
    for (int i = tid; i < TM * KC / 8; i += kThreads) {
      const int row = i / (KC / 8), c8 = i % (KC / 8);
      const int k = kc + c8 * 8;
      u32x4 v = {0, 0, 0, 0};
      if (m0 + row < M && k < kend) v = *(const u32x4*)(A + (int64_t)(m0 + row) * K + k);
      *(u32x4*)(lA + row * kAStride + c8 * 16) = v;
    }
    __syncthreads();
    const int ksteps = min(KC, kend - kc);  // multiple of 32
    for (int ks = 0; ks < ksteps; ks += 128) {
      const int k = kc + ks + 32 * g;  // first element of this lane's block
      u32x4 q = {0, 0, 0, 0};
      uint32_t E = kUnitScale;
      if (n < N && k < kend) {
        q = __builtin_nontemporal_load((const u32x4*)(B + (int64_t)n * rowbytes + k / 2));
        E = SB[(int64_t)n * kblocks + k / 32];
      }
      const float s = e8m0_to_float(E);
      const uint8_t* arow = lA + r * kAStride + (ks + 32 * g) * 2;
      const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const bf16x8 a = *(const bf16x8*)(arow + j * 16);
        const bf16x8 w = (E == 255) ? __builtin_bit_cast(bf16x8, u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u})
                                    : expand8(qw[j], s);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w, acc[j], 0, 0, 0);
      }
    }
  }
  const f32x4 sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  // Lane l holds column n (= l % 16 within the wave's 16) for rows 4g + t.
  if (n >= N) return;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int m = m0 + 4 * g + t;
    if (m >= M) continue;
    if (DIRECT) {
      if (OUT == kOutF32)
        ((float*)out)[(int64_t)m * ldc + n] = sum[t];
      else
        ((uint16_t*)out)[(int64_t)m * ldc + n] = bf16_bits(sum[t]);
    } else {
      ((float*)out)[((int64_t)blockIdx.z * M + m) * N + n] = sum[t];
    }
  }
}

template <int OUT>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const float* __restrict__ part,
                                                                 void* __restrict__ C, int64_t ldc,
                                                                 int M, int N, int splits) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int m = (int)(i / N), n = (int)(i % N);
  float s = 0.0f;
  for (int z = 0; z < splits; z++) s += part[(int64_t)z * M * N + i];
  if (OUT == kOutF32)
    ((float*)C)[(int64_t)m * ldc + n] = s;
  else
    ((uint16_t*)C)[(int64_t)m * ldc + n] = bf16_bits(s);
}

struct Plan {
  int splits;
  int kper;
};

// Enough workgroups to cover the chip several times (7 per CU on 256 CUs),
// with each split at most 16 steps of 128 elements (16 MFMAs per chain).
Plan plan(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((N + TN - 1) / TN) * ((M + TM - 1) / TM);
  const int64_t ksteps = (K + 127) / 128;
  int splits = 1;
  while (splits < 64 && (tiles * splits < 1792 || (ksteps + splits - 1) / splits > 16) &&
         splits * 2 <= ksteps)
    splits *= 2;
  const int64_t kper_steps = (ksteps + splits - 1) / splits;
  Plan p;
  p.kper = (int)(kper_steps * 128);
  p.splits = (int)((K + p.kper - 1) / p.kper);
  return p;
}

}  // namespace

size_t gemm_w4a16_workspace(int64_t M, int64_t N, int64_t K) {
  const Plan p = plan(M, N, K);
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

hipError_t gemm_w4a16(int64_t M, int64_t N, int64_t K, const void* a, const void* b,
                      const void* sb, int out_dtype, void* c, int64_t ldc, void* workspace,
                      hipStream_t s) {
  const Plan p = plan(M, N, K);
  const dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM), (unsigned)p.splits);
  const uint16_t* A = (const uint16_t*)a;
  const uint8_t *B = (const uint8_t*)b, *SB = (const uint8_t*)sb;
  const int m = (int)M, n = (int)N, k = (int)K;
  if (p.splits == 1) {
    if (out_dtype == kOutF32)
      gemm_w4a16_kernel<true, kOutF32><<<grid, kThreads, 0, s>>>(A, B, SB, c, ldc, m, n, k, p.kper);
    else
      gemm_w4a16_kernel<true, kOutBF16><<<grid, kThreads, 0, s>>>(A, B, SB, c, ldc, m, n, k, p.kper);
    return hipGetLastError();
  }
  gemm_w4a16_kernel<false, kOutF32><<<grid, kThreads, 0, s>>>(A, B, SB, workspace, 0, m, n, k, p.kper);
  const unsigned rblocks = (unsigned)((M * N + kThreads - 1) / kThreads);
  if (out_dtype == kOutF32)
    splitk_reduce_kernel<kOutF32><<<rblocks, kThreads, 0, s>>>((const float*)workspace, c, ldc, m, n, p.splits);
  else
    splitk_reduce_kernel<kOutBF16><<<rblocks, kThreads, 0, s>>>((const float*)workspace, c, ldc, m, n, p.splits);
  return hipGetLastError();
}

}  // namespace mx
