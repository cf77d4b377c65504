// Block-scaled GEMM for MXFP4 x MXFP4 on gfx950's scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4), the 128 x 128-tile kernel for shapes
// the 256 x 256-tile kernel (gemm_mxfp4.hip) does not take (K % 256 != 0, or
// offsets beyond 32 bits). C = A * B^T, A is M x K codes, B is stored N x K
// codes, one E8M0 scale per 32 K per row. The matrix core applies both E8M0
// scales inside its fp32 accumulation, so codes go to the instruction
// unexpanded (the block-scaled dot product described in "Arquitetura
// Blackwell SM100 e aceleracao nativa de NVFP4" on the produtoramaxvision
// page, there for B200 tensor cores). (MXFP8 does not come here: the FP8
// scaled MFMA truncates within a block, see gemm_bf16x.hip.)
//
// Operand layout of the 16x16x128 instruction (measured on gfx950): lane
// l = r + 16 g (r = row in the 16-row tile, g = 0..3) supplies K elements
// [32g, 32g + 32) of row r, 16 bytes, even element in the low nibble (the same
// packing as the codes in memory), and the E8M0 scale of K block g of row r.
// Output: lane l holds column l % 16, rows 4 (l / 16) + 0..3.
//
// MXFP4-MBS (static macro-block scaling; gist.science summary of "Unveiling
// the Potential of Quantization with MXFP4", section 2.B): a K step of 128 is
// exactly one macro block, so each step's MFMA starts from zero and yields the
// block-scaled partial sum P of that macro block; the vector ALU then adds
// P * f_A(row) * f_B(col) to the accumulator (f_A f_B has 18 significant bits
// and is exact in fp32), the factor being applied alongside the matrix core
// as the summary describes. With 16-element base blocks (MXFP4-MBS16) each
// lane's 32 codes carry two scales, so P takes two MFMAs, one per 16-element
// half with the other half zero.
#include "bf16.h"
#include "mx_internal.h"

namespace mx {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 128;  // tile sizes in elements
constexpr uint32_t kUnitScale = 127u;        // 2^0 for padded blocks
constexpr int kSegSteps = 48;                // K steps per accumulation chain

template <int FMT>
struct MxTile {
  static constexpr int kBits = (FMT == kMXFP4) ? 4 : 8;
  static constexpr int kRowBytes = BK * kBits / 8;          // bytes per tile row per K step
  static constexpr int kStride = kRowBytes + 16;            // padded LDS row
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kLoads = BM * kChunksPerRow / kThreads;  // 16-byte loads per thread
  static constexpr int kMfmaFmt = (FMT == kMXFP4) ? 4 : 0;  // cbsz / blgp selector
};

// MBS: MA / MB are the macro mantissa planes [rows][K/128] (unused otherwise);
// BASE: the E8M0 block size, 32, or 16 for MXFP4-MBS16.
template <int FMT, int OUT, bool MBS, int BASE = 32>
__global__ __launch_bounds__(kThreads) void gemm_mx_kernel(const uint8_t* __restrict__ A,
                                                           const uint8_t* __restrict__ SA,
                                                           const uint8_t* __restrict__ B,
                                                           const uint8_t* __restrict__ SB,
                                                           const uint8_t* __restrict__ MA,
                                                           const uint8_t* __restrict__ MB,
                                                           void* __restrict__ C, int64_t ldc,
                                                           int M, int N, int K) {
  using T = MxTile<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t lA[BM * T::kStride];
  __shared__ __attribute__((aligned(16))) uint8_t lB[BN * T::kStride];
  __shared__ uint32_t lSA[BM];
  __shared__ uint32_t lSB[BN];
  // BASE 16: scales of the second 16 elements of each 32 (the first 16's are
  // in lSA / lSB).
  __shared__ uint32_t lSA2[BASE == 16 ? BM : 1];
  __shared__ uint32_t lSB2[BASE == 16 ? BN : 1];
  __shared__ float lFA[MBS ? BM : 1];
  __shared__ float lFB[MBS ? BN : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int64_t rowbytes = (int64_t)K * T::kBits / 8;
  const int kblocks = K / BASE;
  const int nk = (K + BK - 1) / BK;

  u32x4 ra[T::kLoads], rb[T::kLoads];
  uint32_t rs = 0, rs2 = 0;
  float rf = 1.0f;

  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < T::kLoads; i++) {
      const int chunk = tid + i * kThreads;
      const int row = chunk / T::kChunksPerRow, c16 = chunk % T::kChunksPerRow;
      const int64_t kb = (int64_t)kt * T::kRowBytes + c16 * 16;
      const int ga = m0 + row, gb = n0 + row;
      ra[i] = (ga < M && kb < rowbytes) ? *(const u32x4*)(A + ga * rowbytes + kb) : u32x4{0, 0, 0, 0};
      rb[i] = (gb < N && kb < rowbytes) ? *(const u32x4*)(B + gb * rowbytes + kb) : u32x4{0, 0, 0, 0};
    }
    // Threads 0..127 fetch the 4 A-scale bytes of one tile row, 128..255 B's.
    const int row = tid & 127;
    const bool isA = tid < 128;
    const int grow = (isA ? m0 : n0) + row;
    const int glim = isA ? M : N;
    const uint8_t* S = isA ? SA : SB;
    rs = 0;
    rs2 = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (BASE == 32) {
        const int kbk = kt * 4 + j;
        const uint32_t e = (grow < glim && kbk < kblocks) ? S[(int64_t)grow * kblocks + kbk] : kUnitScale;
        rs |= e << (8 * j);
      } else {
        // 32-element group j of the step: 16-blocks 2 j (rs) and 2 j + 1 (rs2)
        const int kbk = kt * 8 + 2 * j;
        const bool in = grow < glim && kbk < kblocks;
        const uint32_t e0 = in ? S[(int64_t)grow * kblocks + kbk] : kUnitScale;
        const uint32_t e1 = in ? S[(int64_t)grow * kblocks + kbk + 1] : kUnitScale;
        rs |= e0 << (8 * j);
        rs2 |= e1 << (8 * j);
      }
    }
    if (MBS) {
      // Macro factor 1 + m / 256 of this step's macro block (K step = 128).
      const uint8_t* Mp = isA ? MA : MB;
      const uint32_t m = (grow < glim) ? Mp[(int64_t)grow * (K / 128) + kt] : 0u;
      rf = (float)(256u + m) * 0x1p-8f;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < T::kLoads; i++) {
      const int chunk = tid + i * kThreads;
      const int row = chunk / T::kChunksPerRow, c16 = chunk % T::kChunksPerRow;
      *(u32x4*)(lA + row * T::kStride + c16 * 16) = ra[i];
      *(u32x4*)(lB + row * T::kStride + c16 * 16) = rb[i];
    }
    if (tid < 128)
      lSA[tid] = rs;
    else
      lSB[tid - 128] = rs;
    if (BASE == 16) {
      if (tid < 128)
        lSA2[tid] = rs2;
      else
        lSB2[tid - 128] = rs2;
    }
    if (MBS) {
      if (tid < 128)
        lFA[tid] = rf;
      else
        lFB[tid - 128] = rf;
    }
  };

  f32x4 acc[4][4], tot[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = tot[i][j] = f32x4{0, 0, 0, 0};

  const int r = lane & 15, g = lane >> 4;
  gload(0);
  for (int kt = 0; kt < nk; kt++) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (kt + 1 < nk) gload(kt + 1);
    i32x8 af[4], bf[4];
    int sa[4], sb[4], sa2[4], sb2[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int ra_ = wm * 64 + i * 16 + r;
      const int rb_ = wn * 64 + i * 16 + r;
      const u32x4 x = *(const u32x4*)(lA + ra_ * T::kStride + g * 16);
      const u32x4 y = *(const u32x4*)(lB + rb_ * T::kStride + g * 16);
      af[i] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
      bf[i] = i32x8{(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
      sa[i] = (int)((lSA[ra_] >> (8 * g)) & 0xFFu);
      sb[i] = (int)((lSB[rb_] >> (8 * g)) & 0xFFu);
      if (BASE == 16) {
        sa2[i] = (int)((lSA2[ra_] >> (8 * g)) & 0xFFu);
        sb2[i] = (int)((lSB2[rb_] >> (8 * g)) & 0xFFu);
      }
    }
    if (MBS) {
      float fa[4][4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        fb[i] = lFB[wn * 64 + i * 16 + r];
#pragma unroll
        for (int t = 0; t < 4; t++) fa[i][t] = lFA[wm * 64 + i * 16 + 4 * g + t];
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          f32x4 p;
          if (BASE == 32) {
            p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af[i], bf[j], f32x4{0, 0, 0, 0}, T::kMfmaFmt, T::kMfmaFmt, 0, sa[i], 0, sb[j]);
          } else {
            // One scale per lane's 32 codes: each 32 split into its two
            // 16-blocks (the other half zero), one MFMA under each scale.
            const i32x8 alo = i32x8{af[i][0], af[i][1], 0, 0, 0, 0, 0, 0};
            const i32x8 ahi = i32x8{0, 0, af[i][2], af[i][3], 0, 0, 0, 0};
            const i32x8 blo = i32x8{bf[j][0], bf[j][1], 0, 0, 0, 0, 0, 0};
            const i32x8 bhi = i32x8{0, 0, bf[j][2], bf[j][3], 0, 0, 0, 0};
            p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                alo, blo, f32x4{0, 0, 0, 0}, T::kMfmaFmt, T::kMfmaFmt, 0, sa[i], 0, sb[j]);
            p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                ahi, bhi, p, T::kMfmaFmt, T::kMfmaFmt, 0, sa2[i], 0, sb2[j]);
          }
#pragma unroll
          for (int t = 0; t < 4; t++)
            acc[i][j][t] = __builtin_fmaf(p[t], fa[i][t] * fb[j], acc[i][j][t]);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[i], bf[j], acc[i][j], T::kMfmaFmt, T::kMfmaFmt, 0, sa[i], 0, sb[j]);
    }
    // Accumulation chains of at most kSegSteps K steps (one MFMA, or one fma
    // for MBS, per step), added into a running total (one fp32 rounding per
    // segment).
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

#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int col = n0 + wn * 64 + j * 16 + r;
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const int row = m0 + wm * 64 + i * 16 + 4 * g + t;
        if (row < M && col < N) {
          if (OUT == kOutF32)
            ((float*)C)[(int64_t)row * ldc + col] = acc[i][j][t];
          else
            ((uint16_t*)C)[(int64_t)row * ldc + col] = bf16_bits(acc[i][j][t]);
        }
      }
    }
}

}  // namespace

hipError_t gemm_mx(int64_t M, int64_t N, int64_t K, const void* a, const void* sa, const void* b,
                   const void* sb, int out_dtype, void* c, int64_t ldc, hipStream_t s) {
  if (gemm_mxfp4_fits(M, N, K))
    return gemm_mxfp4(M, N, K, a, sa, b, sb, out_dtype, c, ldc, s, false, false);
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  const int m = (int)M, n = (int)N, k = (int)K;
  if (out_dtype == kOutF32)
    return launch_kernel(&gemm_mx_kernel<kMXFP4, kOutF32, false>, grid, kThreads, 0, s, A, SA, B, SB, nullptr, nullptr, c, ldc, m, n, k);
  return launch_kernel(&gemm_mx_kernel<kMXFP4, kOutBF16, false>, grid, kThreads, 0, s, A, SA, B, SB, nullptr, nullptr, c, ldc, m, n, k);
}

hipError_t gemm_mbs_small(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                          const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                          hipStream_t s, int base) {
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  const uint8_t* MA = SA + M * (K / base);  // macro planes follow the E8M0 planes
  const uint8_t* MB = SB + N * (K / base);
  const int m = (int)M, n = (int)N, k = (int)K;
  if (base == 16) {
    if (out_dtype == kOutF32)
      return launch_kernel(&gemm_mx_kernel<kMXFP4, kOutF32, true, 16>, grid, kThreads, 0, s, A, SA, B, SB, MA, MB, c, ldc, m, n, k);
    return launch_kernel(&gemm_mx_kernel<kMXFP4, kOutBF16, true, 16>, grid, kThreads, 0, s, A, SA, B, SB, MA, MB, c, ldc, m, n, k);
  }
  if (out_dtype == kOutF32)
    MX_TRY(launch_kernel(&gemm_mx_kernel<kMXFP4, kOutF32, true>, grid, kThreads, 0, s, A, SA, B, SB, MA, MB, c, ldc, m, n, k));
  else
    MX_TRY(launch_kernel(&gemm_mx_kernel<kMXFP4, kOutBF16, true>, grid, kThreads, 0, s, A, SA, B, SB, MA, MB, c, ldc, m, n, k));
  return hipSuccess;
}

}  // namespace mx
