// Pieces shared by the large-tile GEMM kernels (2 x WNW waves of 128 x 32 NT,
// each 4 x NT MFMAs of 32 x 32 with operands passed B first: 4 waves of
// 128 x 128, or 8 waves of 128 x 64, for the 256 x 256 tiles): the XCD-aware
// tile order and the epilogue.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bf16.h"
#include "mx_internal.h"

namespace mx {
namespace tile256 {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 256;

// Output tile of workgroup `bid`. Workgroup ids go round-robin over the 8
// XCDs; when the tile count allows, XCD x gets the contiguous id range
// [x n/8, (x+1) n/8), rastered in groups of 4 tile rows, so that its L2 holds
// the A rows and B columns its tiles share.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int ntiles = tiles_m * tiles_n;
  const int t = (ntiles % 8 == 0) ? (bid % 8) * (ntiles / 8) + bid / 8 : bid;
  constexpr int GM = 4;
  const int group = t / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  tm = first_m + (t % (GM * tiles_n)) % gsize;
  tn = (t % (GM * tiles_n)) / gsize;
}

// As tile_of, for a grid of `grid` workgroups padded to a multiple of 8: XCD
// x gets the id range [x grid/8, (x+1) grid/8). Ids past the last tile (the
// padding) return false.
__device__ __forceinline__ bool tile_of_padded(int bid, int grid, int tiles_m, int tiles_n, int& tm,
                                               int& tn) {
  const int ntiles = tiles_m * tiles_n;
  const int t = (grid % 8 == 0) ? (bid % 8) * (grid / 8) + bid / 8 : bid;
  if (t >= ntiles) return false;
  constexpr int GM = 4;
  const int group = t / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  tm = first_m + (t % (GM * tiles_n)) % gsize;
  tn = (t % (GM * tiles_n)) / gsize;
  return true;
}

// Epilogue. Wave w is (wm, wn) = (w / WNW, w % WNW). With B passed as the
// first MFMA operand, accumulator t of tile (i, j) of the wave holds
// C[row][col] with row = m0 + 128 wm + 32 i + r (r = lane % 32) and
// col = n0 + 32 NT wn + 32 j + 8 (t / 4) + 4 g + (t % 4) (g = lane / 32): runs
// of 4 consecutive columns. Each wave stages its 128 x 32 NT block in LDS (its
// own region of `smem`, at least 2 WNW x 128 x (64 NT + 16) bytes; fp32 in
// two halves of 64 rows) and writes it back row-contiguously, 16 bytes per
// lane, so whole lines reach the L2, with non-temporal stores (the output is
// not read again here; 1.5% off the MXFP4 MLP-down GEMM). Values are multiplied by `scale`
// (exactly 1 unless a tensor scale applies). The caller has finished every use
// of `smem` and synchronised the workgroup.
template <int OUT, int NT = 4, int WNW = 2>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][NT], uint8_t* smem, float scale,
                                           void* __restrict__ C, int64_t ldc, int M, int N,
                                           int m0, int n0, int wave, int lane) {
  const int wm = wave / WNW, wn = wave % WNW;
  const int r = lane & 31, g = lane >> 5;
  constexpr int kCols = 32 * NT;                      // columns per wave
  constexpr int kEs = (OUT == kOutF32) ? 4 : 2;       // bytes per element
  constexpr int kRows = (OUT == kOutF32) ? 64 : 128;  // rows staged per pass
  constexpr int kPitch = kCols * kEs + 16;            // padded LDS row
  uint8_t* wbuf = smem + wave * (kRows * kPitch);
  const int wrow0 = m0 + wm * 128, wcol0 = n0 + wn * kCols;
  const bool vec_ok = (ldc % (16 / kEs)) == 0;
#pragma unroll
  for (int pass = 0; pass < 128 / kRows; pass++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if ((i * 32) / kRows != pass) continue;
      const int lrow = i * 32 + r - pass * kRows;
#pragma unroll
      for (int j = 0; j < NT; j++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int lcol = j * 32 + 8 * q + 4 * g;
          uint8_t* dst = wbuf + lrow * kPitch + lcol * kEs;
          const float v0 = acc[i][j][4 * q] * scale, v1 = acc[i][j][4 * q + 1] * scale;
          const float v2 = acc[i][j][4 * q + 2] * scale, v3 = acc[i][j][4 * q + 3] * scale;
          if (OUT == kOutF32)
            *(f32x4*)dst = f32x4{v0, v1, v2, v3};
          else
            *(u32x2*)dst = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        }
    }
    // Row-contiguous write-back: kCols columns, 16 bytes per lane; the wave
    // covers 64 / (lanes per row) rows per step.
    constexpr int kLanesPerRow = kCols * kEs / 16;
    constexpr int kRowsPerStep = 64 / kLanesPerRow;
#pragma unroll 4
    for (int rr = 0; rr < kRows; rr += kRowsPerStep) {
      const int lrow = rr + lane / kLanesPerRow;
      const int lcol = (lane % kLanesPerRow) * (16 / kEs);
      const int row = wrow0 + pass * kRows + lrow;
      const int col = wcol0 + lcol;
      if (row >= M) continue;
      const u32x4 v = *(const u32x4*)(wbuf + lrow * kPitch + lcol * kEs);
      uint8_t* gdst = (uint8_t*)C + ((int64_t)row * ldc + col) * kEs;
      if (vec_ok && col + 16 / kEs <= N) {
        __builtin_nontemporal_store(v, (u32x4*)gdst);
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 16 / kEs; e++) {
          if (col + e >= N) continue;
          if (OUT == kOutF32)
            ((uint32_t*)gdst)[e] = w[e];
          else
            ((uint16_t*)gdst)[e] = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
        }
      }
    }
  }
}

// fp32 accumulation in segments. A wave's fp32 accumulator chain over K is
// kept to at most 48 matrix instructions: after each segment the accumulators
// are added into the wave's block of the fp32 output C (stored on the first
// segment, one fp32 rounding per later one), then cleared. With every
// accumulation step rounding once, an output then errs by at most
// (48 + number of segments) * 2^-24 * sum|ab|, within 2^-18 * sum|ab| for up
// to 16 segments, where one chain over all of K (K / 64 steps for the FP4
// kernel, K / 16 for the 16-bit ones) could not guarantee it beyond 64 steps.
// On the last segment the sum is multiplied by `scale` (the NVFP4 tensor
// scales; 1 otherwise). Same element mapping as store_tile; each lane reads
// and writes its own runs of 4 columns directly (no LDS), so the fold needs no
// barrier. The caller zeroes the accumulators afterwards.
template <int NT = 4, int WNW = 2>
__device__ __forceinline__ void fold_tile(const f32x16 (&acc)[4][NT], float* __restrict__ C,
                                          int64_t ldc, int M, int N, int m0, int n0, int wave,
                                          int lane, bool first, bool last, float scale) {
  const int wm = wave / WNW, wn = wave % WNW;
  const int r = lane & 31, g = lane >> 5;
  constexpr int kCols = 32 * NT;
  const bool vec_ok = (ldc % 4) == 0;
  // This lane's stores of the previous segment are complete before it reads
  // them back (it only ever reads what it wrote itself).
  if (!first) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int row = m0 + wm * 128 + i * 32 + r;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < NT; j++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int col = n0 + wn * kCols + j * 32 + 8 * q + 4 * g;
        float* p = C + (int64_t)row * ldc + col;
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
        if (vec_ok && col + 4 <= N) {
          if (!first) {
            const f32x4 o = *(const f32x4*)p;
            v[0] += o.x;
            v[1] += o.y;
            v[2] += o.z;
            v[3] += o.w;
          }
          if (last) {
#pragma unroll
            for (int e = 0; e < 4; e++) v[e] *= scale;
          }
          *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++) {
            if (col + e >= N) continue;
            float w = v[e];
            if (!first) w += p[e];
            if (last) w *= scale;
            p[e] = w;
          }
        }
        // One run at a time: hoisting all 64 loads ahead would need 256 more
        // VGPRs in a kernel that has none to spare.
        __builtin_amdgcn_sched_barrier(0);
      }
  }
}

}  // namespace tile256
}  // namespace mx
