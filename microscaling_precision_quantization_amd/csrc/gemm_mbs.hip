// MXFP4-MBS x MXFP4-MBS GEMM for gfx950, the large-tile kernel.
//
// Static macro-block scaling (gist.science summary of "Unveiling the Potential
// of Quantization with MXFP4", section 2.B): every 1 x 128 macro block of a row
// carries a factor f = 1 + m / 256 on top of the MXFP4 E8M0 block scales, so
// an element is e * 2^(E-127) * f and
//   C[i][j] = sum over macro blocks q of f_A[i][q] f_B[j][q] P_q[i][j],
// P_q the block-scaled MXFP4 dot product over the 128 K of macro block q. The
// matrix core computes P_q (v_mfma_scale_f32_32x32x64_f8f6f4, two per macro
// block, the first from zero) and the vector ALU adds P_q * (f_A f_B) to the
// accumulator (f_A f_B has 18 significant bits: exact in fp32) -- the factor
// applied on the vector units alongside the matrix core, as the summary
// describes for its kernel.
//
// Design for CDNA4:
//  * The accumulators must sit in VGPRs next to the partial sums, so a wave
//    owns 128 x 64 outputs (4 x 2 MFMA tiles of 32 x 32, 128 accumulators per
//    lane) and a workgroup of 4 waves (one per SIMD) a 256 x 128 tile.
//  * K advances in super-steps of 256 (two macro blocks, 128 code bytes per
//    row). Codes and E8M0 scales go HBM -> LDS with buffer_load ... lds into a
//    2 x 54 KB double buffer; the next super-step's loads are issued between
//    the current one's MFMAs. The two macro-mantissa bytes per row come
//    through VGPRs and are stored in LDS as fp32 factors at the top of the
//    super-step they belong to.
//  * LDS rows are 128 bytes with the chunk swizzle c ^ ((r / 2) mod 8).
//  * K order inside a super-step, identical for A and B: sub-step J (0..3)
//    gives lane group g (lanes 32g .. 32g+31) code block 2J + g, so sub-steps
//    0, 1 cover macro block 0 and 2, 3 macro block 1. A lane's four scales
//    (blocks g, g+2, g+4, g+6 of its row) are gathered into one dword with
//    v_perm_b32, and opsel J picks byte J.
//  * XCD-aware tile order and the LDS-staged epilogue as in the other
//    large-tile kernels.
// 32x32x64 FP4 operand layout (measured): lane l = r + 32 g supplies 32 K
// elements of row r (16 bytes) and their E8M0 scale; output lane l holds
// column l % 32 and rows 8 (t / 4) + 4 g + (t % 4) of accumulator t. B goes
// first, so a lane holds one row of C (fixed f_A) and 16 columns.
#include "mx_internal.h"
#include "tile256.h"

namespace mx {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 128;
constexpr int kSuperK = 256;                        // elements per super-step
constexpr int kRowBytes = kSuperK / 2;              // 128 code bytes per row
constexpr int kOffB = BM * kRowBytes;               // 32 KB of A codes
constexpr int kOffSA = kOffB + BN * kRowBytes;      // + 16 KB of B codes
constexpr int kOffSB = kOffSA + BM * 8;             // + 2 KB of A scales (8 per row)
constexpr int kOffFA = kOffSB + BN * 8;             // + 1 KB of B scales
constexpr int kOffFB = kOffFA + 2 * BM * 4;         // + A factors [2][BM] fp32
constexpr int kStage = kOffFB + 2 * BN * 4;         // + B factors [2][BN] fp32
constexpr int kSmem = 2 * kStage;
constexpr uint32_t kRsrcFlags = 0x00020000u;        // raw buffer, gfx9 data format

static_assert(kSmem >= 4 * 128 * (64 * 2 + 16), "epilogue staging must fit");

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Part P (0..3) of the direct-to-LDS loads of super-step s: A code blocks 2P,
// 2P+1 and B code block P of this wave (1 KB = 8 rows each, lane l filling
// bytes 16l .. 16l+15 of the block), plus one 256-byte scale block (4 bytes per
// lane): A scales for P = 0, 1, B scales for P = 2.
template <int P>
__device__ __forceinline__ void issue_part(uint8_t* stage, __amdgpu_buffer_rsrc_t rA,
                                           __amdgpu_buffer_rsrc_t rB, __amdgpu_buffer_rsrc_t rSA,
                                           __amdgpu_buffer_rsrc_t rSB, uint32_t rowbytes,
                                           uint32_t scalebytes, int s, int wave, int lane) {
  const uint32_t kb = (uint32_t)s * kRowBytes;
#pragma unroll
  for (int i = 2 * P; i < 2 * P + 2; i++) {
    const int b = wave * 8 + i;
    const int row = b * 8 + (lane >> 3);
    const uint32_t off = kb + (uint32_t)(((lane & 7) ^ swz(row)) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(stage + b * 1024), 16,
                                             (uint32_t)row * rowbytes + off, 0, 0, 0);
  }
  {
    const int b = wave * 4 + P;
    const int row = b * 8 + (lane >> 3);
    const uint32_t off = kb + (uint32_t)(((lane & 7) ^ swz(row)) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr_t)(stage + kOffB + b * 1024), 16,
                                             (uint32_t)row * rowbytes + off, 0, 0, 0);
  }
  const uint32_t soff = (uint32_t)s * (kSuperK / 32) + (uint32_t)(lane & 1) * 4u;
  if (P < 2) {
    const int b = wave * 2 + P;  // 8 blocks of 32 rows x 8 bytes
    const int row = b * 32 + (lane >> 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rSA, (lds_ptr_t)(stage + kOffSA + b * 256), 4,
                                             (uint32_t)row * scalebytes + soff, 0, 0, 0);
  } else if (P == 2) {
    const int b = wave;  // 4 blocks
    const int row = b * 32 + (lane >> 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rSB, (lds_ptr_t)(stage + kOffSB + b * 256), 4,
                                             (uint32_t)row * scalebytes + soff, 0, 0, 0);
  }
}

// Macro mantissas of super-step s (two bytes per row) for A row `tid` and B
// row `tid` (tid < BN); rows past M or N read as 0 (factor 1).
__device__ __forceinline__ void load_macro(uint32_t& ma, uint32_t& mb, __amdgpu_buffer_rsrc_t rMA,
                                           __amdgpu_buffer_rsrc_t rMB, uint32_t macrobytes, int s,
                                           int tid) {
  ma = __builtin_amdgcn_raw_buffer_load_b16(rMA, (uint32_t)tid * macrobytes + 2u * s, 0, 0);
  mb = __builtin_amdgcn_raw_buffer_load_b16(rMB, (uint32_t)(tid & (BN - 1)) * macrobytes + 2u * s,
                                            0, 0);
}

__device__ __forceinline__ float macro_factor(uint32_t m) {
  return (float)(256u + m) * 0x1p-8f;
}

// Fragments of macro block q: A tiles i (rows wm*128 + 32 i + r) and B tiles j
// (rows wn*64 + 32 j + r), sub-steps 2q and 2q + 1.
struct Frags {
  i32x4 a[4][2], b[2][2];
};

__device__ __forceinline__ void load_frags(const uint8_t* cur, int q, int wm, int wn, int r, int g,
                                           Frags& f) {
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int c = 2 * (2 * q + h) + g;  // code block of this lane in sub-step 2q + h
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int ra = wm * 128 + i * 32 + r;
      f.a[i][h] = *(const i32x4*)(cur + ra * kRowBytes + ((c ^ swz(ra)) * 16));
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int rb = wn * 64 + j * 32 + r;
      f.b[j][h] = *(const i32x4*)(cur + kOffB + rb * kRowBytes + ((c ^ swz(rb)) * 16));
    }
  }
}

__device__ __forceinline__ i32x8 widen(i32x4 v) { return i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0}; }

// Macro block q of the current super-step: for each of the wave's 8 tiles,
// P = the two MFMAs of the block (the first from zero), then
// acc += P * (f_A f_B).
template <int Q>
__device__ __forceinline__ void macro_step(const uint8_t* cur, const Frags& f, const int (&sa)[4],
                                           const int (&sb)[2], int wm, int wn, int r, int g,
                                           f32x16 (&acc)[4][2]) {
  const float* FA = (const float*)(cur + kOffFA) + Q * BM;
  const float* FB = (const float*)(cur + kOffFB) + Q * BN;
  float fa[4];
#pragma unroll
  for (int i = 0; i < 4; i++) fa[i] = FA[wm * 128 + i * 32 + r];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    float fb[16];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const f32x4 v = *(const f32x4*)(FB + wn * 64 + j * 32 + 8 * u + 4 * g);
      fb[4 * u] = v.x;
      fb[4 * u + 1] = v.y;
      fb[4 * u + 2] = v.z;
      fb[4 * u + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          widen(f.b[j][0]), widen(f.a[i][0]), f32x16{}, 4, 4, 2 * Q, sb[j], 2 * Q, sa[i]);
      p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          widen(f.b[j][1]), widen(f.a[i][1]), p, 4, 4, 2 * Q + 1, sb[j], 2 * Q + 1, sa[i]);
#pragma unroll
      for (int t = 0; t < 16; t++) acc[i][j][t] = __builtin_fmaf(p[t], fa[i] * fb[t], acc[i][j][t]);
    }
  }
}

// The lane's four scale bytes of a row (blocks g, g+2, g+4, g+6 of the
// super-step) as one dword, byte J for sub-step J.
__device__ __forceinline__ int gather_scales(const uint8_t* srow, int g) {
  const u32x2 v = *(const u32x2*)srow;
  return (int)__builtin_amdgcn_perm(v.y, v.x, g ? 0x07050301u : 0x06040200u);
}

template <int OUT>
__global__ __launch_bounds__(kThreads, 1) void gemm_mbs_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ MA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB, const uint8_t* __restrict__ MB,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  int tm, tn;
  tile256::tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Buffer views based at the tile's first rows: rows past M or N read as 0.
  const uint32_t rowbytes = (uint32_t)(K / 2), scalebytes = (uint32_t)(K / 32);
  const uint32_t macrobytes = (uint32_t)(K / 128);
  const int mrows = min(BM, M - m0), nrows = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)m0 * rowbytes), 0, (int)(mrows * rowbytes), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void*)(B + (int64_t)n0 * rowbytes), 0, (int)(nrows * rowbytes), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rSA = __builtin_amdgcn_make_buffer_rsrc((void*)(SA + (int64_t)m0 * scalebytes), 0, (int)(mrows * scalebytes), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rSB = __builtin_amdgcn_make_buffer_rsrc((void*)(SB + (int64_t)n0 * scalebytes), 0, (int)(nrows * scalebytes), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rMA = __builtin_amdgcn_make_buffer_rsrc((void*)(MA + (int64_t)m0 * macrobytes), 0, (int)(mrows * macrobytes), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rMB = __builtin_amdgcn_make_buffer_rsrc((void*)(MB + (int64_t)n0 * macrobytes), 0, (int)(nrows * macrobytes), kRsrcFlags);

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  const int nsteps = K / kSuperK;
  uint32_t ma, mb;
  load_macro(ma, mb, rMA, rMB, macrobytes, 0, tid);
  issue_part<0>(smem, rA, rB, rSA, rSB, rowbytes, scalebytes, 0, wave, lane);
  issue_part<1>(smem, rA, rB, rSA, rSB, rowbytes, scalebytes, 0, wave, lane);
  issue_part<2>(smem, rA, rB, rSA, rSB, rowbytes, scalebytes, 0, wave, lane);
  issue_part<3>(smem, rA, rB, rSA, rSB, rowbytes, scalebytes, 0, wave, lane);
  for (int s = 0; s < nsteps; s++) {
    uint8_t* cur = smem + (s & 1) * kStage;
    uint8_t* nxt = smem + ((s + 1) & 1) * kStage;
    // Super-step s has landed (codes, scales and the macro bytes in VGPRs);
    // its factors go to LDS, then every wave may read it -- and every wave is
    // done with super-step s - 1, whose buffer receives s + 1 below.
    wait_vmem();
    {
      float* FA = (float*)(cur + kOffFA);
      float* FB = (float*)(cur + kOffFB);
      FA[tid] = macro_factor(ma & 0xFFu);
      FA[BM + tid] = macro_factor(ma >> 8);
      if (tid < BN) {
        FB[tid] = macro_factor(mb & 0xFFu);
        FB[BN + tid] = macro_factor(mb >> 8);
      }
    }
    __syncthreads();
    // Branch-free body: the last iteration re-fetches its own super-step into
    // the idle buffer, which nobody reads; the wait after the loop drains it.
    const int snext = min(s + 1, nsteps - 1);
    load_macro(ma, mb, rMA, rMB, macrobytes, snext, tid);
    int sa[4], sb[2];
#pragma unroll
    for (int i = 0; i < 4; i++) sa[i] = gather_scales(cur + kOffSA + (wm * 128 + i * 32 + r) * 8, g);
#pragma unroll
    for (int j = 0; j < 2; j++) sb[j] = gather_scales(cur + kOffSB + (wn * 64 + j * 32 + r) * 8, g);
    Frags f;
    load_frags(cur, 0, wm, wn, r, g, f);
    issue_part<0>(nxt, rA, rB, rSA, rSB, rowbytes, scalebytes, snext, wave, lane);
    issue_part<1>(nxt, rA, rB, rSA, rSB, rowbytes, scalebytes, snext, wave, lane);
    macro_step<0>(cur, f, sa, sb, wm, wn, r, g, acc);
    load_frags(cur, 1, wm, wn, r, g, f);
    issue_part<2>(nxt, rA, rB, rSA, rSB, rowbytes, scalebytes, snext, wave, lane);
    issue_part<3>(nxt, rA, rB, rSA, rSB, rowbytes, scalebytes, snext, wave, lane);
    macro_step<1>(cur, f, sa, sb, wm, wn, r, g, acc);
  }
  wait_vmem();

  // Epilogue: every load has drained; the stage buffers are free once every
  // wave is past its loop.
  __syncthreads();
  tile256::store_tile<OUT, 2>(acc, smem, 1.0f, C, ldc, M, N, m0, n0, wave, lane);
}

}  // namespace

// Whole super-steps along K, and 32-bit buffer offsets within a 256-row slab.
bool gemm_mbs_fits(int64_t M, int64_t N, int64_t K) {
  return K % kSuperK == 0 && (int64_t)BM * (K / 2) < ((int64_t)1 << 31) && M > 0 && N > 0;
}

hipError_t gemm_mbs(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                    const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                    hipStream_t s) {
  if (!gemm_mbs_fits(M, N, K))
    return gemm_mbs_small(M, N, K, a, sa, b, sb, out_dtype, c, ldc, s);
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(tm * tn));
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  const uint8_t* MA = SA + M * (K / 32);  // macro planes follow the E8M0 planes
  const uint8_t* MB = SB + N * (K / 32);
  if (out_dtype == kOutF32)
    gemm_mbs_kernel<kOutF32><<<grid, kThreads, 0, s>>>(A, SA, MA, B, SB, MB, c, ldc, (int)M,
                                                        (int)N, (int)K, tm, tn);
  else
    gemm_mbs_kernel<kOutBF16><<<grid, kThreads, 0, s>>>(A, SA, MA, B, SB, MB, c, ldc, (int)M,
                                                         (int)N, (int)K, tm, tn);
  return hipGetLastError();
}

}  // namespace mx
