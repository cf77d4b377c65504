// MXFP4-MBS x MXFP4-MBS GEMM for gfx950, the large-tile kernel.
//
// Static macro-block scaling (gist.science summary of "Unveiling the Potential
// of Quantization with MXFP4", section 2.B): every 1 x 128 macro block of a row
// carries a factor f = 1 + m / 256 on top of the MXFP4 E8M0 block scales, so
// an element is e * 2^(E-127) * f and
//   C[i][j] = sum over macro blocks q of f_A[i][q] f_B[j][q] P_q[i][j],
// P_q the block-scaled MXFP4 dot product over the 128 K of macro block q. The
// matrix core computes P_q (v_mfma_scale_f32_32x32x64_f8f6f4, two per macro
// block, the first from zero) and the tile of factor products f_A f_B (an
// fp16 MFMA of one nonzero K slot; f_A f_B has 18 significant bits, so it is
// exact), and the vector ALU adds P_q * (f_A f_B) to the accumulator with one
// fma per element -- the factor applied on the vector units alongside the
// matrix core, as the summary describes for its kernel.
//
// Design for CDNA4:
//  * The accumulators must sit in VGPRs next to the partial sums, so a wave
//    owns 128 x 64 outputs (4 x 2 MFMA tiles of 32 x 32, 128 accumulators per
//    lane). A workgroup of 8 waves (two per SIMD, each within 256 registers)
//    covers a 256 x 256 tile, which keeps the operand traffic through L2 at
//    that of the plain MXFP4 kernel; the SIMD's second wave hides each
//    wave's wait between its MFMAs and the vector ALU work that reads them.
//  * K advances in super-steps of 256 (two macro blocks, 128 code bytes per
//    row). Codes and E8M0 scales go HBM -> LDS with buffer_load ... lds into a
//    2 x 72 KB double buffer; the next super-step's loads are issued between
//    the current one's MFMAs. The two macro-mantissa bytes per row come
//    through VGPRs and are stored in LDS as fp16 factor operands at the top
//    of the super-step they belong to.
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 512;
constexpr int kWavesN = 4;                          // waves along N (2 along M)
constexpr int BM = 256, BN = 256;
constexpr int kSuperK = 256;                        // elements per super-step
constexpr int kRowBytes = kSuperK / 2;              // 128 code bytes per row
constexpr int kOffB = BM * kRowBytes;               // 32 KB of A codes
constexpr int kOffSA = kOffB + BN * kRowBytes;      // + 32 KB of B codes
// Then, per stage, the E8M0 scales of A and B (kSB = 8 bytes per row and
// super-step for 32-element base blocks, 16 for 16-element ones) and the
// macro factors: A factors / 2 [2][BM], B factors [2][BN] (fp16 in a dword).
template <int BASE>
struct Lds {
  static constexpr int kSB = kSuperK / BASE;
  static constexpr int kOffSB = kOffSA + BM * kSB;
  static constexpr int kOffFA = kOffSB + BN * kSB;
  static constexpr int kOffFB = kOffFA + 2 * BM * 4;
  static constexpr int kStage = kOffFB + 2 * BN * 4;
  static constexpr int kSmem = 2 * kStage;
  static_assert(kSmem >= 8 * 128 * (64 * 2 + 16), "epilogue staging must fit");
  static_assert(kSmem <= 160 * 1024, "LDS");
};
constexpr uint32_t kRsrcFlags = 0x00020000u;        // raw buffer, gfx9 data format

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Per-lane parts of the direct-to-LDS load addresses, the same for every
// super-step. The K offset of the super-step goes in the scalar offset; the
// row offsets stay in the lane offset, which the buffer range check sees, so
// rows past M or N still read as zeros.
// Code blocks are 8 rows of 128 bytes: lane l fills bytes 16 l .. 16 l + 15 of
// the LDS block, i.e. row l / 8, slot l % 8, which holds chunk
// slot ^ swz(row); for a block starting at row 8 b, swz(row) =
// (l / 16 + 4 (b % 2)) % 8, so two lane offsets (even / odd b) serve every
// code block of A and B. Scale blocks are 32 rows of 8 bytes, 4 per lane.
struct LaneOffsets {
  uint32_t code[2], scale;
};

template <int BASE>
__device__ __forceinline__ LaneOffsets lane_offsets(int lane, uint32_t rowbytes, uint32_t scalebytes) {
  LaneOffsets o;
#pragma unroll
  for (int par = 0; par < 2; par++)
    o.code[par] = (uint32_t)(lane >> 3) * rowbytes +
                  (uint32_t)(((lane & 7) ^ (((lane >> 4) + 4 * par) & 7)) * 16);
  // 4 bytes per lane: 2 lanes per row of 8 scale bytes, 4 per row of 16.
  if (BASE == 32)
    o.scale = (uint32_t)(lane >> 1) * scalebytes + (uint32_t)(lane & 1) * 4u;
  else
    o.scale = (uint32_t)(lane >> 2) * scalebytes + (uint32_t)(lane & 3) * 4u;
  return o;
}

// Part P (0..3) of the direct-to-LDS loads of super-step s: code block
// 4 wave + P of A and of B (1 KB = 8 rows each), plus the scales of 32 rows
// (8 or 16 bytes per row: one or two 256-byte loads of 4 bytes per lane):
// A's for P = 0, B's for P = 1. `wave` is wave-uniform.
template <int P, int BASE>
__device__ __forceinline__ void issue_part(uint8_t* stage, __amdgpu_buffer_rsrc_t rA,
                                           __amdgpu_buffer_rsrc_t rB, __amdgpu_buffer_rsrc_t rSA,
                                           __amdgpu_buffer_rsrc_t rSB, const LaneOffsets& lo,
                                           uint32_t rowbytes, uint32_t scalebytes, int s, int wave) {
  using L = Lds<BASE>;
  const uint32_t kb = (uint32_t)s * kRowBytes;
  const int b = wave * 4 + P;
  const uint32_t voff = lo.code[P & 1] + (uint32_t)(8 * b) * rowbytes;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(stage + b * 1024), 16, voff, (int)kb, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr_t)(stage + kOffB + b * 1024), 16, voff,
                                           (int)kb, 0, 0);
  const uint32_t ks = (uint32_t)s * L::kSB;
  const uint32_t soff = lo.scale + (uint32_t)(32 * wave) * scalebytes;
  // BASE 16: lane offsets cover 16 rows of 16 bytes per load, two loads.
  constexpr int kLoads = L::kSB / 8;
  if (P == 0 || P == 1) {
    const __amdgpu_buffer_rsrc_t rS = (P == 0) ? rSA : rSB;
    uint8_t* dst = stage + ((P == 0) ? kOffSA : L::kOffSB) + wave * 32 * L::kSB;
#pragma unroll
    for (int h = 0; h < kLoads; h++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_ptr_t)(dst + h * 256), 4,
                                               soff + (uint32_t)(16 * h) * scalebytes, (int)ks, 0, 0);
  }
}

// Macro mantissas of super-step s (two bytes per row): waves 0..3 load A row
// `tid`, waves 4..7 B row tid - 256; rows past M or N read as 0 (factor 1).
__device__ __forceinline__ uint32_t load_macro(__amdgpu_buffer_rsrc_t rM, uint32_t macrobytes, int s,
                                               int row) {
  return __builtin_amdgcn_raw_buffer_load_b16(rM, (uint32_t)row * macrobytes, 2 * s, 0);
}

// The macro factor times `w` (1 or 1/2), (1 + m/256) w, as fp16 bits in the
// low half of a dword (exact: 9 significant bits): one K slot of the factor
// MFMA's operand.
__device__ __forceinline__ uint32_t factor_bits(uint32_t m, float w) {
  const _Float16 h = (_Float16)((float)(256u + m) * 0x1p-8f * w);
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
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
// The first 16 codes of a lane's 32 (bytes 0..7), or the last 16, the other
// half zero.
__device__ __forceinline__ i32x8 lo16(i32x4 v) { return i32x8{v.x, v.y, 0, 0, 0, 0, 0, 0}; }
__device__ __forceinline__ i32x8 hi16(i32x4 v) { return i32x8{0, 0, v.z, v.w, 0, 0, 0, 0}; }

// A lane's E8M0 scale bytes for the super-step, byte J for sub-step J: for
// 32-element base blocks one dword per row (a, b); for 16-element ones the
// scale of the first 16 codes (a, b) and of the last 16 (a2, b2).
struct Scales {
  int a[4], b[2], a2[4], b2[2];
};

// The MFMAs of tile (i, j) in macro block Q: the block-scaled partial sum
// over its 128 K, the first from zero. BASE 32: two MFMAs, each lane's 32
// codes under one scale. BASE 16: the scaled MFMA takes one scale per lane's
// 32 codes, so each 32 is split into two MFMAs over its halves, each under
// its own 16-block scales -- exact, at twice the MFMAs. Only the B operand
// needs its other half zeroed (bl / bh, built once per B tile by the
// caller): A's codes there then meet zeros, and every code times a finite
// scale is finite (a NaN scale, 255, makes the output NaN either way, as the
// block it belongs to does).
template <int Q, int BASE>
__device__ __forceinline__ f32x16 partial(const Frags& f, const Scales& sc, int i, int j,
                                          const i32x8 (&bl)[2], const i32x8 (&bh)[2]) {
  if (BASE == 32) {
    f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        widen(f.b[j][0]), widen(f.a[i][0]), f32x16{}, 4, 4, 2 * Q, sc.b[j], 2 * Q, sc.a[i]);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        widen(f.b[j][1]), widen(f.a[i][1]), p, 4, 4, 2 * Q + 1, sc.b[j], 2 * Q + 1, sc.a[i]);
  }
  f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      bl[0], widen(f.a[i][0]), f32x16{}, 4, 4, 2 * Q, sc.b[j], 2 * Q, sc.a[i]);
  p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      bh[0], widen(f.a[i][0]), p, 4, 4, 2 * Q, sc.b2[j], 2 * Q, sc.a2[i]);
  p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      bl[1], widen(f.a[i][1]), p, 4, 4, 2 * Q + 1, sc.b[j], 2 * Q + 1, sc.a[i]);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      bh[1], widen(f.a[i][1]), p, 4, 4, 2 * Q + 1, sc.b2[j], 2 * Q + 1, sc.a2[i]);
}

// Macro block Q of the current super-step, tile by tile over the wave's 8
// tiles k = (i = k % 4, j = k / 4): the matrix core computes the partial sum
// P_k (two FP4 MFMAs) and the factor tile G_k = f_B (x) f_A (one fp16 MFMA:
// each lane supplies its row's f_B, or f_A / 2, in the first K slot of its
// half of K and zeros elsewhere, so G_k = 2 f_B (f_A / 2) = f_A f_B exactly,
// laid out like P_k); the vector ALU then does acc += P_k * G_k. One tile is
// in flight per wave (fences keep the compiler from hoisting the next tile's
// MFMAs, which would not fit in 256 registers); the SIMD's other wave fills
// the wait between a tile's MFMAs and its ALU work.
template <int Q, int BASE>
__device__ __forceinline__ void macro_step(const uint8_t* cur, const Frags& f, const Scales& sc,
                                           int wm, int wn, int r, f32x16 (&acc)[4][2]) {
  const uint32_t* FA = (const uint32_t*)(cur + Lds<BASE>::kOffFA) + Q * BM;
  const uint32_t* FB = (const uint32_t*)(cur + Lds<BASE>::kOffFB) + Q * BN;
  // The block's factor operands, read once (one dword per tile row).
  uint32_t fa[4], fb[2];
#pragma unroll
  for (int i = 0; i < 4; i++) fa[i] = FA[wm * 128 + i * 32 + r];
#pragma unroll
  for (int j = 0; j < 2; j++) fb[j] = FB[wn * 64 + j * 32 + r];
  i32x8 bl[2], bh[2];  // BASE 16: B's halves of the current j, the other half zero
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int i = k & 3, j = k >> 2;
    if (BASE == 16 && i == 0) {
#pragma unroll
      for (int h = 0; h < 2; h++) {
        bl[h] = lo16(f.b[j][h]);
        bh[h] = hi16(f.b[j][h]);
      }
    }
    sched_fence();
    // The factor MFMA first: it runs while the dependent pair of P waits.
    const f32x16 gk = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(f16x4, u32x2{fb[j], 0u}),
                                                            __builtin_bit_cast(f16x4, u32x2{fa[i], 0u}),
                                                            f32x16{}, 0, 0, 0);
    const f32x16 p = partial<Q, BASE>(f, sc, i, j, bl, bh);
#pragma unroll
    for (int t = 0; t < 16; t++) acc[i][j][t] = __builtin_fmaf(p[t], gk[t], acc[i][j][t]);
  }
  sched_fence();
}

// The lane's four scale bytes of a row (blocks g, g+2, g+4, g+6 of the
// super-step) as one dword, byte J for sub-step J.
__device__ __forceinline__ int gather_scales(const uint8_t* srow, int g) {
  const u32x2 v = *(const u32x2*)srow;
  return (int)__builtin_amdgcn_perm(v.y, v.x, g ? 0x07050301u : 0x06040200u);
}

// BASE 16: the row's 16 scale bytes; sub-step J's 32 codes of lane group g
// are 16-blocks 4 J + 2 g (first half) and 4 J + 2 g + 1 (second half), i.e.
// byte 2 g (or 2 g + 1) of dword J.
__device__ __forceinline__ void gather_scales16(const uint8_t* srow, int g, int& lo, int& hi) {
  const u32x4 v = *(const u32x4*)srow;
  const int sl = 16 * g, sh = 16 * g + 8;
  lo = (int)(((v.x >> sl) & 0xFFu) | (((v.y >> sl) & 0xFFu) << 8) | (((v.z >> sl) & 0xFFu) << 16) |
             (((v.w >> sl) & 0xFFu) << 24));
  hi = (int)(((v.x >> sh) & 0xFFu) | (((v.y >> sh) & 0xFFu) << 8) | (((v.z >> sh) & 0xFFu) << 16) |
             (((v.w >> sh) & 0xFFu) << 24));
}

// Super-steps per fp32 accumulation segment (48 macro blocks).
constexpr int kSeg = 24;

template <int OUT, int BASE>
__global__ __launch_bounds__(kThreads, 1) void gemm_mbs_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ MA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB, const uint8_t* __restrict__ MB,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_n) {
  using L = Lds<BASE>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L::kSmem];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int r = lane & 31, g = lane >> 5;
  const bool a_side = wave < 4;               // which operand's macro row this thread loads
  const int mrow = a_side ? tid : tid - BM;
  int tm, tn;
  tile256::tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Buffer views based at the tile's first rows: rows past M or N read as 0.
  const uint32_t rowbytes = (uint32_t)(K / 2), scalebytes = (uint32_t)(K / BASE);
  const uint32_t macrobytes = (uint32_t)(K / 128);
  const LaneOffsets lo = lane_offsets<BASE>(lane, rowbytes, scalebytes);
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
  const __amdgpu_buffer_rsrc_t rM = a_side ? rMA : rMB;
  uint32_t mv = load_macro(rM, macrobytes, 0, mrow);
  issue_part<0, BASE>(smem, rA, rB, rSA, rSB, lo, rowbytes, scalebytes, 0, wave);
  issue_part<1, BASE>(smem, rA, rB, rSA, rSB, lo, rowbytes, scalebytes, 0, wave);
  issue_part<2, BASE>(smem, rA, rB, rSA, rSB, lo, rowbytes, scalebytes, 0, wave);
  issue_part<3, BASE>(smem, rA, rB, rSA, rSB, lo, rowbytes, scalebytes, 0, wave);
  for (int s = 0; s < nsteps; s++) {
    uint8_t* cur = smem + (s & 1) * L::kStage;
    uint8_t* nxt = smem + ((s + 1) & 1) * L::kStage;
    // Super-step s has landed (codes, scales and the macro bytes in VGPRs);
    // its factors go to LDS, then every wave may read it -- and every wave is
    // done with super-step s - 1, whose buffer receives s + 1 below.
    wait_vmem();
    {
      // A factors are stored halved: the factor MFMA sums two K slots.
      uint32_t* F = (uint32_t*)(cur + (a_side ? L::kOffFA : L::kOffFB));
      const float w = a_side ? 0.5f : 1.0f;
      F[mrow] = factor_bits(mv & 0xFFu, w);
      F[BM + mrow] = factor_bits(mv >> 8, w);
    }
    __syncthreads();
    // Branch-free body: the last iteration re-fetches its own super-step into
    // the idle buffer, which nobody reads; the wait after the loop drains it.
    const int snext = min(s + 1, nsteps - 1);
    mv = load_macro(rM, macrobytes, snext, mrow);
    Scales sc;
    if (BASE == 32) {
#pragma unroll
      for (int i = 0; i < 4; i++) sc.a[i] = gather_scales(cur + kOffSA + (wm * 128 + i * 32 + r) * 8, g);
#pragma unroll
      for (int j = 0; j < 2; j++) sc.b[j] = gather_scales(cur + L::kOffSB + (wn * 64 + j * 32 + r) * 8, g);
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++)
        gather_scales16(cur + kOffSA + (wm * 128 + i * 32 + r) * 16, g, sc.a[i], sc.a2[i]);
#pragma unroll
      for (int j = 0; j < 2; j++)
        gather_scales16(cur + L::kOffSB + (wn * 64 + j * 32 + r) * 16, g, sc.b[j], sc.b2[j]);
    }
    Frags f;
    load_frags(cur, 0, wm, wn, r, g, f);
    issue_part<0, BASE>(nxt, rA, rB, rSA, rSB, lo, rowbytes, scalebytes, snext, wave);
    issue_part<1, BASE>(nxt, rA, rB, rSA, rSB, lo, rowbytes, scalebytes, snext, wave);
    macro_step<0, BASE>(cur, f, sc, wm, wn, r, acc);
    load_frags(cur, 1, wm, wn, r, g, f);
    issue_part<2, BASE>(nxt, rA, rB, rSA, rSB, lo, rowbytes, scalebytes, snext, wave);
    issue_part<3, BASE>(nxt, rA, rB, rSA, rSB, lo, rowbytes, scalebytes, snext, wave);
    macro_step<1, BASE>(cur, f, sc, wm, wn, r, acc);
    // fp32 output: the fma chain into the accumulators is kept to kSeg
    // macro blocks (2 per super-step), each segment folded into C.
    if (OUT == kOutF32 && nsteps > kSeg && ((s + 1) % kSeg == 0 || s + 1 == nsteps)) {
      tile256::fold_tile<2, kWavesN>(acc, (float*)C, ldc, M, N, m0, n0, wave, lane, s + 1 == kSeg,
                                     s + 1 == nsteps, 1.0f);
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
          for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;
    }
  }
  wait_vmem();
  if (OUT == kOutF32 && nsteps > kSeg) return;

  // Epilogue: every load has drained; the stage buffers are free once every
  // wave is past its loop.
  __syncthreads();
  tile256::store_tile<OUT, 2, kWavesN>(acc, smem, 1.0f, C, ldc, M, N, m0, n0, wave, lane);
}

}  // namespace

// Whole super-steps along K, and 32-bit buffer offsets within a 256-row slab.
bool gemm_mbs_fits(int64_t M, int64_t N, int64_t K) {
  return K % kSuperK == 0 && (int64_t)BM * (K / 2) < ((int64_t)1 << 31) && M > 0 && N > 0;
}

hipError_t gemm_mbs(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                    const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                    hipStream_t s, int base) {
  if (!gemm_mbs_fits(M, N, K))
    return gemm_mbs_small(M, N, K, a, sa, b, sb, out_dtype, c, ldc, s, base);
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(tm * tn));
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  const uint8_t* MA = SA + M * (K / base);  // macro planes follow the E8M0 planes
  const uint8_t* MB = SB + N * (K / base);
  const int m = (int)M, n = (int)N, k = (int)K;
  if (base == 16) {
    if (out_dtype == kOutF32)
      return launch_kernel(&gemm_mbs_kernel<kOutF32, 16>, grid, kThreads, 0, s, A, SA, MA, B, SB, MB, c, ldc, m, n, k, tm, tn);
    return launch_kernel(&gemm_mbs_kernel<kOutBF16, 16>, grid, kThreads, 0, s, A, SA, MA, B, SB, MB, c, ldc, m, n, k, tm, tn);
  }
  if (out_dtype == kOutF32)
    return launch_kernel(&gemm_mbs_kernel<kOutF32, 32>, grid, kThreads, 0, s, A, SA, MA, B, SB, MB, c, ldc, m, n, k, tm, tn);
  return launch_kernel(&gemm_mbs_kernel<kOutBF16, 32>, grid, kThreads, 0, s, A, SA, MA, B, SB, MB, c, ldc, m, n, k, tm, tn);
}

}  // namespace mx
