// MXFP4 x MXFP4 block-scaled GEMM for gfx950, the large-tile kernel.
//
// C = A * B^T with A: M x K E2M1 codes, B: N x K codes (the Linear weight
// layout), one E8M0 scale per 32 K per row. The matrix core applies both E8M0
// scales during its fp32 accumulation (v_mfma_scale_f32_32x32x64_f8f6f4), so
// codes travel from HBM to the MFMA unexpanded -- the block-scaled dot product
// described in "Arquitetura Blackwell SM100 e aceleracao nativa de NVFP4" on
// the produtoramaxvision page (there for B200 tensor cores).
//
// Design for CDNA4:
//  * 256 x 256 output tile per workgroup, 4 waves (one per SIMD) of 128 x 128,
//    each wave 4 x 4 MFMAs of 32 x 32 with 256 fp32 accumulators per lane.
//  * K advances in super-steps of 256 elements (128 code bytes per row). A
//    super-step (both code tiles and their scales, 68 KB) moves through a
//    three-deep pipeline: global -> VGPRs (16-byte buffer loads, issued two
//    super-steps ahead), VGPRs -> LDS (ds_write, one super-step ahead, into
//    the idle half of a 2 x 68 KB double buffer), LDS -> MFMA. With both
//    operands in K panels there are two register stages and the loads go
//    three super-steps ahead (four-deep), which pays at sustained clocks.
//    The barrier between super-steps waits for LDS work only, so global loads
//    stay in flight across it. Buffer range checking returns zeros for rows
//    past M or N.
//  * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at slot
//    c ^ ((r / 2) mod 8) so that the lanes reading one column of chunks hit
//    distinct banks (measured with the LDS bank-conflict counter).
//  * K order inside a super-step is permuted identically for A and B: the MFMA
//    of sub-step j gives lane group g (lanes 32g .. 32g+31) code block 4g + j.
//    A lane therefore owns 4 consecutive blocks of its row: its 4 scales are
//    one dword, and opsel j picks byte j for sub-step j.
//  * Workgroup ids are remapped so that each XCD (ids round-robin over 8
//    XCDs) gets a contiguous, grouped block of output tiles and its L2 serves
//    the shared A rows and B columns.
//  * A and B may come in the K-panel layout (mx_pack, or mx_quantize_ex's
//    panel output): the 128 code bytes of all rows for one super-step back to
//    back, so a tile's loads of one super-step cover one contiguous 32 KB
//    range instead of 256 pieces of 128 bytes K / 2 bytes apart, which keeps
//    the HBM reads in open DRAM pages. The buffer view is then rebuilt per
//    super-step to span that panel's rows, so rows past M or N still fall
//    outside its range.
// 32x32x64 FP4 operand layout (measured): lane l = r + 32 g supplies K
// elements [32g, 32g + 32) of row r (16 bytes, even element in the low
// nibble) and the E8M0 scale of that K block; the output lane l holds column
// l % 32 and rows 8 (t / 4) + 4 g + (t % 4) in accumulator t. The kernel passes
// B as the first operand, so the output tile is C^T and each lane holds runs
// of 4 consecutive columns of one row of C.
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

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256;
constexpr int kSuperK = 256;                       // elements per super-step
constexpr int kRowBytes = kSuperK / 2;             // 128 code bytes per row
constexpr int kTileBytes = BM * kRowBytes;         // 32 KB per operand
constexpr int kScaleBytes = BM * (kSuperK / 32);   // 2 KB per operand (8 per row)
constexpr int kStage = 2 * kTileBytes + 2 * kScaleBytes;
constexpr uint32_t kRsrcFlags = 0x00020000u;       // raw buffer, gfx9 data format

// LDS swizzle: the 16-byte chunk c of tile row r lives in slot c ^ swz(r).
// gfx950's LDS serves a ds_read_b128 16 lanes at a time across 64 banks
// (256 bytes); two 128-byte rows share that window, so the 16 rows read by one
// group must spread over 8 slots per row parity: swz(r) = (r / 2) mod 8.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// One wave's share of a super-step, staged in registers: 8 KB of each code
// tile (8 blocks of 8 rows x 128 B; lane l holds 16 bytes of row l / 8) and
// 512 B of each scale tile (64 rows x 8 B, one row per lane).
struct Stage {
  i32x4 a[8], b[8];
  u32x2 sa, sb;
};

// Part P (0..3) of the global loads of super-step s: code blocks 2P and 2P+1
// of A and B, plus the A scales (P = 0) or the B scales (P = 1). Rows past M
// or N fall outside the buffer range and load as zeros.
// An operand in the K-panel layout (PANEL_A, PANEL_B): panel s of the codes
// starts at byte s * rows * 128, of the scales at s * rows * 8; its buffer
// views span the panel's rows.
template <int P, bool PANEL_A, bool PANEL_B>
__device__ __forceinline__ void load_part(Stage& st, __amdgpu_buffer_rsrc_t rA,
                                          __amdgpu_buffer_rsrc_t rB, __amdgpu_buffer_rsrc_t rSA,
                                          __amdgpu_buffer_rsrc_t rSB, int m0, int n0,
                                          uint32_t rowbytes, uint32_t scalebytes, int s, int wave,
                                          int lane, const uint8_t* A, const uint8_t* SA, int M,
                                          const uint8_t* B, const uint8_t* SB, int N) {
  const uint32_t kb = (uint32_t)s * kRowBytes;
#pragma unroll
  for (int i = 2 * P; i < 2 * P + 2; i++) {
    const int row = (wave * 8 + i) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);  // slot lane&7 of the LDS row holds this chunk
    const uint32_t off = kb + (uint32_t)chunk * 16u;
    if (PANEL_A) {
      const __amdgpu_buffer_rsrc_t rAp = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(A + (int64_t)s * M * kRowBytes), 0, M * kRowBytes, kRsrcFlags);
      st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rAp, (uint32_t)(m0 + row) * (uint32_t)kRowBytes + (uint32_t)chunk * 16u, 0, 0);
    } else {
      st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, (uint32_t)(m0 + row) * rowbytes + off, 0, 0);
    }
    if (PANEL_B) {
      const __amdgpu_buffer_rsrc_t rBp = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(B + (int64_t)s * N * kRowBytes), 0, N * kRowBytes, kRsrcFlags);
      st.b[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rBp, (uint32_t)(n0 + row) * (uint32_t)kRowBytes + (uint32_t)chunk * 16u, 0, 0);
    } else {
      st.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, (uint32_t)(n0 + row) * rowbytes + off, 0, 0);
    }
  }
  const int srow = wave * 64 + lane;
  const uint32_t soff = (uint32_t)s * (kSuperK / 32);
  if (P == 0) {
    if (PANEL_A) {
      const __amdgpu_buffer_rsrc_t rSAp = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(SA + (int64_t)s * M * (kSuperK / 32)), 0, M * (kSuperK / 32), kRsrcFlags);
      st.sa = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                            rSAp, (uint32_t)(m0 + srow) * (uint32_t)(kSuperK / 32), 0, 0));
    } else {
      st.sa = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                            rSA, (uint32_t)(m0 + srow) * scalebytes + soff, 0, 0));
    }
  }
  if (P == 1) {
    if (PANEL_B) {
      const __amdgpu_buffer_rsrc_t rSBp = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(SB + (int64_t)s * N * (kSuperK / 32)), 0, N * (kSuperK / 32), kRsrcFlags);
      st.sb = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                            rSBp, (uint32_t)(n0 + srow) * (uint32_t)(kSuperK / 32), 0, 0));
    } else {
      st.sb = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                            rSB, (uint32_t)(n0 + srow) * scalebytes + soff, 0, 0));
    }
  }
}

// Part P of the LDS writes of a staged super-step (the same pieces as
// load_part<P>). Code rows are 128 bytes with the chunk swizzle applied by
// the loads; scales are 8 bytes per row.
template <int P>
__device__ __forceinline__ void store_part(const Stage& st, uint8_t* stage, int wave, int lane) {
#pragma unroll
  for (int i = 2 * P; i < 2 * P + 2; i++) {
    *(i32x4*)(stage + (wave * 8 + i) * 1024 + lane * 16) = st.a[i];
    *(i32x4*)(stage + kTileBytes + (wave * 8 + i) * 1024 + lane * 16) = st.b[i];
  }
  if (P == 0) *(u32x2*)(stage + 2 * kTileBytes + (wave * 64 + lane) * 8) = st.sa;
  if (P == 1) *(u32x2*)(stage + 2 * kTileBytes + kScaleBytes + (wave * 64 + lane) * 8) = st.sb;
}

// Operand fragments of one 64-element sub-step: 4 A and 4 B tiles of 32 rows,
// 16 code bytes per lane each.
struct Frags {
  i32x4 a[4], b[4];
};

template <int J>
__device__ __forceinline__ void load_frags(const uint8_t* As, const uint8_t* Bs, int wm, int wn,
                                           int r, int g, Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int ra = wm * 128 + i * 32 + r;
    const int rb = wn * 128 + i * 32 + r;
    f.a[i] = *(const i32x4*)(As + ra * kRowBytes + (((4 * g + J) ^ swz(ra)) * 16));
    f.b[i] = *(const i32x4*)(Bs + rb * kRowBytes + (((4 * g + J) ^ swz(rb)) * 16));
  }
}

template <int J>
__device__ __forceinline__ void mfma_substep(const Frags& f, const int (&sa)[4], const int (&sb)[4],
                                             f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const i32x8 a = i32x8{f.a[i].x, f.a[i].y, f.a[i].z, f.a[i].w, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const i32x8 b = i32x8{f.b[j].x, f.b[j].y, f.b[j].z, f.b[j].w, 0, 0, 0, 0};
      // Operands swapped (B first): the result tile is C^T, so a lane ends up
      // with 4 consecutive output columns of one output row.
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[i][j], 4, 4, J, sb[j],
                                                                  J, sa[i]);
    }
  }
}

// Keep the compiler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Issue order of one region of 16 MFMAs (sched_group_barrier masks: 0x008
// MFMA, 0x100 LDS read, 0x200 LDS write, 0x020 VMEM read), closed by a fence:
// the next sub-step's 8 fragment reads go out within the first 4 MFMAs, so
// they reach the LDS queue ahead of the other waves' staging writes and land
// before the region ends; then the global loads, then the LDS writes of the
// staged super-step, which are only needed by the next barrier.
template <bool WITH_READS>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int k = 0; k < 4; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (WITH_READS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
#pragma unroll
  for (int k = 0; k < 5; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
#pragma unroll
  for (int k = 0; k < 5; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  __builtin_amdgcn_sched_barrier(0);
}

template <int OUT, bool PANEL_A, bool PANEL_B>
__global__ __launch_bounds__(kThreads, 1) void gemm_mxfp4_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, void* __restrict__ C, int64_t ldc, int M, int N, int K,
    int tiles_m, int tiles_n) {
  // Both operands in K panels (the layout of the benchmarked step): two
  // register stages fit without spills in the loop; the other layouts keep one.
  constexpr bool DEEP = PANEL_A && PANEL_B;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;

  int tm, tn;
  tile256::tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const uint32_t rowbytes = (uint32_t)(K / 2), scalebytes = (uint32_t)(K / 32);
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, (int)((uint32_t)M * rowbytes), kRsrcFlags);
  // (unused for a K-panel B, whose views are made per super-step)
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void*)B, 0, (int)((uint32_t)N * rowbytes), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rSA = __builtin_amdgcn_make_buffer_rsrc((void*)SA, 0, (int)((uint32_t)M * scalebytes), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rSB = __builtin_amdgcn_make_buffer_rsrc((void*)SB, 0, (int)((uint32_t)N * scalebytes), kRsrcFlags);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  const int nsteps = K / kSuperK;
  // One super-step: MFMAs on LDS buffer s & 1 while the registers Rx (super-
  // step s + 1) go to LDS buffer (s + 1) & 1 and then receive super-step
  // s + ahead from memory.
  auto step = [&](int s, Stage& Rx, int ahead) {
    // Every wave's LDS writes of super-step s are done and every wave is done
    // reading super-step s-1, whose buffer receives super-step s+1 below. Only
    // LDS work is waited for: the global loads stay in flight.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    sched_fence();
    const uint8_t* cur = smem + (s & 1) * kStage;
    uint8_t* nxt = smem + ((s + 1) & 1) * kStage;
    // Branch-free body (a branch here lets the compiler sink the MFMAs): the
    // last iterations re-stage the final super-step into the idle buffer.
    // The registers Rx hold super-step s + 1 and then receive s + ahead.
    const int s2 = min(s + ahead, nsteps - 1);
    const uint8_t* As = cur;
    const uint8_t* Bs = cur + kTileBytes;
    const uint8_t* SAs = cur + 2 * kTileBytes;
    const uint8_t* SBs = SAs + kScaleBytes;
    int sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sa[i] = *(const int*)(SAs + (wm * 128 + i * 32 + r) * 8 + g * 4);
      sb[i] = *(const int*)(SBs + (wn * 128 + i * 32 + r) * 8 + g * 4);
    }
    // Each of the 4 regions below issues the 16 MFMAs of one sub-step, the 8
    // LDS reads of the next sub-step's fragments, a quarter of the staged
    // super-step's LDS writes and a quarter of the next global loads,
    // interleaved so that each memory instruction issues in an MFMA's shadow.
    Frags f0, f1;
    load_frags<0>(As, Bs, wm, wn, r, g, f0);
    sched_fence();
    load_frags<1>(As, Bs, wm, wn, r, g, f1);
    store_part<0>(Rx, nxt, wave, lane);
    load_part<0, PANEL_A, PANEL_B>(Rx, rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, s2, wave, lane, A, SA, M, B, SB, N);
    mfma_substep<0>(f0, sa, sb, acc);
    interleave<true>();
    load_frags<2>(As, Bs, wm, wn, r, g, f0);
    store_part<1>(Rx, nxt, wave, lane);
    load_part<1, PANEL_A, PANEL_B>(Rx, rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, s2, wave, lane, A, SA, M, B, SB, N);
    mfma_substep<1>(f1, sa, sb, acc);
    interleave<true>();
    load_frags<3>(As, Bs, wm, wn, r, g, f1);
    store_part<2>(Rx, nxt, wave, lane);
    load_part<2, PANEL_A, PANEL_B>(Rx, rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, s2, wave, lane, A, SA, M, B, SB, N);
    mfma_substep<2>(f0, sa, sb, acc);
    interleave<true>();
    store_part<3>(Rx, nxt, wave, lane);
    load_part<3, PANEL_A, PANEL_B>(Rx, rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, s2, wave, lane, A, SA, M, B, SB, N);
    mfma_substep<3>(f1, sa, sb, acc);
    interleave<false>();
  };
  // Super-step 0 goes to LDS buffer 0 through the registers first.
  Stage R[DEEP ? 2 : 1];
  load_part<0, PANEL_A, PANEL_B>(R[0], rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, 0, wave, lane, A, SA, M, B, SB, N);
  load_part<1, PANEL_A, PANEL_B>(R[0], rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, 0, wave, lane, A, SA, M, B, SB, N);
  load_part<2, PANEL_A, PANEL_B>(R[0], rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, 0, wave, lane, A, SA, M, B, SB, N);
  load_part<3, PANEL_A, PANEL_B>(R[0], rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, 0, wave, lane, A, SA, M, B, SB, N);
  store_part<0>(R[0], smem, wave, lane);
  store_part<1>(R[0], smem, wave, lane);
  store_part<2>(R[0], smem, wave, lane);
  store_part<3>(R[0], smem, wave, lane);
  // Then the register stages are filled with super-steps 1 (and 2), issued in
  // the loop's order (the fences keep the scheduler from reordering them), so
  // that the in-order load counter lets the loop's first LDS writes wait only
  // for their own part.
#pragma unroll
  for (int x = 0; x < (DEEP ? 2 : 1); x++) {
    const int sx = min(1 + x, nsteps - 1);
    sched_fence();
    load_part<0, PANEL_A, PANEL_B>(R[x], rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, sx, wave, lane, A, SA, M, B, SB, N);
    sched_fence();
    load_part<1, PANEL_A, PANEL_B>(R[x], rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, sx, wave, lane, A, SA, M, B, SB, N);
    sched_fence();
    load_part<2, PANEL_A, PANEL_B>(R[x], rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, sx, wave, lane, A, SA, M, B, SB, N);
    sched_fence();
    load_part<3, PANEL_A, PANEL_B>(R[x], rA, rB, rSA, rSB, m0, n0, rowbytes, scalebytes, sx, wave, lane, A, SA, M, B, SB, N);
    sched_fence();
  }
  // fp32 output with more than kSeg super-steps: K in segments of kSeg
  // super-steps (48 MFMAs per chain), each folded into C
  // (tile256::fold_tile); otherwise one chain. The pipeline runs on across
  // segment boundaries; kSeg is even, so every segment but the last starts
  // and ends on the same register stage.
  constexpr int kSeg = 12;
  auto run = [&](int s0, int s1) {
    if (DEEP) {
      // Four-deep pipeline: two register stages alternate, so every load has
      // two super-steps to land.
      int s = s0;
      for (; s + 1 < s1; s += 2) {
        step(s, R[0], 3);
        step(s + 1, R[DEEP ? 1 : 0], 3);
      }
      if (s < s1) step(s, R[0], 3);
    } else {
      // Three-deep pipeline: one register stage, each load has one super-step.
      for (int s = s0; s < s1; s++) step(s, R[0], 2);
    }
  };
  if constexpr (OUT == kOutF32) {
    if (nsteps > kSeg) {
      for (int s0 = 0; s0 < nsteps; s0 += kSeg) {
        const int s1 = min(s0 + kSeg, nsteps);
        run(s0, s1);
        tile256::fold_tile(acc, (float*)C, ldc, M, N, m0, n0, wave, lane, s0 == 0, s1 == nsteps, 1.0f);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int j = 0; j < 4; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;
      }
      return;
    }
  }
  run(0, nsteps);

  // Epilogue: the stage buffers are free once every wave is past its loop.
  __syncthreads();
  tile256::store_tile<OUT>(acc, smem, 1.0f, C, ldc, M, N, m0, n0, wave, lane);
}

}  // namespace

// The large-tile kernel needs whole super-steps along K and 32-bit buffer
// offsets (including the zero-filled rows past the last tile).
bool gemm_mxfp4_fits(int64_t M, int64_t N, int64_t K) {
  if (K % kSuperK != 0) return false;
  const int64_t lim = (int64_t)1 << 31;
  return (M + BM) * (K / 2) < lim && (N + BN) * (K / 2) < lim;
}

template <int OUT>
hipError_t launch(dim3 grid, hipStream_t s, bool panel_a, bool panel_b, const uint8_t* A,
            const uint8_t* SA, const uint8_t* B, const uint8_t* SB, void* c, int64_t ldc, int m,
            int n, int k, int tm, int tn) {
  if (panel_a && panel_b)
    MX_TRY(launch_kernel(&gemm_mxfp4_kernel<OUT, true, true>, grid, kThreads, 0, s, A, SA, B, SB, c, ldc, m, n, k, tm, tn));
  else if (panel_a)
    MX_TRY(launch_kernel(&gemm_mxfp4_kernel<OUT, true, false>, grid, kThreads, 0, s, A, SA, B, SB, c, ldc, m, n, k, tm, tn));
  else if (panel_b)
    MX_TRY(launch_kernel(&gemm_mxfp4_kernel<OUT, false, true>, grid, kThreads, 0, s, A, SA, B, SB, c, ldc, m, n, k, tm, tn));
  else
    MX_TRY(launch_kernel(&gemm_mxfp4_kernel<OUT, false, false>, grid, kThreads, 0, s, A, SA, B, SB, c, ldc, m, n, k, tm, tn));
  return hipSuccess;
}

hipError_t gemm_mxfp4(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                      const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                      hipStream_t s, bool panel_a, bool panel_b) {
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(tm * tn));
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  if (out_dtype == kOutF32)
    return launch<kOutF32>(grid, s, panel_a, panel_b, A, SA, B, SB, c, ldc, (int)M, (int)N, (int)K, tm, tn);
  return launch<kOutBF16>(grid, s, panel_a, panel_b, A, SA, B, SB, c, ldc, (int)M, (int)N, (int)K, tm, tn);
}

}  // namespace mx
