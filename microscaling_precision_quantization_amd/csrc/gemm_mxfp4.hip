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
//    the idle half of a 2 x 68 KB double buffer), LDS -> MFMA. The barrier
//    between super-steps waits for LDS work only, so global loads stay in
//    flight across it. Buffer range checking returns zeros for rows past M
//    or N.
//  * The barrier would leave the matrix core idle while a wave's first LDS
//    reads of the new super-step (its scales and first fragments) come back.
//    So the second half of each super-step's last sub-step (8 MFMAs, whose
//    fragments are already in registers) is issued after the barrier, beside
//    those reads. Each accumulator still sees its MFMAs in K order.
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
#include <type_traits>

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

// Buffer views of one super-step s. An operand in the K-panel layout
// (PANEL_A, PANEL_B) gets views spanning panel s: its codes start at byte
// s * rows * 128, its scales at s * rows * 8, and rows past M or N fall
// outside the view and load as zeros. They are made once per super-step, in
// 32-bit offsets (a whole operand stays below 2^31 bytes, gemm_mxfp4_fits). A
// row-layout operand keeps its whole-operand view, and the super-step's byte
// offsets within a row are kb (codes) and ks (scales).
struct Views {
  __amdgpu_buffer_rsrc_t a, b, sa, sb;
  uint32_t kb, ks;
};

template <bool PANEL_A, bool PANEL_B>
__device__ __forceinline__ Views views_of(int s, __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB,
                                          __amdgpu_buffer_rsrc_t rSA, __amdgpu_buffer_rsrc_t rSB,
                                          const uint8_t* A, const uint8_t* SA, int M,
                                          const uint8_t* B, const uint8_t* SB, int N) {
  const uint32_t us = (uint32_t)s;
  Views v;
  v.kb = us * kRowBytes;
  v.ks = us * (kSuperK / 32);
  v.a = PANEL_A ? __builtin_amdgcn_make_buffer_rsrc((void*)(A + us * (uint32_t)(M * kRowBytes)), 0,
                                                    M * kRowBytes, kRsrcFlags)
                : rA;
  v.b = PANEL_B ? __builtin_amdgcn_make_buffer_rsrc((void*)(B + us * (uint32_t)(N * kRowBytes)), 0,
                                                    N * kRowBytes, kRsrcFlags)
                : rB;
  v.sa = PANEL_A ? __builtin_amdgcn_make_buffer_rsrc((void*)(SA + us * (uint32_t)(M * (kSuperK / 32))),
                                                     0, M * (kSuperK / 32), kRsrcFlags)
                 : rSA;
  v.sb = PANEL_B ? __builtin_amdgcn_make_buffer_rsrc((void*)(SB + us * (uint32_t)(N * (kSuperK / 32))),
                                                     0, N * (kSuperK / 32), kRsrcFlags)
                 : rSB;
  return v;
}

// Part P (0..3) of the global loads of a super-step (its views v): code
// blocks 2P and 2P+1 of A and B, plus the A scales (P = 0) or the B scales
// (P = 1). Rows past M or N fall outside the buffer range and load as zeros.
template <int P, bool PANEL_A, bool PANEL_B>
__device__ __forceinline__ void load_part(Stage& st, const Views& v, int m0, int n0,
                                          uint32_t rowbytes, uint32_t scalebytes, int wave,
                                          int lane) {
#pragma unroll
  for (int i = 2 * P; i < 2 * P + 2; i++) {
    const int row = (wave * 8 + i) * 8 + (lane >> 3);
    const uint32_t cb = (uint32_t)((lane & 7) ^ swz(row)) * 16u;  // slot lane&7 of the LDS row holds this chunk
    st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(
        v.a, PANEL_A ? (uint32_t)(m0 + row) * (uint32_t)kRowBytes + cb
                     : (uint32_t)(m0 + row) * rowbytes + v.kb + cb, 0, 0);
    st.b[i] = __builtin_amdgcn_raw_buffer_load_b128(
        v.b, PANEL_B ? (uint32_t)(n0 + row) * (uint32_t)kRowBytes + cb
                     : (uint32_t)(n0 + row) * rowbytes + v.kb + cb, 0, 0);
  }
  const int srow = wave * 64 + lane;
  if (P == 0)
    st.sa = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
        v.sa, PANEL_A ? (uint32_t)(m0 + srow) * (uint32_t)(kSuperK / 32)
                      : (uint32_t)(m0 + srow) * scalebytes + v.ks, 0, 0));
  if (P == 1)
    st.sb = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
        v.sb, PANEL_B ? (uint32_t)(n0 + srow) * (uint32_t)(kSuperK / 32)
                      : (uint32_t)(n0 + srow) * scalebytes + v.ks, 0, 0));
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

// Rows I0 .. I1-1 of sub-step J's MFMAs: those A fragments against all four
// B fragments (a split sub-step).
template <int J, int I0, int I1>
__device__ __forceinline__ void mfma_rows(const Frags& f, const int (&sa)[4], const int (&sb)[4],
                                          f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = I0; i < I1; i++) {
    const i32x8 a = i32x8{f.a[i].x, f.a[i].y, f.a[i].z, f.a[i].w, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const i32x8 b = i32x8{f.b[j].x, f.b[j].y, f.b[j].z, f.b[j].w, 0, 0, 0, 0};
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
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int k = 0; k < 4; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
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

// Head of a super-step: the 8 MFMAs carried over from the previous one, with
// this super-step's 12 LDS reads (scales and sub-step 0's fragments) and the
// scalar work that makes its load views.
__device__ __forceinline__ void interleave_head() {
#pragma unroll
  for (int k = 0; k < 4; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x004, 3, 0);
  }
#pragma unroll
  for (int k = 0; k < 4; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x004, 3, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Sub-step 2: the last sub-step's 8 fragment reads, then the LDS writes of
// the staged super-step's last two parts (so they are complete well before
// the barrier) and the global loads of its third part.
__device__ __forceinline__ void interleave_third() {
#pragma unroll
  for (int k = 0; k < 4; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
#pragma unroll
  for (int k = 0; k < 4; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// First half of sub-step 3 (8 MFMAs) with the last part's global loads.
__device__ __forceinline__ void interleave_last() {
#pragma unroll
  for (int k = 0; k < 4; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  __builtin_amdgcn_sched_barrier(0);
}

template <int OUT, bool PANEL_A, bool PANEL_B>
__global__ __launch_bounds__(kThreads, 1) void gemm_mxfp4_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, void* __restrict__ C, int64_t ldc, int M, int N, int K,
    int tiles_m, int tiles_n, int s_begin, int s_end, int fold) {
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

  // Super-steps s_begin .. s_end-1 of K (all of K unless the fp32 output is
  // accumulated over several launches, see gemm_mxfp4 below).
  // Fragments of the odd sub-steps (f1) stay live from one super-step into
  // the next: the second half of sub-step 3 runs after the barrier.
  Frags f0, f1;
  // One super-step: MFMAs on LDS buffer s & 1 while the registers R (super-
  // step s + 1) go to LDS buffer (s + 1) & 1 and then receive super-step s + 2
  // from memory. Its scales go to (sa, sb); (pa, pb) hold the previous
  // super-step's, for the MFMAs carried over from it when `carry` is true.
  auto step = [&](auto carry, int s, Stage& R, int (&sa)[4], int (&sb)[4], const int (&pa)[4],
                  const int (&pb)[4]) __attribute__((always_inline)) {
    // Every wave's LDS writes of super-step s are done and every wave is done
    // reading super-step s-1, whose buffer receives super-step s+1 below. Only
    // LDS work is waited for: the global loads stay in flight.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    sched_fence();
    const uint8_t* cur = smem + (s & 1) * kStage;
    uint8_t* nxt = smem + ((s + 1) & 1) * kStage;
    // Branch-free body (a branch here lets the compiler sink the MFMAs): the
    // last iterations re-stage the final super-step into the idle buffer.
    const int s2 = min(s + 2, s_end - 1);
    const Views v = views_of<PANEL_A, PANEL_B>(s2, rA, rB, rSA, rSB, A, SA, M, B, SB, N);
    const uint8_t* As = cur;
    const uint8_t* Bs = cur + kTileBytes;
    const uint8_t* SAs = cur + 2 * kTileBytes;
    const uint8_t* SBs = SAs + kScaleBytes;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sb[i] = *(const int*)(SBs + (wn * 128 + i * 32 + r) * 8 + g * 4);
      sa[i] = *(const int*)(SAs + (wm * 128 + i * 32 + r) * 8 + g * 4);
    }
    load_frags<0>(As, Bs, wm, wn, r, g, f0);
    if constexpr (decltype(carry)::value) {
      mfma_rows<3, 2, 4>(f1, pa, pb, acc);
      interleave_head();
    } else {
      sched_fence();
    }
    // Each region below issues the MFMAs of one sub-step, the LDS reads of
    // the next sub-step's fragments, part of the staged super-step's LDS
    // writes and part of the next global loads, interleaved so that each
    // memory instruction issues in an MFMA's shadow.
    load_frags<1>(As, Bs, wm, wn, r, g, f1);
    store_part<0>(R, nxt, wave, lane);
    load_part<0, PANEL_A, PANEL_B>(R, v, m0, n0, rowbytes, scalebytes, wave, lane);
    mfma_substep<0>(f0, sa, sb, acc);
    interleave();
    load_frags<2>(As, Bs, wm, wn, r, g, f0);
    store_part<1>(R, nxt, wave, lane);
    load_part<1, PANEL_A, PANEL_B>(R, v, m0, n0, rowbytes, scalebytes, wave, lane);
    mfma_substep<1>(f1, sa, sb, acc);
    interleave();
    load_frags<3>(As, Bs, wm, wn, r, g, f1);
    store_part<2>(R, nxt, wave, lane);
    store_part<3>(R, nxt, wave, lane);
    load_part<2, PANEL_A, PANEL_B>(R, v, m0, n0, rowbytes, scalebytes, wave, lane);
    mfma_substep<2>(f0, sa, sb, acc);
    interleave_third();
    load_part<3, PANEL_A, PANEL_B>(R, v, m0, n0, rowbytes, scalebytes, wave, lane);
    mfma_rows<3, 0, 2>(f1, sa, sb, acc);
    interleave_last();
  };
  // Super-step s_begin goes to its LDS buffer through the registers first;
  // then the registers receive the next one, in the loop's order (the fences keep the
  // scheduler from reordering the parts), so that the in-order load counter
  // lets the loop's first LDS writes wait only for their own part.
  Stage R;
  const Views v0 = views_of<PANEL_A, PANEL_B>(s_begin, rA, rB, rSA, rSB, A, SA, M, B, SB, N);
  load_part<0, PANEL_A, PANEL_B>(R, v0, m0, n0, rowbytes, scalebytes, wave, lane);
  load_part<1, PANEL_A, PANEL_B>(R, v0, m0, n0, rowbytes, scalebytes, wave, lane);
  load_part<2, PANEL_A, PANEL_B>(R, v0, m0, n0, rowbytes, scalebytes, wave, lane);
  load_part<3, PANEL_A, PANEL_B>(R, v0, m0, n0, rowbytes, scalebytes, wave, lane);
  uint8_t* first_buf = smem + (s_begin & 1) * kStage;
  store_part<0>(R, first_buf, wave, lane);
  store_part<1>(R, first_buf, wave, lane);
  store_part<2>(R, first_buf, wave, lane);
  store_part<3>(R, first_buf, wave, lane);
  {
    const int s1 = min(s_begin + 1, s_end - 1);
    const Views v1 = views_of<PANEL_A, PANEL_B>(s1, rA, rB, rSA, rSB, A, SA, M, B, SB, N);
    sched_fence();
    load_part<0, PANEL_A, PANEL_B>(R, v1, m0, n0, rowbytes, scalebytes, wave, lane);
    sched_fence();
    load_part<1, PANEL_A, PANEL_B>(R, v1, m0, n0, rowbytes, scalebytes, wave, lane);
    sched_fence();
    load_part<2, PANEL_A, PANEL_B>(R, v1, m0, n0, rowbytes, scalebytes, wave, lane);
    sched_fence();
    load_part<3, PANEL_A, PANEL_B>(R, v1, m0, n0, rowbytes, scalebytes, wave, lane);
    sched_fence();
  }
  // Super-steps s0 .. s1-1 into the accumulators: the first carries nothing
  // over, each later one carries the previous one's last 8 MFMAs, and the
  // last one's are issued after the loop. The two scale sets alternate.
  int sa0[4], sb0[4], sa1[4], sb1[4];
  auto run = [&](int s0, int s1) __attribute__((always_inline)) {
    const std::false_type first;
    const std::true_type carry;
    step(first, s0, R, sa0, sb0, sa1, sb1);
    int s = s0 + 1;
    for (; s + 1 < s1; s += 2) {
      step(carry, s, R, sa1, sb1, sa0, sb0);
      step(carry, s + 1, R, sa0, sb0, sa1, sb1);
    }
    if (s < s1) {
      step(carry, s, R, sa1, sb1, sa0, sb0);
      mfma_rows<3, 2, 4>(f1, sa1, sb1, acc);
    } else {
      mfma_rows<3, 2, 4>(f1, sa0, sb0, acc);
    }
  };
  run(s_begin, s_end);

  if constexpr (OUT == kOutF32) {
    // One K segment of several (bit 0 of `fold`): add this segment's sums
    // into C (bit 1: the first segment stores them; bit 2: the last one).
    if (fold & 1) {
      tile256::fold_tile(acc, (float*)C, ldc, M, N, m0, n0, wave, lane, (fold & 2) != 0,
                         (fold & 4) != 0, 1.0f);
      return;
    }
  }
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
            int n, int k, int tm, int tn, int s0, int s1, int fold) {
  if (panel_a && panel_b)
    MX_TRY(launch_kernel(&gemm_mxfp4_kernel<OUT, true, true>, grid, kThreads, 0, s, A, SA, B, SB, c, ldc, m, n, k, tm, tn, s0, s1, fold));
  else if (panel_a)
    MX_TRY(launch_kernel(&gemm_mxfp4_kernel<OUT, true, false>, grid, kThreads, 0, s, A, SA, B, SB, c, ldc, m, n, k, tm, tn, s0, s1, fold));
  else if (panel_b)
    MX_TRY(launch_kernel(&gemm_mxfp4_kernel<OUT, false, true>, grid, kThreads, 0, s, A, SA, B, SB, c, ldc, m, n, k, tm, tn, s0, s1, fold));
  else
    MX_TRY(launch_kernel(&gemm_mxfp4_kernel<OUT, false, false>, grid, kThreads, 0, s, A, SA, B, SB, c, ldc, m, n, k, tm, tn, s0, s1, fold));
  return hipSuccess;
}

hipError_t gemm_mxfp4(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                      const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                      hipStream_t s, bool panel_a, bool panel_b) {
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(tm * tn));
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  const int nsteps = (int)(K / kSuperK);
  if (out_dtype == kOutF32) {
    // fp32 accumulation chains of at most 48 MFMAs (tile256::fold_tile): K in
    // segments of 12 super-steps, one launch each, every launch after the
    // first adding its sums into C (launches on one stream run in order).
    constexpr int kSeg = 12;
    if (nsteps <= kSeg)
      return launch<kOutF32>(grid, s, panel_a, panel_b, A, SA, B, SB, c, ldc, (int)M, (int)N, (int)K, tm, tn, 0, nsteps, 0);
    for (int s0 = 0; s0 < nsteps; s0 += kSeg) {
      const int s1 = s0 + kSeg < nsteps ? s0 + kSeg : nsteps;
      const int fold = 1 | (s0 == 0 ? 2 : 0) | (s1 == nsteps ? 4 : 0);
      MX_TRY(launch<kOutF32>(grid, s, panel_a, panel_b, A, SA, B, SB, c, ldc, (int)M, (int)N, (int)K, tm, tn, s0, s1, fold));
    }
    return hipSuccess;
  }
  return launch<kOutBF16>(grid, s, panel_a, panel_b, A, SA, B, SB, c, ldc, (int)M, (int)N, (int)K, tm, tn, 0, nsteps, 0);
}

}  // namespace mx
