// Large-tile GEMM for gfx950 on the 16-bit MFMAs for MXFP8 (E4M3 or E5M2
// elements), MXFP6 (E3M2) and NVFP4, each operand pair of one format, every
// operand expanded exactly to bf16 (MX formats) or fp16 (NVFP4) (why not the
// FP8/FP4 matrix paths is explained in gemm_bf16x.hip; E5M2 and E3M2 have 3
// significant bits, exact in bf16 like E4M3).
//
// Design for CDNA4:
//  * 256 x 256 output tile per workgroup of 8 waves, two per SIMD, each wave
//    128 x 64 (4 x 2 MFMAs of 32 x 32, 128 fp32 accumulators per lane): while
//    one wave of a SIMD expands codes on the vector ALU, the other's MFMAs
//    keep the matrix core busy (6% faster than 4 waves of 128 x 128 on NVFP4,
//    2% on MXFP8).
//  * Or 224 x 256 tiles, when the tile count then fills the device's CUs in
//    fewer rows of rounds (4608-row activations: 756 tiles in 3 rounds of 256
//    CUs instead of 648 tiles in 3, 1008 in 4 instead of 864 in 4). The
//    SIMD's second wave then covers 96 rows (3 x 2 MFMAs); A is still staged
//    as 256 rows, the last 32 outside its buffer view.
//  * K advances in stages of 64 elements. A stage moves through a four-deep
//    pipeline: global -> VGPRs (16-byte code chunks, range-checked buffer
//    loads issued three stages ahead into two alternating register stages),
//    VGPRs -> bf16 -> LDS (each code expanded once, one stage ahead, into the
//    idle half of a 2 x 64 KB double buffer), LDS -> MFMA. The barrier between stages waits for LDS work only, so the
//    global loads stay in flight across it.
//  * Expansion: MXFP8 to bf16 with v_cvt_scalef32_pk_bf16_fp8 (E4M3) or
//    _bf8 (E5M2), MXFP6 with v_cvt_scalef32_pk32_bf16_bf6, the E8M0 scale
//    passed as an fp32 power of two (the instructions read only the scale's
//    exponent; 255 makes every output NaN, as in the oracle). NVFP4 to fp16:
//    v_cvt_scalef32_pk_f16_fp4 at unit scale and one packed fp16 multiply by
//    the E4M3 block scale, exact because every E2M1 x E4M3 product has at
//    most 6 significant bits and lies in [2^-10, 2688]; the NVFP4 kernel then
//    runs on v_mfma_f32_32x32x16_f16.
//  * LDS rows hold 64 16-bit values (128 bytes, 8 chunks of 16); chunk k of row m
//    lives in slot k ^ ((m / 2) mod 8), conflict-free for the staging writes
//    and for the MFMA reads (16 rows at one chunk index per 16-lane group).
//  * MFMA sub-step s (K = 16) gives lane group g chunk 2 s + g of its row
//    (32 x 32 x 16 layout: lane r + 32 g supplies K elements
//    [8 g, 8 g + 8) of row r), the same permutation for A and B.
//  * Tile order and epilogue as in the MXFP4 kernel (tile256.h); the NVFP4
//    tensor scales multiply the fp32 result there.
#include <type_traits>

#include "mx_internal.h"
#include "tile256.h"

namespace mx {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
typedef __bf16 bf16x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;                     // 8 waves, two per SIMD
constexpr int kWavesN = 4;                        // waves along N (2 along M)
constexpr int BM = 256, BN = 256;
constexpr int BK = 64;                            // K elements per stage
constexpr int kRowBytes = BK * 2;                 // one LDS row: 64 bf16
constexpr int kTileBytes = BM * kRowBytes;        // 32 KB per operand
constexpr int kStage = 2 * kTileBytes;            // 64 KB
constexpr int kSmem = 147456;                     // 2 stages (128 KB) or the epilogue (144 KB)
constexpr uint32_t kRsrcFlags = 0x00020000u;      // raw buffer, gfx9 data format
constexpr uint32_t kOOB = 0x80000000u;            // an offset past every buffer's range

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Per-format staging geometry. A thread owns kChunks code chunks per operand
// per stage: MXFP8 chunk = 16 codes (4 per row, rows t/4 + 128u, two
// chunks), NVFP4 / MXFP6 chunk = 32 codes (2 per row, row t/2, one chunk).
template <int FMT>
struct Geo {
  static constexpr bool kByte = (FMT == kMXFP8 || FMT == kMXFP8E5M2);   // 8-bit codes
  static constexpr int kCodesPerChunk = kByte ? 16 : 32;
  static constexpr int kChunksPerRow = BK / kCodesPerChunk;      // 4 or 2
  static constexpr int kChunks = BM * kChunksPerRow / kThreads;  // per thread per operand: 2 or 1
  static constexpr int kRowStep = kThreads / kChunksPerRow;      // 128 or 256
  static constexpr int kBlock = (FMT == kNVFP4) ? 16 : 32;       // elements per scale
  static constexpr bool kFp16 = (FMT == kNVFP4);                  // fp16 operands
};

// Code bytes per row of K elements.
template <int FMT>
__host__ __device__ constexpr int64_t row_bytes(int64_t K) {
  return (FMT == kMXFP8 || FMT == kMXFP8E5M2) ? K : (FMT == kMXFP6) ? K * 3 / 4 : K / 2;
}

// One thread's share of a stage for both operands: codes and raw scale bits
// (MXFP8: the E8M0 byte of the chunk's block; NVFP4: the chunk's two E4M3
// bytes).
template <int FMT>
struct Stage {
  u32x4 qa[Geo<FMT>::kChunks], qb[Geo<FMT>::kChunks];
  u32x4 ta[Geo<FMT>::kChunks], tb[Geo<FMT>::kChunks];  // MXFP6: bytes 16 .. 23 of a chunk (.xy)
  uint32_t sa[Geo<FMT>::kChunks], sb[Geo<FMT>::kChunks];
};

// One operand's buffer views. Row layout: views based at the tile's first
// row, so that rows past M or N read as 0. K-panel layout (PANEL): views of
// the whole operand, the tile's first row at row0, and stage s's panel at
// byte s * pcodes (codes) and s * pscales (scales) -- the panel's size; the
// tile's rows past M or N then read other rows' codes, which only reach
// outputs that are never stored (row i of A feeds row i of C alone, row j of
// B column j), or zeros past the operand's end.
struct OpView {
  __amdgpu_buffer_rsrc_t codes, scales;
  int row0;
  uint32_t pcodes, pscales;
};

template <int FMT, bool PANEL>
__device__ __forceinline__ void load_op(u32x4 (&q)[Geo<FMT>::kChunks], u32x4 (&t)[Geo<FMT>::kChunks],
                                        uint32_t (&sc)[Geo<FMT>::kChunks], const OpView& v,
                                        uint32_t rowbytes, uint32_t scalebytes, int K, int s,
                                        int tid, int u) {
  using G = Geo<FMT>;
  const int row = tid / G::kChunksPerRow + G::kRowStep * u;
  const int c = tid % G::kChunksPerRow;
  uint32_t off, so, soff = 0, ssoff = 0;
  bool ok = true;
  if (PANEL) {
    // Panels of BK elements: row r's codes at r * row_bytes(BK), its scales at
    // r * BK / kBlock (whole panels only, so every chunk is in range).
    constexpr uint32_t kPw = (uint32_t)row_bytes<FMT>(BK), kPs = BK / G::kBlock;
    off = (uint32_t)(v.row0 + row) * kPw + (uint32_t)row_bytes<FMT>(c * G::kCodesPerChunk);
    so = (uint32_t)(v.row0 + row) * kPs + (uint32_t)(c * G::kCodesPerChunk / G::kBlock);
    soff = (uint32_t)s * v.pcodes;
    ssoff = (uint32_t)s * v.pscales;
  } else {
    const int k = s * BK + c * G::kCodesPerChunk;  // first element of the chunk
    ok = k < K;
    off = (uint32_t)row * rowbytes + (uint32_t)row_bytes<FMT>(k);
    so = (uint32_t)row * scalebytes + (uint32_t)(k / G::kBlock);
  }
  q[u] = __builtin_amdgcn_raw_buffer_load_b128(v.codes, ok ? off : kOOB, soff, 0);
  if (FMT == kMXFP6) {
    const u32x2 t2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(v.codes, ok ? off + 16 : kOOB, soff, 0));
    t[u] = u32x4{t2.x, t2.y, 0, 0};
  }
  if (FMT == kNVFP4)
    sc[u] = __builtin_amdgcn_raw_buffer_load_b16(v.scales, ok ? so : kOOB, ssoff, 0);
  else
    sc[u] = __builtin_amdgcn_raw_buffer_load_b8(v.scales, ok ? so : kOOB, ssoff, 0);
}

// The stage's staging work is split into 4 parts, one per MFMA sub-step: an
// item is one (operand, chunk u) pair, 2 kChunks items per stage, so a part
// holds 1 item (8-bit codes: chunk P % 2 of A for P < 2, of B otherwise) or
// none or one (4- and 6-bit codes: A in part 0, B in part 2).
template <int FMT, int P, bool PANEL>
__device__ __forceinline__ void load_part(Stage<FMT>& st, const OpView& va, const OpView& vb,
                                          uint32_t rowbytes, uint32_t scalebytes, int K, int s,
                                          int tid) {
  if (Geo<FMT>::kChunks == 2) {
    // Part P: operand P / 2, chunk P % 2.
    if (P < 2)
      load_op<FMT, PANEL>(st.qa, st.ta, st.sa, va, rowbytes, scalebytes, K, s, tid, P % 2);
    else
      load_op<FMT, PANEL>(st.qb, st.tb, st.sb, vb, rowbytes, scalebytes, K, s, tid, P % 2);
  } else {
    // One chunk per operand: A in part 0, B in part 2.
    if (P == 0) load_op<FMT, PANEL>(st.qa, st.ta, st.sa, va, rowbytes, scalebytes, K, s, tid, 0);
    if (P == 2) load_op<FMT, PANEL>(st.qb, st.tb, st.sb, vb, rowbytes, scalebytes, K, s, tid, 0);
  }
}

// Expands one chunk to bf16 and writes it to LDS row `row` of `tile`.
template <int FMT>
__device__ __forceinline__ void expand_chunk(const u32x4& q, const u32x4& qt, uint32_t sbits,
                                             uint8_t* tile, int row, int c) {
  uint8_t* base = tile + row * kRowBytes;
  const int sw = swz(row);
  if (FMT == kMXFP8 || FMT == kMXFP8E5M2) {
    // 16 codes -> LDS chunks 2c, 2c + 1.
    const float s = __builtin_bit_cast(float, sbits << 23);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if (FMT == kMXFP8) {
        o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], s, false));
        o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], s, true));
      } else {
        o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w[i], s, false));
        o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w[i], s, true));
      }
    }
    *(u32x4*)(base + (((2 * c) ^ sw) * 16)) = u32x4{o[0], o[1], o[2], o[3]};
    *(u32x4*)(base + (((2 * c + 1) ^ sw) * 16)) = u32x4{o[4], o[5], o[6], o[7]};
  } else if (FMT == kMXFP6) {
    // 32 codes (24 bytes) -> LDS chunks 4c .. 4c + 3.
    const float s = __builtin_bit_cast(float, sbits << 23);
    const u32x6 w = __builtin_shufflevector(q, qt, 0, 1, 2, 3, 4, 5);
    const u32x16 o = __builtin_bit_cast(u32x16, __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(w, s));
#pragma unroll
    for (int i = 0; i < 4; i++)
      *(u32x4*)(base + (((4 * c + i) ^ sw) * 16)) = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
  } else {
    // 32 codes (two 16-blocks) -> LDS chunks 4c .. 4c + 3, as fp16: every
    // e * s_b (E2M1 times E4M3: at most 6 significant bits, magnitude in
    // [2^-10, 2688]) is exact in fp16, so one packed fp16 multiply per pair
    // is exact; v_cvt_scalef32_pk_f16_fp4 at unit scale gives the codes.
    const f16x2 s0 = (f16x2)(_Float16)__builtin_amdgcn_cvt_f32_fp8((int)(sbits & 0xFFu), 0);
    const f16x2 s1 = (f16x2)(_Float16)__builtin_amdgcn_cvt_f32_fp8((int)(sbits >> 8), 0);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const f16x2 sc = (i < 2) ? s0 : s1;
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; p++) {
        f16x2 e;
        switch (p) {
          case 0: e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0); break;
          case 1: e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1); break;
          case 2: e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2); break;
          default: e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3); break;
        }
        o[p] = __builtin_bit_cast(uint32_t, e * sc);
      }
      *(u32x4*)(base + (((4 * c + i) ^ sw) * 16)) = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

// Part P of a staged stage's expansion (the items of load_part<P>).
template <int FMT, int P>
__device__ __forceinline__ void store_part(const Stage<FMT>& st, uint8_t* stage, int tid) {
  using G = Geo<FMT>;
  const int c = tid % G::kChunksPerRow;
  if (G::kChunks == 2) {
    const int u = P % 2;
    const int row = tid / G::kChunksPerRow + G::kRowStep * u;
    if (P < 2)
      expand_chunk<FMT>(st.qa[u], st.ta[u], st.sa[u], stage, row, c);
    else
      expand_chunk<FMT>(st.qb[u], st.tb[u], st.sb[u], stage + kTileBytes, row, c);
  } else {
    const int row = tid / G::kChunksPerRow;
    if (P == 0) expand_chunk<FMT>(st.qa[0], st.ta[0], st.sa[0], stage, row, c);
    if (P == 2) expand_chunk<FMT>(st.qb[0], st.tb[0], st.sb[0], stage + kTileBytes, row, c);
  }
}

template <int FMT, bool PANEL>
__device__ __forceinline__ void load_stage(Stage<FMT>& st, const OpView& va, const OpView& vb,
                                           uint32_t rowbytes, uint32_t scalebytes, int K, int s,
                                           int tid) {
  __builtin_amdgcn_sched_barrier(0);
  load_part<FMT, 0, PANEL>(st, va, vb, rowbytes, scalebytes, K, s, tid);
  __builtin_amdgcn_sched_barrier(0);
  load_part<FMT, 1, PANEL>(st, va, vb, rowbytes, scalebytes, K, s, tid);
  __builtin_amdgcn_sched_barrier(0);
  load_part<FMT, 2, PANEL>(st, va, vb, rowbytes, scalebytes, K, s, tid);
  __builtin_amdgcn_sched_barrier(0);
  load_part<FMT, 3, PANEL>(st, va, vb, rowbytes, scalebytes, K, s, tid);
  __builtin_amdgcn_sched_barrier(0);
}

// Fragments of sub-step S: NI A tiles and 2 B tiles of 32 rows, chunk 2S + g.
template <int S, int NI, typename V>
__device__ __forceinline__ void load_frags(const uint8_t* As, const uint8_t* Bs, int wm, int wn,
                                           int r, int g, V (&fa)[4], V (&fb)[2]) {
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int ra = wm * 128 + i * 32 + r;
    fa[i] = *(const V*)(As + ra * kRowBytes + (((2 * S + g) ^ swz(ra)) * 16));
  }
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int rb = wn * 64 + j * 32 + r;
    fb[j] = *(const V*)(Bs + rb * kRowBytes + (((2 * S + g) ^ swz(rb)) * 16));
  }
}

template <int NI>
__device__ __forceinline__ void mfma16(const bf16x8 (&fa)[4], const bf16x8 (&fb)[2], f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < NI; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
      // Operands swapped (B first): the result tile is C^T (see tile256.h).
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
}

template <int NI>
__device__ __forceinline__ void mfma16(const f16x8 (&fa)[4], const f16x8 (&fb)[2], f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < NI; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Issue order of one sub-step region (sched_group_barrier masks: 0x008 MFMA,
// 0x100 LDS read, 0x200 LDS write, 0x020 VMEM read, 0x002 VALU), closed by a
// fence: the next sub-step's 6 fragment reads go out within the first 3
// MFMAs, then the global loads, then the expansion and its LDS writes spread
// over the MFMAs that remain.
template <int FMT, bool WITH_READS>
__device__ __forceinline__ void region_order() {
  if (WITH_READS) {
#pragma unroll
    for (int k = 0; k < 3; k++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
  }
#pragma unroll
  for (int k = 0; k < 2; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
#pragma unroll
  for (int k = 0; k < 3; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, Geo<FMT>::kByte ? 4 : 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, Geo<FMT>::kByte ? 1 : 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// The K loop and epilogue of one tile, for a wave with NI row blocks of 32
// (4, or 3 for the second row of waves of a 224-row tile). Mlim is the first
// row past the tile's valid rows.
template <int FMT, int OUT, int NI, bool PANEL>
__device__ __forceinline__ void tile_body(uint8_t* smem, const OpView& va, const OpView& vb,
                                          uint32_t rowbytes, uint32_t scalebytes, int K, int tid,
                                          int lane, int wave, int wm, int wn, int r, int g,
                                          const float* __restrict__ TA, const float* __restrict__ TB,
                                          void* __restrict__ C, int64_t ldc, int Mlim, int N, int m0,
                                          int n0, int s_begin, int s_end, int fold) {
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  // Stages s_begin .. s_end-1 of K (all of K unless the fp32 output is
  // accumulated over several launches, see gemm_bf16x_large below).
  // Four-deep pipeline: LDS buffer s & 1 feeds the MFMAs while one of two
  // register stages (holding stage s + 1) is expanded into LDS buffer
  // (s + 1) & 1 and then receives stage s + 3 from memory; the other holds
  // s + 2. Every load has two stages to land.
  // Stage s uses LDS buffer `par` (its position in this launch's range, mod 2:
  // a constant in the unrolled loop, so the LDS addresses are too).
  auto step = [&](int s, int par, Stage<FMT>& Rx) {
    // Every thread's LDS writes of stage s are done and every wave is done
    // reading stage s-1, whose buffer receives stage s+1 below. Only LDS work
    // is waited for: the global loads stay in flight.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    fence();
    const uint8_t* cur = smem + par * kStage;
    uint8_t* nxt = smem + (par ^ 1) * kStage;
    // Branch-free body (a branch lets the compiler sink the MFMAs): the last
    // iterations re-stage the final stage into the idle buffer. The registers
    // Rx hold stage s + 1 and then receive stage s + 3.
    const int s2 = min(s + 3, s_end - 1);
    const uint8_t* As = cur;
    const uint8_t* Bs = cur + kTileBytes;
    // Operand elements: bf16 for the MX formats, fp16 for NVFP4.
    using V = typename std::conditional<Geo<FMT>::kFp16, f16x8, bf16x8>::type;
    V fa0[4], fb0[2], fa1[4], fb1[2];
    load_frags<0, NI>(As, Bs, wm, wn, r, g, fa0, fb0);
    fence();
    // Sub-step 0: next fragments, expansion of chunk 0 of stage s+1, loads of
    // chunk 0 of stage s+3, MFMAs. Likewise for the other sub-steps.
    load_frags<1, NI>(As, Bs, wm, wn, r, g, fa1, fb1);
    store_part<FMT, 0>(Rx, nxt, tid);
    load_part<FMT, 0, PANEL>(Rx, va, vb, rowbytes, scalebytes, K, s2, tid);
    mfma16<NI>(fa0, fb0, acc);
    region_order<FMT, true>();
    load_frags<2, NI>(As, Bs, wm, wn, r, g, fa0, fb0);
    store_part<FMT, 1>(Rx, nxt, tid);
    load_part<FMT, 1, PANEL>(Rx, va, vb, rowbytes, scalebytes, K, s2, tid);
    mfma16<NI>(fa1, fb1, acc);
    region_order<FMT, true>();
    load_frags<3, NI>(As, Bs, wm, wn, r, g, fa1, fb1);
    store_part<FMT, 2>(Rx, nxt, tid);
    load_part<FMT, 2, PANEL>(Rx, va, vb, rowbytes, scalebytes, K, s2, tid);
    mfma16<NI>(fa0, fb0, acc);
    region_order<FMT, true>();
    store_part<FMT, 3>(Rx, nxt, tid);
    load_part<FMT, 3, PANEL>(Rx, va, vb, rowbytes, scalebytes, K, s2, tid);
    mfma16<NI>(fa1, fb1, acc);
    region_order<FMT, false>();
  };
  // Prologue: the first stage to LDS buffer 0, the next two in registers
  // (issued in the loop's order so that the in-order load counter lets the
  // loop's first expansions wait only for their own part).
  Stage<FMT> R[2];
  load_stage<FMT, PANEL>(R[0], va, vb, rowbytes, scalebytes, K, s_begin, tid);
  store_part<FMT, 0>(R[0], smem, tid);
  store_part<FMT, 1>(R[0], smem, tid);
  store_part<FMT, 2>(R[0], smem, tid);
  store_part<FMT, 3>(R[0], smem, tid);
  load_stage<FMT, PANEL>(R[0], va, vb, rowbytes, scalebytes, K, min(s_begin + 1, s_end - 1), tid);
  load_stage<FMT, PANEL>(R[1], va, vb, rowbytes, scalebytes, K, min(s_begin + 2, s_end - 1), tid);
  const float ts = (FMT == kNVFP4) ? TA[0] * TB[0] : 1.0f;
  int s = s_begin;
  for (; s + 1 < s_end; s += 2) {
    step(s, 0, R[0]);
    step(s + 1, 1, R[1]);
  }
  if (s < s_end) step(s, 0, R[0]);
  if constexpr (OUT == kOutF32) {
    // One K segment of several (bit 0 of `fold`): add this segment's sums
    // into C (bit 1: the first segment stores them; bit 2: the last one,
    // which also applies the NVFP4 tensor scales).
    if (fold & 1) {
      tile256::fold_tile<2, kWavesN>(acc, (float*)C, ldc, Mlim, N, m0, n0, wave, lane,
                                     (fold & 2) != 0, (fold & 4) != 0, ts);
      return;
    }
  }
  __syncthreads();
  tile256::store_tile<OUT, 2, kWavesN>(acc, smem, ts, C, ldc, Mlim, N, m0, n0, wave, lane);
}

template <int FMT, int OUT, int BMT, bool PANEL>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16x_large_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const float* __restrict__ TA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB, const float* __restrict__ TB,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_n, int s_begin,
    int s_end, int fold) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int r = lane & 31, g = lane >> 5;
  int tm, tn;
  if (!tile256::tile_of_padded(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn)) return;
  const int m0 = tm * BMT, n0 = tn * BN;

  const uint32_t rowbytes = (uint32_t)row_bytes<FMT>(K);
  const uint32_t scalebytes = (uint32_t)(K / Geo<FMT>::kBlock);
  const int mrows = min(BMT, M - m0), nrows = min(BN, N - n0);
  OpView va, vb;
  if (PANEL) {
    va = {__builtin_amdgcn_make_buffer_rsrc((void*)A, 0, (int)(M * rowbytes), kRsrcFlags),
          __builtin_amdgcn_make_buffer_rsrc((void*)SA, 0, (int)(M * scalebytes), kRsrcFlags), m0,
          (uint32_t)M * (uint32_t)row_bytes<FMT>(BK), (uint32_t)M * (uint32_t)(BK / Geo<FMT>::kBlock)};
    vb = {__builtin_amdgcn_make_buffer_rsrc((void*)B, 0, (int)(N * rowbytes), kRsrcFlags),
          __builtin_amdgcn_make_buffer_rsrc((void*)SB, 0, (int)(N * scalebytes), kRsrcFlags), n0,
          (uint32_t)N * (uint32_t)row_bytes<FMT>(BK), (uint32_t)N * (uint32_t)(BK / Geo<FMT>::kBlock)};
  } else {
    // Views based at the tile's first rows: rows past M or N read as 0.
    va = {__builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)m0 * rowbytes), 0, (int)(mrows * rowbytes), kRsrcFlags),
          __builtin_amdgcn_make_buffer_rsrc((void*)(SA + (int64_t)m0 * scalebytes), 0, (int)(mrows * scalebytes), kRsrcFlags),
          0, 0u, 0u};
    vb = {__builtin_amdgcn_make_buffer_rsrc((void*)(B + (int64_t)n0 * rowbytes), 0, (int)(nrows * rowbytes), kRsrcFlags),
          __builtin_amdgcn_make_buffer_rsrc((void*)(SB + (int64_t)n0 * scalebytes), 0, (int)(nrows * scalebytes), kRsrcFlags),
          0, 0u, 0u};
  }

  // A 224-row tile: the first row of waves holds 128 rows (4 blocks), the
  // second 96 (3 blocks); the staged rows 224 .. 255 lie outside A's view and
  // are never read.
  const int Mlim = m0 + mrows;
  if (BMT == 256 || wm == 0)
    tile_body<FMT, OUT, 4, PANEL>(smem, va, vb, rowbytes, scalebytes, K, tid, lane, wave, wm, wn, r, g, TA, TB, C, ldc, Mlim, N, m0, n0, s_begin, s_end, fold);
  else
    tile_body<FMT, OUT, 3, PANEL>(smem, va, vb, rowbytes, scalebytes, K, tid, lane, wave, wm, wn, r, g, TA, TB, C, ldc, Mlim, N, m0, n0, s_begin, s_end, fold);
}

template <int FMT, int BMT, bool PANEL>
hipError_t launch(hipStream_t s, int tm, int tn, const uint8_t* A, const uint8_t* SA, const float* TA,
            const uint8_t* B, const uint8_t* SB, const float* TB, int out_dtype, void* c,
            int64_t ldc, int M, int N, int K) {
  // The grid is padded to whole groups of 8 workgroups (one per XCD); the
  // padding workgroups return at once (tile256::tile_of_padded).
  const dim3 grid((unsigned)((tm * tn + 7) / 8 * 8));
  const int nsteps = (K + BK - 1) / BK;
  if (out_dtype == kOutF32) {
    // fp32 accumulation chains of at most 48 MFMAs (tile256::fold_tile): K in
    // segments of 12 stages, one launch each, every launch after the first
    // adding its sums into C (launches on one stream run in order).
    constexpr int kSeg = 12;
    if (nsteps <= kSeg) {
      MX_TRY(launch_kernel(&gemm_bf16x_large_kernel<FMT, kOutF32, BMT, PANEL>, grid, kThreads, 0, s, A, SA, TA, B, SB, TB, c, ldc, M, N, K, tm, tn, 0, nsteps, 0));
      return hipSuccess;
    }
    for (int s0 = 0; s0 < nsteps; s0 += kSeg) {
      const int s1 = s0 + kSeg < nsteps ? s0 + kSeg : nsteps;
      const int fold = 1 | (s0 == 0 ? 2 : 0) | (s1 == nsteps ? 4 : 0);
      MX_TRY(launch_kernel(&gemm_bf16x_large_kernel<FMT, kOutF32, BMT, PANEL>, grid, kThreads, 0, s, A, SA, TA, B, SB, TB, c, ldc, M, N, K, tm, tn, s0, s1, fold));
    }
    return hipSuccess;
  }
  MX_TRY(launch_kernel(&gemm_bf16x_large_kernel<FMT, kOutBF16, BMT, PANEL>, grid, kThreads, 0, s, A, SA, TA, B, SB, TB, c, ldc, M, N, K, tm, tn, 0, nsteps, 0));
  return hipSuccess;
}

template <int FMT>
hipError_t launch_rows(bool rows224, bool panel, hipStream_t s, int64_t M, int tn, const uint8_t* A,
                       const uint8_t* SA, const float* TA, const uint8_t* B, const uint8_t* SB,
                       const float* TB, int out_dtype, void* c, int64_t ldc, int N, int K) {
  const int tm224 = (int)((M + 223) / 224), tm256 = (int)((M + 255) / 256);
  if (panel) {
    if (rows224)
      return launch<FMT, 224, true>(s, tm224, tn, A, SA, TA, B, SB, TB, out_dtype, c, ldc, (int)M, N, K);
    return launch<FMT, 256, true>(s, tm256, tn, A, SA, TA, B, SB, TB, out_dtype, c, ldc, (int)M, N, K);
  }
  if (rows224)
    return launch<FMT, 224, false>(s, tm224, tn, A, SA, TA, B, SB, TB, out_dtype, c, ldc, (int)M, N, K);
  return launch<FMT, 256, false>(s, tm256, tn, A, SA, TA, B, SB, TB, out_dtype, c, ldc, (int)M, N, K);
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

// 32-bit buffer offsets cover the tile's rows (codes and scales).
bool gemm_bf16x_large_fits(int fmt, int64_t M, int64_t N, int64_t K) {
  const int64_t rowbytes = (fmt == kMXFP8 || fmt == kMXFP8E5M2) ? K : (fmt == kMXFP6) ? K * 3 / 4 : K / 2;
  const int64_t lim = (int64_t)1 << 31;
  return (int64_t)BM * rowbytes < lim && (M + N) > 0;
}

hipError_t gemm_bf16x_large(int fmt, int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                            const float* ta, const void* b, const void* sb, const float* tb,
                            int out_dtype, void* c, int64_t ldc, hipStream_t s, bool panel) {
  const int tn = (int)((N + BN - 1) / BN);
  // Tile height: every tile of a round of the device's CUs takes about as
  // long as its rows, so 224-row tiles pay when they need fewer rows of
  // rounds, rounds x tile rows, than 256-row tiles (4608 rows by 36 or 48
  // tile columns: 3 rounds of 224 against 3 of 256, 4 of 224 against 4 of 256).
  const int64_t cus = device_cus();
  const int64_t r256 = ((M + 255) / 256 * tn + cus - 1) / cus;
  const int64_t r224 = ((M + 223) / 224 * tn + cus - 1) / cus;
  const bool rows224 = r224 * 224 < r256 * 256;
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  if (fmt == kMXFP8)
    return launch_rows<kMXFP8>(rows224, panel, s, M, tn, A, SA, ta, B, SB, tb, out_dtype, c, ldc, (int)N, (int)K);
  if (fmt == kMXFP8E5M2)
    return launch_rows<kMXFP8E5M2>(rows224, panel, s, M, tn, A, SA, ta, B, SB, tb, out_dtype, c, ldc, (int)N, (int)K);
  if (fmt == kMXFP6)
    return launch_rows<kMXFP6>(rows224, panel, s, M, tn, A, SA, ta, B, SB, tb, out_dtype, c, ldc, (int)N, (int)K);
  return launch_rows<kNVFP4>(rows224, panel, s, M, tn, A, SA, ta, B, SB, tb, out_dtype, c, ldc, (int)N, (int)K);
}

}  // namespace mx
