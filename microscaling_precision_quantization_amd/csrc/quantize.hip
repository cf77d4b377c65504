// Block quantization kernels for gfx950 (MXFP4, MXFP8 with E4M3 or E5M2
// elements, MXFP6 with E3M2 elements, NVFP4).
//
// Shared-exponent rule: FAQ of "Microscaling MXFP4/NVFP4 on Blackwell for
// reasoning LLMs" (E = ceil(log2(amax / max_elem)) + 127); element and scale
// formats from its section "Fundamentos matematicos do formato MXFP4 e E8M0";
// NVFP4 block size 16 from the zubnet.ai summary.
//
// Layout of the work: the input is treated as a flat array of 16-byte chunks
// (8 bf16). Blocks never straddle rows because cols is a multiple of the block,
// so codes and scales are flat too. MX: 4 consecutive lanes own one 32-block;
// NVFP4: 2 lanes own one 16-block. The block amax is an integer max of
// (bits & 0x7FFF) over the lanes' chunks, reduced with DPP quad permutes.
//
// Variants (MX formats): overflow-aware scaling for MXFP4 (gist.science
// summary of "Unveiling the Potential of Quantization with MXFP4", section
// 2.A: the scaled amax range (3, 6] becomes (3.5, 7], values in (6, 7]
// saturate), i.e. the rule with 7 in place of 6; and a 32-point
// Walsh-Hadamard rotation of every block before quantization
// (produtoramaxvision page, QuaRot / SpinQuant section), computed in fp32 by
// the radix-2 butterfly with spans 1, 2, 4 inside a lane and 8, 16 across the
// block's 4 lanes (DPP quad permutes), then scaled by fl32(1/sqrt(32)) and
// rounded to bf16 (v_cvt_pk_bf16_f32, nearest-even) before the usual steps.
//
// MXFP4 with static macro-block scaling (MBS; the same gist.science summary,
// section 2.B): a macro block of 128 elements (16 lanes, one DPP row) gets one
// factor f = 1 + m / 256 from its amax, and each base block inside (16
// elements as the summary prints, or 32, MXFP4's own) quantizes x / f by the
// MX rule with its own E8M0 scale (details at quant_mbs_kernel).
//
// Encoding uses gfx950's scaled converts. v_cvt_scalef32_pk_fp4_bf16 and
// v_cvt_scalef32_pk_fp8_bf16 return nearest-even of x / scale (saturating for
// FP4, -0 kept); with scale = 2^(E-127) that is exactly the MX element
// encoding (checked exhaustively over all bf16 inputs and all scales).
#include "mx_internal.h"

namespace mx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte chunks per thread

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_shr:n.
constexpr int kDppSwap1 = 0xB1;
constexpr int kDppSwap2 = 0x4E;
constexpr int dpp_row_shr(int n) { return 0x110 + n; }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Max of |x| over the 8 bf16 of a chunk, as the integer bits & 0x7FFF (a
// larger magnitude has larger bits; Inf is 0x7F80 and NaN is above it).
__device__ __forceinline__ uint32_t chunk_absmax(u32x4 v) {
  const uint32_t m = 0x7FFF7FFFu;
  u16x2 a = __builtin_bit_cast(u16x2, v.x & m);
  u16x2 b = __builtin_bit_cast(u16x2, v.y & m);
  u16x2 c = __builtin_bit_cast(u16x2, v.z & m);
  u16x2 d = __builtin_bit_cast(u16x2, v.w & m);
  u16x2 r = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return r.x > r.y ? r.x : r.y;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// 2^(E-127) as an fp32 bit pattern; E = 0 is the subnormal 2^-127.
__device__ __forceinline__ float e8m0_to_float(uint32_t E) {
  return __builtin_bit_cast(float, E == 0 ? 0x00400000u : E << 23);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// fl32(1/sqrt(32)).
constexpr float kInvSqrt32 = 0x1.6a09e6p-3f;

// The 32-point Walsh-Hadamard rotation of the block whose 8 elements
// 8 j .. 8 j + 7 this lane holds (j = lane % 4): y = bf16(fl32(H x) * c), the
// butterfly pairing (i, i + h) into (x_i + x_{i+h}, x_i - x_{i+h}) for
// h = 1, 2, 4 (inside the lane) and 8, 16 (lane j with j ^ 1, j ^ 2).
__device__ __forceinline__ u32x4 wht32_chunk(u32x4 v, int lane) {
  float f[8];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
  }
#pragma unroll
  for (int h = 1; h < 8; h *= 2)
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if (i & h) continue;
      const float a = f[i], d = f[i + h];
      f[i] = a + d;
      f[i + h] = a - d;
    }
  const bool up8 = (lane & 1) != 0, up16 = (lane & 2) != 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float p = __builtin_bit_cast(float, dpp<kDppSwap1>(__builtin_bit_cast(uint32_t, f[i])));
    f[i] = up8 ? p - f[i] : f[i] + p;
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float p = __builtin_bit_cast(float, dpp<kDppSwap2>(__builtin_bit_cast(uint32_t, f[i])));
    f[i] = up16 ? p - f[i] : f[i] + p;
  }
  u32x4 o;
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float lo = f[2 * i] * kInvSqrt32, hi = f[2 * i + 1] * kInvSqrt32;
    r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  }
  o.x = r[0]; o.y = r[1]; o.z = r[2]; o.w = r[3];
  return o;
}

// MXFP4 / MXFP8 (E4M3) / MXFP8 (E5M2); OAS: MXFP4's overflow-aware scale
// rule; ROT: rotate every block first.
// PANEL: codes and scales in the K-panel layout, panels of kPanel elements
// (MXFP4 256: [cols/256][rows][128] and [cols/256][rows][8]; MXFP8 64:
// [cols/64][rows][64] and [cols/64][rows][2]), i.e. kCpp 16-byte input
// chunks per row and panel. The grid is then 2-D: workgroup (x, y) takes
// rows kRpw x .. kRpw x + kRpw - 1 of panel y, consecutive lanes the chunks
// of a row, so loads, code stores and scale stores stay contiguous and no
// index needs a division by a runtime value. nchunks is then rows, cpr the
// chunks per row.
template <int FMT>
struct PanelGeo {
  static constexpr int kPanel = (FMT == kMXFP4) ? 256 : 64;
  static constexpr int kCpp = kPanel / 8;                    // chunks per row and panel
  static constexpr int kRpw = kThreads * kUnroll / kCpp;      // rows per workgroup
};

template <int FMT, bool OAS, bool ROT, bool PANEL = false>
__global__ __launch_bounds__(kThreads) void quant_mx_kernel(const u32x4* __restrict__ x,
                                                            void* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            int64_t nchunks, int64_t cpr = 0) {
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  // Source chunk, and (PANEL) destination dword of the codes, for item u.
  using PG = PanelGeo<FMT>;
  auto src_of = [&](int u) -> int64_t {
    if (!PANEL) return base + u * kThreads;
    const int t = u * kThreads + (int)threadIdx.x;
    const int64_t r = (int64_t)blockIdx.x * PG::kRpw + t / PG::kCpp;
    return r * cpr + (int64_t)blockIdx.y * PG::kCpp + t % PG::kCpp;
  };
  // Row of item u of this thread, or of the same item of lane t (PANEL).
  auto prow = [&](int u, int t) -> int64_t {
    return (int64_t)blockIdx.x * PG::kRpw + (u * kThreads + t) / PG::kCpp;
  };
  auto valid = [&](int u) -> bool {
    if (!PANEL) return base + u * kThreads < nchunks;
    return prow(u, (int)threadIdx.x) < nchunks;
  };
  auto dst_of = [&](int u) -> int64_t {
    if (!PANEL) return base + u * kThreads;
    const int t = u * kThreads + (int)threadIdx.x;
    return ((int64_t)blockIdx.y * nchunks + prow(u, (int)threadIdx.x)) * PG::kCpp + t % PG::kCpp;
  };
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; u++)
    v[u] = valid(u) ? __builtin_nontemporal_load(x + src_of(u)) : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < kUnroll; u++) {
    const int64_t c = dst_of(u);
    const bool ok = valid(u);
    if (ROT) v[u] = wht32_chunk(v[u], lane);
    uint32_t m = chunk_absmax(v[u]);
    m = umax(m, dpp<kDppSwap1>(m));
    m = umax(m, dpp<kDppSwap2>(m));
    // E = ceil(log2(amax / emax)) + 127 from the bf16 fields of amax:
    // emax = 6 = 1.5 * 2^2  -> E = ea - 2 + [mantissa > 0x40]
    // emax = 7 = 1.75 * 2^2 (OAS) -> E = ea - 2 + [mantissa > 0x60]
    // emax = 448 = 1.75 * 2^8 -> E = ea - 8 + [mantissa > 0x60]
    // emax = 57344 = 1.75 * 2^15 (E5M2) -> E = ea - 15 + [mantissa > 0x60]
    const int ea = (int)(m >> 7), ma = (int)(m & 0x7F);
    int e = (FMT == kMXFP4) ? ea - 2 + (ma > (OAS ? 0x60 : 0x40))
            : (FMT == kMXFP8) ? ea - 8 + (ma > 0x60)
                              : ea - 15 + (ma > 0x60);
    e = e < 0 ? 0 : e;
    const bool nonfinite = m >= 0x7F80u;
    const uint32_t E = nonfinite ? 255u : (uint32_t)e;
    const float scale = e8m0_to_float((uint32_t)e);
    if (FMT == kMXFP4) {
      uint32_t q = 0;
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, as_bf16x2(v[u].x), scale, 0);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, as_bf16x2(v[u].y), scale, 1);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, as_bf16x2(v[u].z), scale, 2);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, as_bf16x2(v[u].w), scale, 3);
      if (nonfinite) q = 0;
      // K-panel codes are activations that a GEMM reads next: plain stores
      // leave them in the caches (the MLP-down step 0.6-0.8 us faster).
      if (ok && PANEL) ((uint32_t*)codes)[c] = q;
      if (ok && !PANEL) __builtin_nontemporal_store(q, (uint32_t*)codes + c);
    } else {
      i16x2 lo = {0, 0}, hi = {0, 0};
      if (FMT == kMXFP8) {
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, as_bf16x2(v[u].x), scale, false);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, as_bf16x2(v[u].y), scale, true);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, as_bf16x2(v[u].z), scale, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, as_bf16x2(v[u].w), scale, true);
      } else {
        lo = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(lo, as_bf16x2(v[u].x), scale, false);
        lo = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(lo, as_bf16x2(v[u].y), scale, true);
        hi = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(hi, as_bf16x2(v[u].z), scale, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(hi, as_bf16x2(v[u].w), scale, true);
      }
      u32x2 q = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      if (nonfinite) q = u32x2{0, 0};
      if (ok && PANEL) ((u32x2*)codes)[c] = q;
      if (ok && !PANEL) __builtin_nontemporal_store(q, (u32x2*)codes + c);
    }
    // Scale bytes: lanes 3, 7, 11, 15 of each 16-lane DPP row hold 4
    // consecutive blocks; lane 15 assembles them into one dword store. (With
    // PANEL the byte index c / 4 is (panel * rows + row) * kPanel / 32 +
    // block, so a DPP row's 4 blocks are consecutive there too.)
    const uint32_t s4 = dpp<dpp_row_shr(4)>(E);
    const uint32_t s8 = dpp<dpp_row_shr(8)>(E);
    const uint32_t s12 = dpp<dpp_row_shr(12)>(E);
    const int64_t blk = c >> 2;
    if ((lane & 15) == 15 && ok) {
      *(uint32_t*)(scales + (blk - 3)) = s12 | (s8 << 8) | (s4 << 16) | (E << 24);
    }
    // Ragged end: the DPP row's lane 15 is past the end, store bytes instead.
    // Row layout: past the tensor's last chunk. PANEL: a row's chunks are all
    // in or all out, so this only happens where a DPP row spans two rows of
    // 8 chunks (64-element panels) and the second is past the last row.
    const bool last_out = PANEL ? prow(u, ((int)threadIdx.x & ~15) | 15) >= nchunks
                                : c - (lane & 15) + 15 >= nchunks;
    if ((lane & 3) == 0 && ok && last_out) scales[blk] = (uint8_t)E;
  }
}

// ---- MXFP4 with static macro-block scaling ----------------------------------

// DPP row_ror:n (rotate right by n lanes inside a row of 16).
constexpr int dpp_row_ror(int n) { return 0x120 + n; }

// Macro mantissa m from the macro amax (bf16 magnitude bits a): with S the
// 8-bit significand of a normalised to [128, 255] and n the smallest integer
// with amax <= 6 * 2^n, rho = amax / 2^n is S / 32 (S <= 192) or S / 64
// (S > 192); m is the smallest integer with 3 (1 + m / 256) >= rho, i.e.
// ceil((256 rho - 768) / 3), and 256 (rho within 2^-8 of 6) becomes 0. Zero
// and non-finite amax give 0.
__device__ __forceinline__ uint32_t mbs_mantissa(uint32_t a) {
  if (a == 0 || a >= 0x7F80u) return 0;
  const uint32_t S = (a >> 7) ? (0x80u | (a & 0x7Fu)) : (a << (__builtin_clz(a) - 24));
  const uint32_t num = (S <= 192 ? 8 * S : 4 * S) - 768;
  const uint32_t m = (num + 2) / 3;
  return m >= 256 ? 0 : m;
}

// x / (f 2^(E-127)) for the E2M1 decision: u = x 2^(127-E) is exact (or far
// below the smallest midpoint), then one Newton step on u * rcp(f). The
// residual u - q0 f is exact (fma), so q1 is the exact quotient when that is
// representable -- every tie lands on its midpoint -- and within a few ulps
// otherwise, while a non-tie quotient differs from every midpoint by more than
// 2^-13 relative (x has 8 significant bits, midpoint * f at most 12). The sign
// is copied so that -0 keeps its code.
__device__ __forceinline__ float mbs_quotient(float x, int sh, float f, float r) {
  const float u = __builtin_ldexpf(x, sh);
  const float q0 = u * r;
  const float e = __builtin_fmaf(-q0, f, u);
  const float q1 = __builtin_fmaf(e, r, q0);
  return __builtin_copysignf(q1, u);
}

// One lane per 16-byte chunk as in quant_mx_kernel; a DPP row of 16 lanes is
// one macro block. BASE = 32: 4 lanes per base block (MXFP4's own block);
// BASE = 16 (the summary's 1 x 16): 2 lanes per base block. Per base block,
// E is the smallest n with amax <= 6 f 2^n (+127, clamped at 0): the plain
// MX exponent e0 of amax or e0 - 1, since f is in [1, 2); the comparison with
// 6 f 2^(e0-128) is exact in fp32.
template <int BASE>
__global__ __launch_bounds__(kThreads) void quant_mbs_kernel(const u32x4* __restrict__ x,
                                                             uint32_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             uint8_t* __restrict__ macro,
                                                             int64_t nchunks) {
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; u++) {
    const int64_t c = base + u * kThreads;
    v[u] = (c < nchunks) ? __builtin_nontemporal_load(x + c) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < kUnroll; u++) {
    const int64_t c = base + u * kThreads;
    uint32_t mb = chunk_absmax(v[u]);
    mb = umax(mb, dpp<kDppSwap1>(mb));  // the base block's amax (BASE = 16)
    uint32_t mm = umax(mb, dpp<kDppSwap2>(mb));
    if (BASE == 32) mb = mm;
    mm = umax(mm, dpp<dpp_row_ror(4)>(mm));
    mm = umax(mm, dpp<dpp_row_ror(8)>(mm));
    const uint32_t mq = mbs_mantissa(mm);
    const float f = (float)(256u + mq) * 0x1p-8f;
    const float r = __builtin_amdgcn_rcpf(f);
    const int ea = (int)(mb >> 7), ma = (int)(mb & 0x7F);
    int e0 = ea - 2 + (ma > 0x40);
    e0 = e0 < 0 ? 0 : e0;
    const float bamax = __builtin_bit_cast(float, mb << 16);
    const int e = (e0 >= 1 && bamax <= __builtin_ldexpf(6.0f * f, e0 - 128)) ? e0 - 1 : e0;
    const bool nonfinite = mb >= 0x7F80u;
    const uint32_t E = nonfinite ? 255u : (uint32_t)e;
    const int sh = 127 - e;
    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    float o[8];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      o[2 * k] = mbs_quotient(__builtin_bit_cast(float, w[k] << 16), sh, f, r);
      o[2 * k + 1] = mbs_quotient(__builtin_bit_cast(float, w[k] & 0xFFFF0000u), sh, f, r);
    }
    uint32_t q = 0;
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, o[0], o[1], 1.0f, 0);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, o[2], o[3], 1.0f, 1);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, o[4], o[5], 1.0f, 2);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, o[6], o[7], 1.0f, 3);
    if (nonfinite) q = 0;
    // Plain stores: the GEMM that reads the activation codes next finds them
    // in the caches (MBS step ~2.5% faster; the quantize alone ~7% slower).
    if (c < nchunks) codes[c] = q;
    if (BASE == 32) {
      // Lanes 3, 7, 11, 15 of the row hold the macro block's 4 scales.
      const uint32_t s4 = dpp<dpp_row_shr(4)>(E);
      const uint32_t s8 = dpp<dpp_row_shr(8)>(E);
      const uint32_t s12 = dpp<dpp_row_shr(12)>(E);
      if ((lane & 15) == 15 && c < nchunks)
        *(uint32_t*)(scales + ((c >> 2) - 3)) = s12 | (s8 << 8) | (s4 << 16) | (E << 24);
    } else {
      // Lanes 1, 3, 5, 7 (and 9 .. 15) hold 4 consecutive scales each.
      const uint32_t s2 = dpp<dpp_row_shr(2)>(E);
      const uint32_t s4 = dpp<dpp_row_shr(4)>(E);
      const uint32_t s6 = dpp<dpp_row_shr(6)>(E);
      if ((lane & 7) == 7 && c < nchunks)
        *(uint32_t*)(scales + ((c >> 1) - 3)) = s6 | (s4 << 8) | (s2 << 16) | (E << 24);
    }
    if ((lane & 15) == 0 && c < nchunks) macro[c >> 4] = (uint8_t)mq;
  }
}

// ---- MXFP6 (E3M2) ---------------------------------------------------------

typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
typedef __bf16 bf16x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

// One lane per 32-block: 64 bytes of bf16 in, 24 bytes of 6-bit codes out
// (v_cvt_scalef32_pk32_bf6_bf16: nearest-even of x / scale, element i in bits
// 6i .. 6i+5), one scale byte. emax = 28 = 1.75 * 2^4 -> E = ea - 4 + [m > 0x60].
// MXFP6 (E3M2): one lane per 32-block, because the convert takes all 32
// elements of a block at once (v_cvt_scalef32_pk32_bf6_bf16: 32 bf16 -> 24
// bytes). A workgroup takes 256 consecutive blocks, and both its global
// traffic directions go through LDS so that every load and store instruction
// of a wave covers one contiguous range:
//  * load: 16-byte chunk c of the workgroup's range (lane-consecutive) goes
//    to LDS at 80 (c / 4) + 16 (c mod 4): blocks padded to 80 bytes, so the
//    16 lanes of a quarter-wave reading their own blocks' chunk j hit 16
//    distinct 16-byte bank groups (80 / 16 = 5 is odd);
//  * store: each lane writes its block's 24 code bytes to LDS at 24 t, and
//    the workgroup's 6 KB of codes leave as lane-consecutive 16-byte chunks.
// PANEL: the K-panel layout with 64-element panels ([cols/64][rows][48] and
// [cols/64][rows][2]). Workgroup (x, y) then takes the two blocks of rows
// 128 x .. 128 x + 127 in panel y: 8 chunks of 128 contiguous input bytes per
// row, and its output is again one contiguous range of codes and of scales.
// nblocks is then the row count and cpr the input chunks per row.
constexpr int kF6Pad = 80;                              // LDS bytes per staged block
constexpr int kF6Codes = kThreads * 24;                 // code bytes per workgroup

template <bool PANEL>
__global__ __launch_bounds__(kThreads) void quant_mxfp6_kernel(const u32x4* __restrict__ x,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               int64_t nblocks, int64_t cpr) {
  __shared__ __attribute__((aligned(16))) uint8_t lin[kThreads * kF6Pad];
  __shared__ __attribute__((aligned(16))) uint8_t lout[kF6Codes];
  const int tid = threadIdx.x;
  // b0: first output block of the workgroup (row layout: also its first
  // input block); nb: blocks in it.
  int64_t b0, nb, r0 = 0;
  if (PANEL) {
    r0 = (int64_t)blockIdx.x * (kThreads / 2);
    b0 = ((int64_t)blockIdx.y * nblocks + r0) * 2;
    nb = 2 * min((int64_t)(kThreads / 2), nblocks - r0);
  } else {
    b0 = (int64_t)blockIdx.x * kThreads;
    nb = min((int64_t)kThreads, nblocks - b0);
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int c = i * kThreads + tid;                              // chunk within the workgroup
    if (c < 4 * nb) {
      const int64_t src = PANEL ? (r0 + (c >> 3)) * cpr + (int64_t)blockIdx.y * 8 + (c & 7)
                                : 4 * b0 + c;
      const u32x4 v = __builtin_nontemporal_load(x + src);
      *(u32x4*)(lin + (c >> 2) * kF6Pad + (c & 3) * 16) = v;
    }
  }
  __syncthreads();
  if (tid < nb) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] = *(const u32x4*)(lin + tid * kF6Pad + j * 16);
    const uint32_t m = umax(umax(chunk_absmax(v[0]), chunk_absmax(v[1])),
                            umax(chunk_absmax(v[2]), chunk_absmax(v[3])));
    const int ea = (int)(m >> 7), ma = (int)(m & 0x7F);
    int e = ea - 4 + (ma > 0x60);
    e = e < 0 ? 0 : e;
    const bool nonfinite = m >= 0x7F80u;
    const u32x16 w = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w,
                      v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
    u32x6 q = __builtin_bit_cast(u32x6, __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(
                                            __builtin_bit_cast(bf16x32, w), e8m0_to_float((uint32_t)e)));
    if (nonfinite) q = u32x6{0, 0, 0, 0, 0, 0};
    *(u32x2*)(lout + tid * 24) = u32x2{q[0], q[1]};
    *(u32x2*)(lout + tid * 24 + 8) = u32x2{q[2], q[3]};
    *(u32x2*)(lout + tid * 24 + 16) = u32x2{q[4], q[5]};
    scales[b0 + tid] = nonfinite ? (uint8_t)255 : (uint8_t)e;
  }
  __syncthreads();
  // 24 nb bytes of codes: 16-byte chunks while whole, then 8-byte pieces
  // (24 nb is a multiple of 8).
  uint8_t* out = codes + 24 * b0;
  const int nbytes = (int)(24 * nb);
#pragma unroll
  for (int i = 0; i < (kF6Codes + 16 * kThreads - 1) / (16 * kThreads); i++) {
    const int o = 16 * (i * kThreads + tid);
    if (o + 16 <= nbytes)
      __builtin_nontemporal_store(*(const u32x4*)(lout + o), (u32x4*)(out + o));
    else if (o + 8 <= nbytes)
      __builtin_nontemporal_store(*(const u32x2*)(lout + o), (u32x2*)(out + o));
  }
}

// ---- NVFP4 ---------------------------------------------------------------

constexpr int kMaxPartials = 1024;
constexpr int kAmaxThreads = 1024;   // amax workgroups: 16 waves
constexpr int kAmaxPartials = 256;   // at most one amax workgroup per CU
constexpr int kAmaxLoads = 8;        // 16-byte loads in flight per thread

// Per-workgroup partial of max |x| (as bf16 magnitude bits). Few, large
// workgroups: the encode kernel reduces all partials in every workgroup, one
// load per thread when there are at most 256 of them.
__global__ __launch_bounds__(kAmaxThreads) void nvfp4_amax_partial(const u32x4* __restrict__ x,
                                                                   int64_t nchunks,
                                                                   uint32_t* __restrict__ partial) {
  // kAmaxLoads loads in flight per thread: chunks c + i G, G the grid's width.
  // Plain loads, so that the encode kernel finds x in the caches.
  uint32_t m = 0;
  const int64_t G = (int64_t)gridDim.x * kAmaxThreads;
  for (int64_t c = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x; c < nchunks; c += kAmaxLoads * G) {
    u32x4 v[kAmaxLoads];
#pragma unroll
    for (int i = 0; i < kAmaxLoads; i++)
      v[i] = (c + i * G < nchunks) ? x[c + i * G] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kAmaxLoads; i++) m = umax(m, chunk_absmax(v[i]));
  }
  for (int off = 32; off > 0; off >>= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[kAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kAmaxThreads / 64; w++) r = umax(r, wmax[w]);
    partial[blockIdx.x] = r;
  }
}

// The tensor scale from the amax partials, in every workgroup of the encode
// kernel (the maximum does not depend on the order): s_t = T / 2688
// (T = 0 -> 1, non-finite T -> NaN). Workgroup 0 writes it out.
// fdir (see nv_codes): 1 - 2^-19 where s_t > T / 2688, 1 + 2^-19 where
// s_t < T / 2688 (the sign of the exact fma s_t 2688 - T), both for a normal
// s_t; 1 for T = 0; 0 (the bracketing path) for s_t = T / 2688 exactly or a
// subnormal s_t.
__device__ __forceinline__ float nvfp4_tensor_scale(const uint32_t* __restrict__ partial,
                                                    int npartial, float* __restrict__ tensor_scale,
                                                    float& fdir) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npartial; i += kThreads) m = umax(m, partial[i]);
  for (int off = 32; off > 0; off >>= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = 0;
  for (int w = 0; w < kThreads / 64; w++) r = umax(r, wmax[w]);
  float st;
  fdir = 0.0f;
  if (r >= 0x7F80u) {
    st = __builtin_nanf("");
  } else {
    const float T = __builtin_bit_cast(float, r << 16);
    st = (T == 0.0f) ? 1.0f : T / 2688.0f;  // 2688 = 6 * 448
    const float e = __builtin_fmaf(st, 2688.0f, -T);
    if (T == 0.0f)
      fdir = 1.0f;
    else if (st >= 0x1p-126f && e != 0.0f)
      fdir = e > 0.0f ? 1.0f - 0x1p-19f : 1.0f + 0x1p-19f;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) tensor_scale[0] = st;
  return st;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// NVFP4 codes are the nearest-even E2M1 values of the exact quotient
// Q = x / (s_b s_t). x and s_t are both taken times xs = 2^64 when
// s_t < 2^-60 (exact), so that D = s_b s_t xs and R = rcp(fl(D)) (v_rcp_f32,
// within 1 ulp) are normal fp32 numbers; fl(x xs fl(R f)) is then within
// 5 2^-24 relative of Q f.
//
// Fast path (nv_codes), for a normal s_t = (T / 2688)(1 + eps) that is not
// exact: 2688 |x| and m s_b T (m an E2M1 midpoint) are integers below 2^13
// and 2^17 times powers of two, so Q0 = 2688 |x| / (s_b T) either equals m
// or lies 2^-17 or more (relative) away from it, and Q = Q0 / (1 + eps)
// with |eps| <= 2^-24. Where Q0 = m, Q falls below m exactly when eps > 0.
// So the code of fl(x xs fl(R f)) with f = 1 - 2^-19 (eps > 0) or 1 + 2^-19
// (eps < 0) is Q's: the 2^-19 pushes the quotients that sit on a midpoint in
// Q0 to the side eps puts them on, and moves no other across one.
//
// Bracketing path (nv_bracket + nv_resolve), for s_t exact or subnormal:
// x xs R (1 -+ 2^-18), each product rounded, lie on either side of Q.
// Rounding to E2M1 is monotone, so where the codes of the two agree that is
// Q's code; the lower one's magnitude is never above the upper one's.
__device__ __forceinline__ float nv_elem(const u32x4& v, int j) {
  const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
  return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}

template <int P, bool SCALED>
__device__ __forceinline__ uint32_t nv_pair(const u32x4& v, float rf, uint32_t c) {
  const float e0 = SCALED ? nv_elem(v, 2 * P) * 0x1p64f : nv_elem(v, 2 * P);
  const float e1 = SCALED ? nv_elem(v, 2 * P + 1) * 0x1p64f : nv_elem(v, 2 * P + 1);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, e0 * rf, e1 * rf, 1.0f, P);
}

template <bool SCALED>
__device__ __forceinline__ uint32_t nv_codes(const u32x4& v, float rf) {
  uint32_t c = 0;
  c = nv_pair<0, SCALED>(v, rf, c);
  c = nv_pair<1, SCALED>(v, rf, c);
  c = nv_pair<2, SCALED>(v, rf, c);
  return nv_pair<3, SCALED>(v, rf, c);
}

template <int P, bool SCALED>
__device__ __forceinline__ void nv_bracket_pair(const u32x4& v, float rlo, float rhi, uint32_t& cl,
                                                uint32_t& ch) {
  cl = nv_pair<P, SCALED>(v, rlo, cl);
  ch = nv_pair<P, SCALED>(v, rhi, ch);
}

template <bool SCALED>
__device__ __forceinline__ void nv_bracket(const u32x4& v, float rlo, float rhi, uint32_t& cl, uint32_t& ch) {
  cl = 0;
  ch = 0;
  nv_bracket_pair<0, SCALED>(v, rlo, rhi, cl, ch);
  nv_bracket_pair<1, SCALED>(v, rlo, rhi, cl, ch);
  nv_bracket_pair<2, SCALED>(v, rlo, rhi, cl, ch);
  nv_bracket_pair<3, SCALED>(v, rlo, rhi, cl, ch);
}

// Where the two codes differ, exactly one E2M1 midpoint m lies between them
// (the window is 2^-17 wide, midpoints are 29% or more apart): the one above
// the lower code's magnitude k. The sign of fma(m s_b, s_t xs, -|x xs|) then
// places the quotient below, above or on it (ties to the even code). m s_b is
// exact; the exact difference is 0 or a multiple of 2^-133 (2^-96 when
// scaled), so its sign survives the rounding. Branch-free over the 8 codes:
// where the two agree, either choice gives the same code. 4 m for k = 0..6 is
// 1, 3, 5, 7, 10, 14, 20.
__device__ __forceinline__ uint32_t nv_resolve(const u32x4& v, uint32_t cl, uint32_t ch, float xs,
                                               float sb, float stx) {
  constexpr uint64_t kMid4 = 0x00140E0A07050301ull;
  const float sbq = sb * 0.25f;
  uint32_t out = 0;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const uint32_t a = (cl >> (4 * j)) & 0xFu, b = (ch >> (4 * j)) & 0xFu;
    const uint32_t k = a & 7u;
    const float m4 = (float)(uint32_t)((kMid4 >> (8 * k)) & 0xFFu);
    const float d = __builtin_fmaf(m4 * sbq, stx, -__builtin_fabsf(nv_elem(v, j) * xs));
    const bool up = d < 0.0f || (d == 0.0f && (k & 1u));
    out |= (up ? b : a) << (4 * j);
  }
  return out;
}

// PANEL: codes and scales in the K-panel layout with 64-element panels
// ([cols/64][rows][32] and [cols/64][rows][4]). The grid is then 2-D:
// workgroup (x, y) takes rows 128 x .. 128 x + 127 of panel y, each group of
// 8 lanes the 8 chunks of one row; nchunks is then the row count and cpr the
// chunks per row.
template <bool PANEL>
__global__ __launch_bounds__(kThreads) void quant_nvfp4_kernel(const u32x4* __restrict__ x,
                                                               uint32_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               const uint32_t* __restrict__ partial,
                                                               int npartial,
                                                               float* __restrict__ tensor_scale,
                                                               int64_t nchunks, int64_t cpr) {
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  // Input chunk, output chunk and validity of item u.
  auto row_of = [&](int u) -> int64_t {
    return (int64_t)blockIdx.x * (kThreads * kUnroll / 8) + (u * kThreads + (int)threadIdx.x) / 8;
  };
  auto src_of = [&](int u) -> int64_t {
    if (!PANEL) return base + u * kThreads;
    return row_of(u) * cpr + (int64_t)blockIdx.y * 8 + (threadIdx.x & 7);
  };
  auto dst_of = [&](int u) -> int64_t {
    if (!PANEL) return base + u * kThreads;
    return ((int64_t)blockIdx.y * nchunks + row_of(u)) * 8 + (threadIdx.x & 7);
  };
  auto valid = [&](int u) -> bool {
    return PANEL ? row_of(u) < nchunks : base + u * kThreads < nchunks;
  };
  // The element loads go out first; the tensor scale is reduced meanwhile.
  // Plain loads here and in the amax pass (not non-temporal): the second
  // read of x then comes from the caches, 4% faster over both kernels.
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; u++)
    v[u] = valid(u) ? x[src_of(u)] : u32x4{0, 0, 0, 0};
  float fdir;
  const float st = nvfp4_tensor_scale(partial, npartial, tensor_scale, fdir);
  const bool bad = __builtin_isnan(st);
  const float d6 = 6.0f * st;
  const float xs = st < 0x1p-60f ? 0x1p64f : 1.0f;  // see nv_bracket
  const float stx = st * xs;
#pragma unroll
  for (int u = 0; u < kUnroll; u++) {
    const int64_t c = dst_of(u);
    const bool ok = valid(u);
    uint32_t m = chunk_absmax(v[u]);
    m = umax(m, dpp<kDppSwap1>(m));  // the partner lane holds the other half
    const float bamax = __builtin_bit_cast(float, m << 16);
    const float r = bamax / d6;
    // E4M3 nearest-even, saturating: clamp to 448 first (the convert itself
    // does not saturate above 448).
    const float rs = r < 448.0f ? r : 448.0f;
    uint32_t sbc = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(rs, rs, 0, false) & 0xFFu;
    const float sb = __builtin_amdgcn_cvt_f32_fp8((int)sbc, 0);
    // s_b = 0: sign-only zeros (x * 0). Otherwise D is normal (s_b >= 2^-9,
    // s_t xs >= 2^-85) and so is R.
    const float D = sb * stx;
    const float rz = (sb == 0.0f) ? 0.0f : __builtin_amdgcn_rcpf(D);
    uint32_t q;
    if (fdir != 0.0f) {
      const float rf = rz * fdir;
      if (xs == 1.0f)
        q = nv_codes<false>(v[u], rf);
      else
        q = nv_codes<true>(v[u], rf);
    } else {
      const float rlo = rz * (1.0f - 0x1p-18f), rhi = rz * (1.0f + 0x1p-18f);
      uint32_t qh;
      if (xs == 1.0f)
        nv_bracket<false>(v[u], rlo, rhi, q, qh);
      else
        nv_bracket<true>(v[u], rlo, rhi, q, qh);
      if (q != qh) q = nv_resolve(v[u], q, qh, xs, sb, stx);
    }
    if (bad) {
      q = 0;
      sbc = 0x7F;
    }
    if (ok) __builtin_nontemporal_store(q, codes + c);
    // Lanes 1, 3, 5, 7 of each group of 8 hold 4 consecutive block scales
    // (with PANEL, the 4 scales of one row's panel).
    const uint32_t s2 = dpp<dpp_row_shr(2)>(sbc);
    const uint32_t s4 = dpp<dpp_row_shr(4)>(sbc);
    const uint32_t s6 = dpp<dpp_row_shr(6)>(sbc);
    const int64_t blk = c >> 1;
    if ((lane & 7) == 7 && ok) {
      *(uint32_t*)(scales + (blk - 3)) = s6 | (s4 << 8) | (s2 << 16) | (sbc << 24);
    }
    // Ragged end of the row layout (with PANEL a row's 8 lanes are all in or out).
    if (!PANEL && (lane & 1) == 0 && ok && c - (lane & 7) + 7 >= nchunks) scales[blk] = (uint8_t)sbc;
  }
}

int64_t grid_for(int64_t nchunks) { return (nchunks + kThreads * kUnroll - 1) / (kThreads * kUnroll); }

}  // namespace

hipError_t quant_mx(int fmt, int64_t rows, int64_t cols, const void* x, void* codes, void* scales,
                    hipStream_t s, bool oas, bool rot, bool panel) {
  const int64_t nchunks = rows * cols / 8;
  const dim3 grid((unsigned)grid_for(nchunks));
  const u32x4* X = (const u32x4*)x;
  uint8_t* S = (uint8_t*)scales;
  if (panel && fmt != kMXFP4) {
    // MXFP8 / E5M2 in the K-panel layout: workgroups of 128 rows x one
    // 64-element panel (MXFP6 below).
    const int64_t cpr = cols / 8;
    if (fmt == kMXFP8) {
      const dim3 pgrid((unsigned)((rows + PanelGeo<kMXFP8>::kRpw - 1) / PanelGeo<kMXFP8>::kRpw), (unsigned)(cols / 64));
      if (rot)
        MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP8, false, true, true>, pgrid, kThreads, 0, s, X, codes, S, rows, cpr));
      else
        MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP8, false, false, true>, pgrid, kThreads, 0, s, X, codes, S, rows, cpr));
      return hipSuccess;
    }
    if (fmt == kMXFP8E5M2) {
      const dim3 pgrid((unsigned)((rows + PanelGeo<kMXFP8E5M2>::kRpw - 1) / PanelGeo<kMXFP8E5M2>::kRpw), (unsigned)(cols / 64));
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP8E5M2, false, false, true>, pgrid, kThreads, 0, s, X, codes, S, rows, cpr));
      return hipSuccess;
    }
  }
  if (panel && fmt == kMXFP4) {
    // MXFP4 in the K-panel layout: workgroups of 32 rows x one 256-element panel.
    const dim3 pgrid((unsigned)((rows + 31) / 32), (unsigned)(cols / 256));
    const int64_t cpr = cols / 8;
    if (oas && rot)
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP4, true, true, true>, pgrid, kThreads, 0, s, X, codes, S, rows, cpr));
    else if (oas)
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP4, true, false, true>, pgrid, kThreads, 0, s, X, codes, S, rows, cpr));
    else if (rot)
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP4, false, true, true>, pgrid, kThreads, 0, s, X, codes, S, rows, cpr));
    else
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP4, false, false, true>, pgrid, kThreads, 0, s, X, codes, S, rows, cpr));
    return hipSuccess;
  }
  if (fmt == kMXFP4) {
    if (oas && rot)
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP4, true, true>, grid, kThreads, 0, s, X, codes, S, nchunks, (int64_t)0));
    else if (oas)
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP4, true, false>, grid, kThreads, 0, s, X, codes, S, nchunks, (int64_t)0));
    else if (rot)
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP4, false, true>, grid, kThreads, 0, s, X, codes, S, nchunks, (int64_t)0));
    else
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP4, false, false>, grid, kThreads, 0, s, X, codes, S, nchunks, (int64_t)0));
  } else if (fmt == kMXFP8) {
    if (rot)
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP8, false, true>, grid, kThreads, 0, s, X, codes, S, nchunks, (int64_t)0));
    else
      MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP8, false, false>, grid, kThreads, 0, s, X, codes, S, nchunks, (int64_t)0));
  } else if (fmt == kMXFP8E5M2) {
    MX_TRY(launch_kernel(&quant_mx_kernel<kMXFP8E5M2, false, false>, grid, kThreads, 0, s, X, codes, S, nchunks, (int64_t)0));
  } else if (panel) {
    // MXFP6 in the K-panel layout: workgroups of 128 rows x one 64-element panel.
    const dim3 pgrid((unsigned)((rows + kThreads / 2 - 1) / (kThreads / 2)), (unsigned)(cols / 64));
    MX_TRY(launch_kernel(&quant_mxfp6_kernel<true>, pgrid, kThreads, 0, s, X, (uint8_t*)codes, S, rows,
                         cols / 8));
  } else {
    const int64_t nblocks = rows * cols / 32;
    MX_TRY(launch_kernel(&quant_mxfp6_kernel<false>, (unsigned)((nblocks + kThreads - 1) / kThreads), kThreads, 0, s,
                         X, (uint8_t*)codes, S, nblocks, (int64_t)0));
  }
  return hipSuccess;
}

// nchunks is a multiple of 16 (cols % 128 = 0), so every DPP row is either
// wholly inside the tensor or wholly past its end.
hipError_t quant_mbs(int64_t rows, int64_t cols, const void* x, void* codes, void* scales,
                     hipStream_t s, int base) {
  const int64_t nchunks = rows * cols / 8;
  uint8_t* S = (uint8_t*)scales;
  if (base == 16)
    MX_TRY(launch_kernel(&quant_mbs_kernel<16>, (unsigned)grid_for(nchunks), kThreads, 0, s,
                         (const u32x4*)x, (uint32_t*)codes, S, S + rows * (cols / 16), nchunks));
  else
    MX_TRY(launch_kernel(&quant_mbs_kernel<32>, (unsigned)grid_for(nchunks), kThreads, 0, s,
                         (const u32x4*)x, (uint32_t*)codes, S, S + rows * (cols / 32), nchunks));
  return hipSuccess;
}

size_t quant_nvfp4_workspace(int64_t, int64_t) { return kMaxPartials * sizeof(uint32_t); }

hipError_t quant_nvfp4(int64_t rows, int64_t cols, const void* x, void* codes, void* scales,
                       float* tensor_scale, void* workspace, hipStream_t s, bool panel) {
  const int64_t nchunks = rows * cols / 8;
  int64_t np = (nchunks + kAmaxThreads * kAmaxLoads - 1) / (kAmaxThreads * kAmaxLoads);
  if (np > kAmaxPartials) np = kAmaxPartials;
  if (np < 1) np = 1;
  uint32_t* partial = (uint32_t*)workspace;
  MX_TRY(launch_kernel(&nvfp4_amax_partial, (unsigned)np, kAmaxThreads, 0, s, (const u32x4*)x, nchunks, partial));
  if (panel) {
    // Workgroups of 128 rows x one 64-element panel.
    const dim3 pgrid((unsigned)((rows + 127) / 128), (unsigned)(cols / 64));
    MX_TRY(launch_kernel(&quant_nvfp4_kernel<true>, pgrid, kThreads, 0, s, (const u32x4*)x,
                         (uint32_t*)codes, (uint8_t*)scales, partial, (int)np, tensor_scale, rows, cols / 8));
  } else {
    MX_TRY(launch_kernel(&quant_nvfp4_kernel<false>, (unsigned)grid_for(nchunks), kThreads, 0, s,
                         (const u32x4*)x, (uint32_t*)codes, (uint8_t*)scales, partial, (int)np,
                         tensor_scale, nchunks, (int64_t)0));
  }
  return hipSuccess;
}

}  // namespace mx
