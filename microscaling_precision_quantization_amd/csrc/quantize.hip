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
// factor f = 1 + m / 256 from its amax, and each 32-block inside quantizes
// x / f by the MX rule (details at quant_mbs_kernel).
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
// PANEL (MXFP4): codes and scales in the K-panel layout ([cols/256][rows][128]
// and [cols/256][rows][8]). The grid is then 2-D: workgroup (x, y) takes
// rows 32 x .. 32 x + 31 of panel y, lanes 32 r' + j of a wave the 32 chunks
// j of a row, so loads, code stores and scale stores stay contiguous and no
// index needs a division. nchunks is then rows, cpr the chunks per row.
template <int FMT, bool OAS, bool ROT, bool PANEL = false>
__global__ __launch_bounds__(kThreads) void quant_mx_kernel(const u32x4* __restrict__ x,
                                                            void* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            int64_t nchunks, int64_t cpr = 0) {
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  // Source chunk, and (PANEL) destination dword of the codes, for item u.
  auto src_of = [&](int u) -> int64_t {
    if (!PANEL) return base + u * kThreads;
    const int t = u * kThreads + (int)threadIdx.x;
    const int64_t r = (int64_t)blockIdx.x * 32 + (t >> 5);
    return r * cpr + (int64_t)blockIdx.y * 32 + (t & 31);
  };
  auto valid = [&](int u) -> bool {
    if (!PANEL) return base + u * kThreads < nchunks;
    return (int64_t)blockIdx.x * 32 + ((u * kThreads + (int)threadIdx.x) >> 5) < nchunks;
  };
  auto dst_of = [&](int u) -> int64_t {
    if (!PANEL) return base + u * kThreads;
    const int t = u * kThreads + (int)threadIdx.x;
    const int64_t r = (int64_t)blockIdx.x * 32 + (t >> 5);
    return ((int64_t)blockIdx.y * nchunks + r) * 32 + (t & 31);
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
      if (ok) __builtin_nontemporal_store(q, (uint32_t*)codes + c);
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
      if (ok) __builtin_nontemporal_store(q, (u32x2*)codes + c);
    }
    // Scale bytes: lanes 3, 7, 11, 15 of each 16-lane DPP row hold 4
    // consecutive blocks; lane 15 assembles them into one dword store. (With
    // PANEL the dword index c / 4 is (panel * rows + row) * 8 + block.)
    const uint32_t s4 = dpp<dpp_row_shr(4)>(E);
    const uint32_t s8 = dpp<dpp_row_shr(8)>(E);
    const uint32_t s12 = dpp<dpp_row_shr(12)>(E);
    const int64_t blk = c >> 2;
    if ((lane & 15) == 15 && ok) {
      *(uint32_t*)(scales + (blk - 3)) = s12 | (s8 << 8) | (s4 << 16) | (E << 24);
    }
    // Ragged end: the row's lane 15 is past the end, store bytes instead
    // (never with PANEL: a row's 32 chunks are all in or all out).
    if (!PANEL && (lane & 3) == 0 && ok && c - (lane & 15) + 15 >= nchunks) scales[blk] = (uint8_t)E;
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
// one macro block. Per 32-block, E is the smallest n with amax <= 6 f 2^n
// (+127, clamped at 0): the plain MX exponent e0 of amax or e0 - 1, since
// f is in [1, 2); the comparison with 6 f 2^(e0-128) is exact in fp32.
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
    mb = umax(mb, dpp<kDppSwap1>(mb));
    mb = umax(mb, dpp<kDppSwap2>(mb));
    uint32_t mm = umax(mb, dpp<dpp_row_ror(4)>(mb));
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
    if (c < nchunks) __builtin_nontemporal_store(q, codes + c);
    const uint32_t s4 = dpp<dpp_row_shr(4)>(E);
    const uint32_t s8 = dpp<dpp_row_shr(8)>(E);
    const uint32_t s12 = dpp<dpp_row_shr(12)>(E);
    if ((lane & 15) == 15 && c < nchunks)
      *(uint32_t*)(scales + ((c >> 2) - 3)) = s12 | (s8 << 8) | (s4 << 16) | (E << 24);
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
__global__ __launch_bounds__(kThreads) void quant_mxfp6_kernel(const u32x4* __restrict__ x,
                                                               u32x2* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nblocks) return;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; i++) v[i] = __builtin_nontemporal_load(x + 4 * b + i);
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
  __builtin_nontemporal_store(u32x2{q[0], q[1]}, codes + 3 * b);
  __builtin_nontemporal_store(u32x2{q[2], q[3]}, codes + 3 * b + 1);
  __builtin_nontemporal_store(u32x2{q[4], q[5]}, codes + 3 * b + 2);
  scales[b] = nonfinite ? (uint8_t)255 : (uint8_t)e;
}

// ---- NVFP4 ---------------------------------------------------------------

constexpr int kMaxPartials = 1024;

// Per-workgroup partial of max |x| (as bf16 magnitude bits).
__global__ __launch_bounds__(kThreads) void nvfp4_amax_partial(const u32x4* __restrict__ x,
                                                               int64_t nchunks,
                                                               uint32_t* __restrict__ partial) {
  // Four loads in flight per thread: chunks c + i G, G the grid's width.
  uint32_t m = 0;
  const int64_t G = (int64_t)gridDim.x * kThreads;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < nchunks; c += 4 * G) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
      v[i] = (c + i * G < nchunks) ? __builtin_nontemporal_load(x + c + i * G) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; i++) m = umax(m, chunk_absmax(v[i]));
  }
  for (int off = 32; off > 0; off >>= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kThreads / 64; w++) r = umax(r, wmax[w]);
    partial[blockIdx.x] = r;
  }
}

// The tensor scale from the amax partials, in every workgroup of the encode
// kernel (the maximum does not depend on the order): s_t = T / 2688
// (T = 0 -> 1, non-finite T -> NaN). Workgroup 0 writes it out.
__device__ __forceinline__ float nvfp4_tensor_scale(const uint32_t* __restrict__ partial,
                                                    int npartial, float* __restrict__ tensor_scale) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npartial; i += kThreads) m = umax(m, partial[i]);
  for (int off = 32; off > 0; off >>= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = 0;
  for (int w = 0; w < kThreads / 64; w++) r = umax(r, wmax[w]);
  float st;
  if (r >= 0x7F80u) {
    st = __builtin_nanf("");
  } else {
    const float T = __builtin_bit_cast(float, r << 16);
    st = (T == 0.0f) ? 1.0f : T / 2688.0f;  // 2688 = 6 * 448
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) tensor_scale[0] = st;
  return st;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// x * (1/D), with x = +-0 kept as is (no 0 * Inf) and D = 0 giving +-0.
__device__ __forceinline__ float nv_scaled(float xv, float rz) { return xv == 0.0f ? xv : xv * rz; }

__global__ __launch_bounds__(kThreads) void quant_nvfp4_kernel(const u32x4* __restrict__ x,
                                                               uint32_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               const uint32_t* __restrict__ partial,
                                                               int npartial,
                                                               float* __restrict__ tensor_scale,
                                                               int64_t nchunks) {
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  // The element loads go out first; the tensor scale is reduced meanwhile.
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; u++) {
    const int64_t c = base + u * kThreads;
    v[u] = (c < nchunks) ? __builtin_nontemporal_load(x + c) : u32x4{0, 0, 0, 0};
  }
  const float st = nvfp4_tensor_scale(partial, npartial, tensor_scale);
  const bool bad = __builtin_isnan(st);
  const float d6 = 6.0f * st;
#pragma unroll
  for (int u = 0; u < kUnroll; u++) {
    const int64_t c = base + u * kThreads;
    uint32_t m = chunk_absmax(v[u]);
    m = umax(m, dpp<kDppSwap1>(m));  // the partner lane holds the other half
    const float bamax = __builtin_bit_cast(float, m << 16);
    const float r = bamax / d6;
    // E4M3 nearest-even, saturating: clamp to 448 first (the convert itself
    // does not saturate above 448).
    const float rs = r < 448.0f ? r : 448.0f;
    uint32_t sbc = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(rs, rs, 0, false) & 0xFFu;
    const float sb = __builtin_amdgcn_cvt_f32_fp8((int)sbc, 0);
    const float D = sb * st;
    const float R = 1.0f / D;
    const float rz = (D == 0.0f) ? 0.0f : R;
    uint32_t q = 0;
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, nv_scaled(bf16_lo(v[u].x), rz), nv_scaled(bf16_hi(v[u].x), rz), 1.0f, 0);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, nv_scaled(bf16_lo(v[u].y), rz), nv_scaled(bf16_hi(v[u].y), rz), 1.0f, 1);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, nv_scaled(bf16_lo(v[u].z), rz), nv_scaled(bf16_hi(v[u].z), rz), 1.0f, 2);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, nv_scaled(bf16_lo(v[u].w), rz), nv_scaled(bf16_hi(v[u].w), rz), 1.0f, 3);
    if (bad) {
      q = 0;
      sbc = 0x7F;
    }
    if (c < nchunks) __builtin_nontemporal_store(q, codes + c);
    // Lanes 1, 3, 5, 7 of each group of 8 hold 4 consecutive block scales.
    const uint32_t s2 = dpp<dpp_row_shr(2)>(sbc);
    const uint32_t s4 = dpp<dpp_row_shr(4)>(sbc);
    const uint32_t s6 = dpp<dpp_row_shr(6)>(sbc);
    const int64_t blk = c >> 1;
    if ((lane & 7) == 7 && c < nchunks) {
      *(uint32_t*)(scales + (blk - 3)) = s6 | (s4 << 8) | (s2 << 16) | (sbc << 24);
    }
    if ((lane & 1) == 0 && c < nchunks && c - (lane & 7) + 7 >= nchunks) scales[blk] = (uint8_t)sbc;
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
  if (panel) {
    // MXFP4 in the K-panel layout: workgroups of 32 rows x one 256-element panel.
    const dim3 pgrid((unsigned)((rows + 31) / 32), (unsigned)(cols / 256));
    const int64_t cpr = cols / 8;
    if (oas && rot)
      quant_mx_kernel<kMXFP4, true, true, true><<<pgrid, kThreads, 0, s>>>(X, codes, S, rows, cpr);
    else if (oas)
      quant_mx_kernel<kMXFP4, true, false, true><<<pgrid, kThreads, 0, s>>>(X, codes, S, rows, cpr);
    else if (rot)
      quant_mx_kernel<kMXFP4, false, true, true><<<pgrid, kThreads, 0, s>>>(X, codes, S, rows, cpr);
    else
      quant_mx_kernel<kMXFP4, false, false, true><<<pgrid, kThreads, 0, s>>>(X, codes, S, rows, cpr);
    return hipGetLastError();
  }
  if (fmt == kMXFP4) {
    if (oas && rot)
      quant_mx_kernel<kMXFP4, true, true><<<grid, kThreads, 0, s>>>(X, codes, S, nchunks);
    else if (oas)
      quant_mx_kernel<kMXFP4, true, false><<<grid, kThreads, 0, s>>>(X, codes, S, nchunks);
    else if (rot)
      quant_mx_kernel<kMXFP4, false, true><<<grid, kThreads, 0, s>>>(X, codes, S, nchunks);
    else
      quant_mx_kernel<kMXFP4, false, false><<<grid, kThreads, 0, s>>>(X, codes, S, nchunks);
  } else if (fmt == kMXFP8) {
    if (rot)
      quant_mx_kernel<kMXFP8, false, true><<<grid, kThreads, 0, s>>>(X, codes, S, nchunks);
    else
      quant_mx_kernel<kMXFP8, false, false><<<grid, kThreads, 0, s>>>(X, codes, S, nchunks);
  } else if (fmt == kMXFP8E5M2) {
    quant_mx_kernel<kMXFP8E5M2, false, false><<<grid, kThreads, 0, s>>>(X, codes, S, nchunks);
  } else {
    const int64_t nblocks = rows * cols / 32;
    quant_mxfp6_kernel<<<(unsigned)((nblocks + kThreads - 1) / kThreads), kThreads, 0, s>>>(
        X, (u32x2*)codes, S, nblocks);
  }
  return hipGetLastError();
}

// nchunks is a multiple of 16 (cols % 128 = 0), so every DPP row is either
// wholly inside the tensor or wholly past its end.
hipError_t quant_mbs(int64_t rows, int64_t cols, const void* x, void* codes, void* scales,
                     hipStream_t s) {
  const int64_t nchunks = rows * cols / 8;
  uint8_t* S = (uint8_t*)scales;
  quant_mbs_kernel<<<(unsigned)grid_for(nchunks), kThreads, 0, s>>>(
      (const u32x4*)x, (uint32_t*)codes, S, S + rows * (cols / 32), nchunks);
  return hipGetLastError();
}

size_t quant_nvfp4_workspace(int64_t, int64_t) { return kMaxPartials * sizeof(uint32_t); }

hipError_t quant_nvfp4(int64_t rows, int64_t cols, const void* x, void* codes, void* scales,
                       float* tensor_scale, void* workspace, hipStream_t s) {
  const int64_t nchunks = rows * cols / 8;
  int64_t np = (nchunks + kThreads * 8 - 1) / (kThreads * 8);
  if (np > kMaxPartials) np = kMaxPartials;
  if (np < 1) np = 1;
  uint32_t* partial = (uint32_t*)workspace;
  nvfp4_amax_partial<<<(unsigned)np, kThreads, 0, s>>>((const u32x4*)x, nchunks, partial);
  quant_nvfp4_kernel<<<(unsigned)grid_for(nchunks), kThreads, 0, s>>>(
      (const u32x4*)x, (uint32_t*)codes, (uint8_t*)scales, partial, (int)np, tensor_scale, nchunks);
  return hipGetLastError();
}

}  // namespace mx
