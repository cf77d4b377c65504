// The K-panel layout of a quantized operand (mx_pack): codes
// [panels][rows][wb] and scales [panels][rows][sb] from mx_quantize's
// [rows][panels * wb] and [rows][panels * sb], wb and sb the code and scale
// bytes of one row in one panel (MXFP4: 256-element panels, 128 and 8 bytes;
// MXFP8 / E5M2: 64-element panels, 64 and 2; E3M2: 48 and 2; NVFP4: 32 and
// 4). A byte permutation with no arithmetic; each thread writes one 16-byte
// code chunk (or one row's scales of one panel), so the stores are contiguous
// and the loads gather 16-byte pieces of the source rows.
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Destination chunk i = (p * rows + r) * cpr + c holds bytes 16 (cpr p + c) ..
// + 15 of row r, i.e. source chunk (r * panels + p) * cpr + c (cpr = wb / 16
// chunks per row and panel).
__global__ __launch_bounds__(kThreads) void pack_codes_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst, int64_t rows,
                                                              int64_t panels, int cpr) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows * panels * cpr) return;
  const int64_t c = i % cpr, pr = i / cpr;
  const int64_t r = pr % rows, p = pr / rows;
  dst[i] = src[(r * panels + p) * cpr + c];
}

// Destination unit i = p * rows + r holds the scales of row r in panel p
// (one T: sb bytes), source unit r * panels + p.
template <typename T>
__global__ __launch_bounds__(kThreads) void pack_scales_kernel(const T* __restrict__ src,
                                                               T* __restrict__ dst, int64_t rows,
                                                               int64_t panels) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows * panels) return;
  const int64_t r = i % rows, p = i / rows;
  dst[i] = src[r * panels + p];
}

}  // namespace

hipError_t pack_kpanel(int64_t rows, int64_t panels, int wb, int sb, const void* codes,
                       const void* scales, void* packed_codes, void* packed_scales, hipStream_t s) {
  const int cpr = wb / 16;
  const int64_t nchunks = rows * panels * cpr, ngroups = rows * panels;
  const unsigned cgrid = (unsigned)((nchunks + kThreads - 1) / kThreads);
  const unsigned sgrid = (unsigned)((ngroups + kThreads - 1) / kThreads);
  MX_TRY(launch_kernel(&pack_codes_kernel, cgrid, kThreads, 0, s, (const u32x4*)codes,
                       (u32x4*)packed_codes, rows, panels, cpr));
  if (sb == 8)
    MX_TRY(launch_kernel(&pack_scales_kernel<u32x2>, sgrid, kThreads, 0, s, (const u32x2*)scales,
                         (u32x2*)packed_scales, rows, panels));
  else if (sb == 4)
    MX_TRY(launch_kernel(&pack_scales_kernel<uint32_t>, sgrid, kThreads, 0, s, (const uint32_t*)scales,
                         (uint32_t*)packed_scales, rows, panels));
  else
    MX_TRY(launch_kernel(&pack_scales_kernel<uint16_t>, sgrid, kThreads, 0, s, (const uint16_t*)scales,
                         (uint16_t*)packed_scales, rows, panels));
  return hipSuccess;
}

}  // namespace mx
