// The K-panel layout of an MXFP4 operand (mx_pack): codes [cols/256][rows][128]
// and scales [cols/256][rows][8] from mx_quantize's [rows][cols/2] and
// [rows][cols/32]. A byte permutation with no arithmetic; each thread writes
// one 16-byte code chunk (or one 8-byte scale group), so the stores are
// contiguous and the loads gather 16-byte pieces of the source rows.
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Destination chunk i = (p * rows + r) * 8 + c holds bytes 128 p + 16 c ..
// + 15 of row r, i.e. source chunk (r * panels + p) * 8 + c.
__global__ __launch_bounds__(kThreads) void pack_codes_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst, int64_t rows,
                                                              int64_t panels) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows * panels * 8) return;
  const int64_t c = i & 7, pr = i >> 3;
  const int64_t r = pr % rows, p = pr / rows;
  dst[i] = src[(r * panels + p) * 8 + c];
}

// Destination group i = p * rows + r holds the 8 scales of blocks 8 p .. 8 p + 7
// of row r, source group r * panels + p.
__global__ __launch_bounds__(kThreads) void pack_scales_kernel(const u32x2* __restrict__ src,
                                                               u32x2* __restrict__ dst, int64_t rows,
                                                               int64_t panels) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows * panels) return;
  const int64_t r = i % rows, p = i / rows;
  dst[i] = src[r * panels + p];
}

}  // namespace

hipError_t pack_mxfp4(int64_t rows, int64_t cols, const void* codes, const void* scales,
                      void* packed_codes, void* packed_scales, hipStream_t s) {
  const int64_t panels = cols / 256;
  const int64_t nchunks = rows * panels * 8, ngroups = rows * panels;
  MX_TRY(launch_kernel(&pack_codes_kernel, (unsigned)((nchunks + kThreads - 1) / kThreads), kThreads, 0, s, 
      (const u32x4*)codes, (u32x4*)packed_codes, rows, panels));
  MX_TRY(launch_kernel(&pack_scales_kernel, (unsigned)((ngroups + kThreads - 1) / kThreads), kThreads, 0, s, 
      (const u32x2*)scales, (u32x2*)packed_scales, rows, panels));
  return hipSuccess;
}

}  // namespace mx
