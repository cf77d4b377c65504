// W4A16 GEMM on gfx950: bf16 activations (M x K, few rows: decode) times MXFP4
// weights (stored N x K) with fp32 accumulation. Weight-only quantization saves
// memory traffic rather than compute (noticiai.com.br page on Nunchaku W4A4:
// dequantizing weights at compute time mainly saves memory), so this kernel is
// built to stream the weight codes once from HBM at full bandwidth:
//  * a workgroup covers TN = 448 weight rows x 16 activation rows x KP = 2048
//    K (16 steps of 128). Wave w owns rows 112 w .. 112 w + 111 as 7 groups
//    of 16; lane l takes row l % 16 of a group, and at step s lane group
//    g = l / 16 takes E8M0 block 4 s + g, so one 16-byte load instruction
//    covers 16 rows x 64 contiguous bytes. With 448 rows, the 28672-row decode
//    weight splits into 64 x 4 K-splits = 256 workgroups: one per CU, every
//    CU with the same work;
//  * a wave loads half a row group at a time, 8 steps back to back (16 rows x
//    512 contiguous bytes, so DRAM pages are read in bursts), through a ring
//    of kRing half buffers in VGPRs: kRing - 1 halves are in flight while one
//    is used (8 KB each, enough to cover the HBM latency at one wave per
//    SIMD). (Steps spread over the whole kernel re-open every page many times
//    and cap the stream at about half of the HBM rate.) Each block (32 codes) is
//    expanded to bf16 with v_cvt_scalef32_pk_bf16_fp4, which multiplies by
//    the power-of-two scale exactly, and feeds four v_mfma_f32_16x16x32_bf16:
//    MFMA j takes elements 8 j .. 8 j + 7 of the block from every lane group.
//    The activations follow the same K permutation, so the sum over K is
//    unchanged;
//  * the workgroup's activations (16 x KP bf16, 64 KB, 16-byte chunks XOR-
//    swizzled by row) are staged once in LDS, loaded before the weights so
//    that the LDS writes wait for them alone; the 4 waves x 4 row groups share
//    them, so the activation traffic is a quarter of the weights';
//  * every global load is a range-checked buffer load without a branch (rows
//    past N or M, and blocks past K, read as zeros), which keeps the in-order
//    load counter exact so that waits name only the data they need;
//  * K is split across workgroups; partial sums go to a workspace and a second
//    kernel adds them in a fixed order (deterministic, no float atomics).
// Two accumulator chains per row, each 32 MFMAs per split.
#include <mutex>

#include "bf16.h"
#include "mx_internal.h"

// Split-K partials of mx_gemm_noalloc's W4A16 calls: device memory of the
// library itself, one copy per GPU, held until the process ends (for callers
// that cannot allocate). Host code never passes this name to a kernel -- on
// the host it is only a stand-in -- but the address hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) float scratch[mx::kNoAllocScratchBytes / sizeof(float)];

namespace mx {

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kGroups = 7;              // row groups of 16 per wave
constexpr int kRing = 2;                // half buffers in the load ring (kRing - 1 in flight)
constexpr int TN = 4 * 16 * kGroups;    // weight rows per workgroup (112 per wave)
constexpr int TM = 16;                  // activation rows per workgroup
constexpr int KP = 2048;                // K elements per split
constexpr int kSteps = KP / 128;        // 16 steps: 4 blocks (one per lane group) each
constexpr int kHalf = kSteps / 2;       // steps loaded together
constexpr int kARow = KP * 2;           // bytes per LDS activation row
constexpr int kALoads = TM * KP / 8 / kThreads;  // 16-byte activation loads per thread
constexpr uint32_t kRsrcFlags = 0x00020000u;     // raw buffer, gfx9 data format
constexpr uint32_t kOOB = 0x80000000u;           // an offset past every buffer's range

// 8 codes (one dword) -> 8 bf16 times 2^(E-127).
__device__ __forceinline__ bf16x8 expand8(uint32_t q, float s) {
  u32x4 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 0));
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 1));
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 2));
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 3));
  return __builtin_bit_cast(bf16x8, o);
}

// The lane's codes of steps 8 u .. 8 u + 7 for one row (block bbase + 4 s + g
// at step s), and their scales: word q of sc[v] holds the scales of blocks
// bbase + 16 (2 u + v) + 4 q .. + 3, byte g being this lane's block of step
// 8 u + 4 v + q. Blocks past K read as zero codes (and scale 0, harmless
// against them); with valid false nothing is read (all offsets out of range).
__device__ __forceinline__ void load_half(u32x4 (&q)[kHalf], u32x4 (&sc)[kHalf / 4],
                                          __amdgpu_buffer_rsrc_t rB, __amdgpu_buffer_rsrc_t rS,
                                          uint32_t wrow, uint32_t srow, int bbase, int g,
                                          int kblocks, int u, bool valid) {
#pragma unroll
  for (int i = 0; i < kHalf; i++) {
    const int b = bbase + 4 * (kHalf * u + i) + g;
    q[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, valid && b < kblocks ? wrow + (uint32_t)b * 16u : kOOB, 0, 0);
  }
  if (kblocks % 16 == 0) {
#pragma unroll
    for (int v = 0; v < kHalf / 4; v++) {
      const int b = bbase + 16 * (2 * u + v);
      sc[v] = __builtin_amdgcn_raw_buffer_load_b128(rS, valid && b < kblocks ? srow + (uint32_t)b : kOOB, 0, 0);
    }
  } else {
#pragma unroll
    for (int v = 0; v < kHalf / 4; v++) {
      uint32_t w[4];
#pragma unroll
      for (int qq = 0; qq < 4; qq++) {
        const int b = bbase + 16 * (2 * u + v) + 4 * qq + g;  // only byte g is used
        w[qq] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rS, valid && b < kblocks ? srow + (uint32_t)b : kOOB, 0, 0) << (8 * g);
      }
      sc[v] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

// The MFMAs of one loaded half: steps kHalf u .. kHalf u + kHalf - 1, two
// accumulator chains. The activation piece of step i and MFMA j is
// x = 16 i' + 4 g + j (i' = kHalf u + i), stored at slot x ^ r: the XOR only
// touches the low 4 bits, so the slot is 16 i' + ((4 g + j) ^ r) and
// ab[j] = arow + 16 ((4 g + j) ^ r) plus the constant 256 i' addresses it.
__device__ __forceinline__ void compute_half(const u32x4 (&q)[kHalf], const u32x4 (&sc)[kHalf / 4],
                                             const uint8_t* arow, int r, int g, int u,
                                             f32x4 (&acc)[2]) {
  const uint8_t* ab[4];
#pragma unroll
  for (int j = 0; j < 4; j++) ab[j] = arow + (((4 * g + j) ^ r) * 16);
#pragma unroll
  for (int i = 0; i < kHalf; i++) {
    // The scaled converts read only the exponent field of their scale, so
    // the E8M0 byte placed in that field scales by 2^(E-127) for every E,
    // E = 0 included (no special case for the fp32 subnormal 2^-127).
    const uint32_t E = (sc[i / 4][i % 4] >> (8 * g)) & 0xFFu;
    const float scale = __builtin_bit_cast(float, E << 23);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const bf16x8 a = *(const bf16x8*)(ab[j] + 256 * (kHalf * u + i));
      // A scale byte of 255 (E8M0 NaN) gives a scale with exponent field
      // 255, for which the scaled converts return NaN for every code (they
      // read only the scale's exponent): the block dequantizes to NaN.
      const bf16x8 w = expand8(q[i][j], scale);
      acc[j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w, acc[j & 1], 0, 0, 0);
    }
    // One step per scheduling window: hoisting later steps' LDS reads and
    // expansions would need more registers than the load ring leaves.
    __builtin_amdgcn_sched_barrier(0);
  }
}

// grid: x = N tiles, y = M tiles, z = K splits of KP elements.
template <bool DIRECT, int OUT>
__global__ __launch_bounds__(kThreads, 1) void gemm_w4a16_kernel(const uint16_t* __restrict__ A,
                                                              const uint8_t* __restrict__ B,
                                                              const uint8_t* __restrict__ SB,
                                                              void* __restrict__ out, int64_t ldc,
                                                              int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[TM * kARow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.y * TM;
  const int kbeg = blockIdx.z * KP;
  const int kend = min(K, kbeg + KP);
  const int kblocks = K / 32;
  const int bbase = kbeg / 32;      // first block of the split

  // Buffer views based at this workgroup's first weight row and first
  // activation row: 32-bit offsets, and rows past N or M read as zeros.
  const int n0 = blockIdx.x * TN;
  const int nrows = min(TN, N - n0), mrows = min(TM, M - m0);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(B + (int64_t)n0 * (K / 2)), 0, nrows * (K / 2), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(SB + (int64_t)n0 * kblocks), 0, nrows * kblocks, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (int64_t)m0 * K), 0, mrows * K * 2, kRsrcFlags);
  const int lr0 = wave * (16 * kGroups) + r;  // row within the tile, row group 0
  const uint32_t wstride = (uint32_t)16 * (uint32_t)(K / 2), sstride = (uint32_t)16 * (uint32_t)kblocks;
  const uint32_t wrow0 = (uint32_t)lr0 * (uint32_t)(K / 2), srow0 = (uint32_t)lr0 * (uint32_t)kblocks;

  // 1. Activation loads first: [m0, m0 + 16) x [kbeg, kbeg + KP), zero-padded.
  u32x4 av[kALoads];
#pragma unroll
  for (int i = 0; i < kALoads; i++) {
    const int idx = tid + i * kThreads;
    const int row = idx / (KP / 8), c8 = idx % (KP / 8);
    const int k = kbeg + c8 * 8;
    const uint32_t off = k < kend ? ((uint32_t)row * (uint32_t)K + (uint32_t)k) * 2u : kOOB;
    av[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0);
  }
  // 2. The first kRing - 1 halves' codes and scales (half i = 2 grp + u).
  u32x4 qb[kRing][kHalf], sb[kRing][kHalf / 4];
#pragma unroll
  for (int i = 0; i < kRing - 1; i++)
    load_half(qb[i], sb[i], rB, rS, wrow0 + (uint32_t)(i / 2) * wstride,
              srow0 + (uint32_t)(i / 2) * sstride, bbase, g, kblocks, i % 2, true);
  // 3. Activations to LDS (waits only for the activation loads, which were
  //    issued first): 16-byte chunk c of row m at slot c ^ (m mod 16).
#pragma unroll
  for (int i = 0; i < kALoads; i++) {
    const int idx = tid + i * kThreads;
    const int row = idx / (KP / 8), c8 = idx % (KP / 8);
    *(u32x4*)(lA + row * kARow + ((c8 ^ (row & 15)) * 16)) = av[i];
  }
  __syncthreads();

  // 4. Halves i = 2 grp + u of the row groups one after another; the loads
  //    run kRing - 1 halves ahead of the MFMAs through the ring of buffers.
  const uint8_t* arow = lA + r * kARow;
  f32x4 acc[2];
#pragma unroll
  for (int i = 0; i < 2 * kGroups; i++) {
    const int grp = i / 2, u = i % 2;
    const int il = i + kRing - 1;  // the half loaded now
    if (il < 2 * kGroups)
      load_half(qb[il % kRing], sb[il % kRing], rB, rS, wrow0 + (uint32_t)(il / 2) * wstride,
                srow0 + (uint32_t)(il / 2) * sstride, bbase, g, kblocks, il % 2, true);
    if (u == 0) acc[0] = acc[1] = f32x4{0, 0, 0, 0};
    compute_half(qb[i % kRing], sb[i % kRing], arow, r, g, u, acc);
    if (u == 1) {
      // Lane l holds column n of activation rows 4 g + t.
      const int n = n0 + lr0 + 16 * grp;
      const f32x4 sum = acc[0] + acc[1];
      if (n < N) {
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const int m = m0 + 4 * g + t;
          if (m >= M) continue;
          if (DIRECT) {
            if (OUT == kOutF32)
              ((float*)out)[(int64_t)m * ldc + n] = sum[t];
            else
              ((uint16_t*)out)[(int64_t)m * ldc + n] = bf16_bits(sum[t]);
          } else {
            ((float*)out)[((int64_t)blockIdx.z * M + m) * N + n] = sum[t];
          }
        }
      }
    }
  }
}

template <int OUT>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const float* __restrict__ part,
                                                                 void* __restrict__ C, int64_t ldc,
                                                                 int M, int N, int splits) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int m = (int)(i / N), n = (int)(i % N);
  float s = 0.0f;
  for (int z = 0; z < splits; z++) s += part[(int64_t)z * M * N + i];
  if (OUT == kOutF32)
    ((float*)C)[(int64_t)m * ldc + n] = s;
  else
    ((uint16_t*)C)[(int64_t)m * ldc + n] = bf16_bits(s);
}

int splits_for(int64_t K) { return (int)((K + KP - 1) / KP); }

}  // namespace

size_t gemm_w4a16_workspace(int64_t M, int64_t N, int64_t K) {
  const int splits = splits_for(K);
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

hipError_t gemm_w4a16(int64_t M, int64_t N, int64_t K, const void* a, const void* b,
                      const void* sb, int out_dtype, void* c, int64_t ldc, void* workspace,
                      hipStream_t s) {
  const int splits = splits_for(K);
  const dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM), (unsigned)splits);
  const uint16_t* A = (const uint16_t*)a;
  const uint8_t *B = (const uint8_t*)b, *SB = (const uint8_t*)sb;
  const int m = (int)M, n = (int)N, k = (int)K;
  if (splits == 1) {
    if (out_dtype == kOutF32)
      MX_TRY(launch_kernel(&gemm_w4a16_kernel<true, kOutF32>, grid, kThreads, 0, s, A, B, SB, c, ldc, m, n, k));
    else
      MX_TRY(launch_kernel(&gemm_w4a16_kernel<true, kOutBF16>, grid, kThreads, 0, s, A, B, SB, c, ldc, m, n, k));
    return hipSuccess;
  }
  MX_TRY(launch_kernel(&gemm_w4a16_kernel<false, kOutF32>, grid, kThreads, 0, s, A, B, SB, workspace, 0, m, n, k));
  const unsigned rblocks = (unsigned)((M * N + kThreads - 1) / kThreads);
  if (out_dtype == kOutF32)
    MX_TRY(launch_kernel(&splitk_reduce_kernel<kOutF32>, rblocks, kThreads, 0, s, (const float*)workspace, c, ldc, m, n, splits));
  else
    MX_TRY(launch_kernel(&splitk_reduce_kernel<kOutBF16>, rblocks, kThreads, 0, s, (const float*)workspace, c, ldc, m, n, splits));
  return hipSuccess;
}

}  // namespace mx
