// fp32 -> bf16 conversion for the kernels' bf16 outputs.
//
// Round to nearest, ties to even, with overflow to +-Inf and NaN kept a
// (quiet) NaN: gfx950's v_cvt_pk_bf16_f32, which the compiler emits for a
// float2 -> __bf16 x 2 vector conversion. Checked on the device against the
// integer definition (add 0x7FFF plus the kept LSB, keep the high half) for
// every tie and both neighbours of every bf16 value and 2^25 random words:
// identical for all non-NaN inputs. One instruction converts two values,
// and it has no data-dependent branch.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace mx {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two values packed as a dword: lo in bits 15:0, hi in bits 31:16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint16_t bf16_bits(float v) { return (uint16_t)pack_bf16x2(v, 0.0f); }

}  // namespace mx
