// bf16 matrix-core wrappers (gfx950 MFMA) shared by the kernels.
//  v_mfma_f32_16x16x32_bf16: A 16x32, B 32x16, C/D 16x16 fp32. Lane i holds
//    A[i%16][8(i/16) .. +8], B[8(i/16) .. +8][i%16], and D rows 4(i/16) .. +4
//    of column i%16.
//  v_mfma_f32_16x16x16_bf16: the same with k-slices of 4.
#pragma once

#include "ls_device.h"

namespace ls {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_16x16x32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_16x16x16(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

}  // namespace ls
