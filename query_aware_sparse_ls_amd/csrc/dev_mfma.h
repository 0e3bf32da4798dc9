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

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane 16G + L' receives, as element j (j < 4), 16-bit element L' % 4 of the
// 8-byte word addressed by lane 16G + 4j + L' / 4. So if lane 16G + 4j + a
// addresses row R(G, j) at columns 4a .. 4a + 3 of a row-major bf16 tile,
// lane 16G + c receives column c of rows R(G, 0) .. R(G, 3): four k-values
// of one column, the B-operand layout of the matrix cores, in one read.
// (Layout checked on the device: lane L reading word L returns words
// 4j + L/4 element L%4 within its 16-lane group.) p must be 8-byte aligned.
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace ls
