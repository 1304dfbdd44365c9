// Matrix-core (MFMA) and transposed-LDS-read wrappers for gfx950.
//
// Operand lane layouts (checked on the hardware):
//   32x32x16: lane l supplies A[row l%32][k 8(l/32)+i], B[k 8(l/32)+i][col l%32],
//             i = 0..7; accumulator j of lane l is C[row 8(j/4)+4(l/32)+j%4][col l%32].
//   16x16x32: A[row l%16][k 8(l/16)+i], B[k 8(l/16)+i][col l%16], i = 0..7;
//   16x16x16: A[row l%16][k 4(l/16)+i], B[k 4(l/16)+i][col l%16], i = 0..3;
//             for both 16x16 shapes accumulator j of lane l is C[row 4(l/16)+j][col l%16].
#pragma once

#include "pa_device.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                     __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
}

// Four 16-bit elements, transposed across each group of 16 lanes
// (ds_read_b64_tr_b16): lane i of a group receives element i % 4 of the four
// elements that group lane 4 j + i / 4 addressed, j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, unsigned char* lds,
                                                  uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           (int)voffset, 0, 0, 0);
}

}  // namespace pa
