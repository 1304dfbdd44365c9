// Device helpers shared by the gfx950 paged-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum : int { DT_F16 = 0, DT_BF16 = 1 };

// Word 3 of a raw buffer resource on the gfx9 family (32-bit data format,
// no swizzle).  Loads past `num_records` bytes return zero without touching
// memory, which is how the kernels mask tail slots and missing blocks.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}

// Cache-policy bits of a buffer instruction on gfx94x/gfx950: nt marks data
// that is read once (streamed), so it does not displace reused lines.
constexpr int kCachePolicyNT = 2;

template <int AUX = 0>
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voffset, 0, AUX);
}

// ---- 16-bit float pairs packed in a dword ------------------------------------
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);

template <>
__device__ __forceinline__ float dot2<DT_BF16>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

template <>
__device__ __forceinline__ float dot2<DT_F16>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                false);
}

template <int DT>
__device__ __forceinline__ float lo_f32(uint32_t x) {
  if constexpr (DT == DT_BF16) {
    return __uint_as_float(x << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
  }
}

template <int DT>
__device__ __forceinline__ float hi_f32(uint32_t x) {
  if constexpr (DT == DT_BF16) {
    return __uint_as_float(x & 0xffff0000u);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  }
}

// Round two fp32 values to the 16-bit type (nearest even) and pack them.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == DT_BF16) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <int DT>
__device__ __forceinline__ uint16_t to_u16(float a) {
  if constexpr (DT == DT_BF16) {
    return __builtin_bit_cast(uint16_t, (__bf16)a);
  } else {
    return __builtin_bit_cast(uint16_t, (_Float16)a);
  }
}

// ---- cross-lane sums within a DPP row ------------------------------------------
#define PA_DPP(x, ctrl) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), (ctrl), 0xF, 0xF, false))

// Sum over groups of LANES consecutive lanes (LANES = 8 or 16); every lane of
// the group receives the total.  Quad swaps, then the half-row and row
// mirrors pair each quad / half with its partner.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 8 || LANES == 16, "group of 8 or 16 lanes");
  x += PA_DPP(x, 0xB1);   // quad_perm [1,0,3,2]
  x += PA_DPP(x, 0x4E);   // quad_perm [2,3,0,1]
  x += PA_DPP(x, 0x141);  // row_half_mirror
  if constexpr (LANES == 16) x += PA_DPP(x, 0x140);  // row_mirror
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
