// Device helpers shared by the gfx950 paged-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"

namespace pa {

// Records an index error in a PA_CHECK_INDICES build (see IndexErrors);
// compiles to nothing in other builds.
__device__ __forceinline__ void report_index_error(IndexErrors* e, bool bad, uint32_t kind,
                                                   int64_t value) {
#ifdef PA_CHECK_INDICES
  if (bad && e != nullptr) {
    atomicOr(&e->kinds, kind);
    if (atomicCAS(&e->first_kind, 0u, kind) == 0u) e->first_value = value;
  }
#else
  (void)e;
  (void)bad;
  (void)kind;
  (void)value;
#endif
}

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

template <int AUX = 0>
__device__ __forceinline__ float buffer_load4f(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voffset, 0, AUX));
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

// ---- rotary embedding ------------------------------------------------------------
// Eight dimensions of one half of a rotated row: `own` holds them, `partner`
// the same eight dimensions of the other half, cs / sn the table entries of
// their pair index.  First half: own c - partner s; second half:
// own c + partner s.  Each product and the sum or difference is rounded to fp32
// on its own (no fused multiply-add), then the result to the 16-bit type, so
// every kernel that rotates produces the same bits.
template <int DT>
__device__ __forceinline__ u32x4 rope_half8(const u32x4& own, const u32x4& partner, const float* cs,
                                            const float* sn, bool first_half) {
#pragma clang fp contract(off)
  const uint32_t ow[4] = {own.x, own.y, own.z, own.w};
  const uint32_t pw[4] = {partner.x, partner.y, partner.z, partner.w};
  uint32_t r[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float ol = lo_f32<DT>(ow[w]), oh = hi_f32<DT>(ow[w]);
    const float pl = lo_f32<DT>(pw[w]), ph = hi_f32<DT>(pw[w]);
    const float cl = cs[2 * w], ch = cs[2 * w + 1], sl = sn[2 * w], sh = sn[2 * w + 1];
    const float al = ol * cl, ah = oh * ch, bl = pl * sl, bh = ph * sh;
    r[w] = first_half ? pack2<DT>(al - bl, ah - bh) : pack2<DT>(al + bl, ah + bh);
  }
  return u32x4{r[0], r[1], r[2], r[3]};
}

// The eight table entries (cos or sin) starting at pair index i0 of row pos.
__device__ __forceinline__ void rope_row8(const float* table, int64_t pos, int half_dim, int i0,
                                          float* out) {
  const float4* p = reinterpret_cast<const float4*>(table + pos * half_dim + i0);
  const float4 a = p[0], b = p[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
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

// Max / sum over the lane pair (l, l ^ 32) or (l, l ^ 16) of a wavefront by a vector-ALU
// lane swap instead of an LDS permute: v_permlane32_swap / v_permlane16_swap with both
// operands x leave, on every lane, x of the pair's lower lane in the first result and x of
// its upper lane in the second (lane layout checked on gfx950).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace pa
