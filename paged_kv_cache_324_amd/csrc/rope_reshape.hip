// rope_reshape_and_cache: rotary position embedding fused with the cache write.
//
// The pages apply the rotary embedding through a device primitive taking
// (x, cos, sin), whose backward is the same primitive with -sin (page
// "Nano-vLLM-Ascend", section 5.1), and they name operator fusion as the way to
// save passes over memory (page "vLLM-Ascend ...", section 5).  Here the keys of
// this step's tokens are rotated on their way into the cache, so the rotated
// key never makes a round trip through HBM; the queries are rotated in place in
// the same launch.
//
// Rotation: the head dimension is cut into halves, and pair (x_i, x_{i+D/2}) of
// a token at position p becomes
//   (x_i c - x_{i+D/2} s,  x_{i+D/2} c + x_i s),  c = cos[p][i], s = sin[p][i],
// each product and the sum/difference rounded to fp32 on its own (no fused
// multiply-add), then rounded once to the 16-bit type (nearest even).
//
// Work items: per token, every query row, key row and value row is split into
// D/16 items; item c of a row owns elements [8c, 8c+8) of the first half and
// the same range of the second half (two 16-byte chunks), so consecutive
// threads read and write whole contiguous rows; one workgroup per token.
// Value items copy their two chunks to the cache bit for bit.  A token whose position is outside the
// table changes nothing; a negative or out-of-pool slot skips the cache write
// (the query is still rotated).
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

// One workgroup per token (blockDim = its item count rounded up to whole
// wavefronts, at most 1024; a token with more items loops).  The token's
// position and slot are read once, as scalars.
template <int DT, int D>
__global__ __launch_bounds__(1024) void rope_reshape_kernel(RopeReshapeArgs a) {
  constexpr int P = D / 16;          // items per row
  constexpr int H2 = D / 2;          // elements per half
  const int64_t t = blockIdx.x;
  const int64_t pos = a.positions[t];
  if (pos < 0 || pos >= a.max_position) return;    // the token is left alone
  const int hq = a.q ? a.num_heads : 0;
  const int items = (hq + 2 * a.num_kv_heads) * P;
  const int64_t slot_raw = a.slot_mapping[t];
  if (threadIdx.x == 0) report_index_error(a.index_errors, slot_raw >= a.num_slots, kErrSlot, slot_raw);
  const bool cache_ok = slot_raw >= 0 && slot_raw < a.num_slots;  // else padding / outside the pool
  const int64_t slot = cache_ok ? slot_raw : 0;
  const float* cos_row = a.cos + pos * H2;
  const float* sin_row = a.sin + pos * H2;
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int row = it / P;
    const int c = it - row * P;
    const bool is_q = row < hq;
    if (!is_q && !cache_ok) continue;
    const int kr = row - hq;                           // key rows, then value rows
    const bool is_v = kr >= a.num_kv_heads;
    const int kvh = is_v ? kr - a.num_kv_heads : kr;
    const int64_t dst_row = (slot * a.num_kv_heads + kvh) * D;     // element offset in a cache
    if (is_v) {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.value) +
                                                        (t * a.num_kv_heads + kvh) * D);
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.v_cache) + dst_row);
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + c), dst + c);
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + P + c), dst + P + c);
      continue;
    }
    const uint16_t* src = is_q ? static_cast<const uint16_t*>(a.q) + (t * hq + row) * D
                               : static_cast<const uint16_t*>(a.key) + (t * a.num_kv_heads + kvh) * D;
    const u32x4 x1 = reinterpret_cast<const u32x4*>(src)[c];
    const u32x4 x2 = reinterpret_cast<const u32x4*>(src + H2)[c];
    const float4* cp = reinterpret_cast<const float4*>(cos_row + 8 * c);
    const float4* sp = reinterpret_cast<const float4*>(sin_row + 8 * c);
    const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
    const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const u32x4 y1 = rope_half8<DT>(x1, x2, cs, sn, true);
    const u32x4 y2 = rope_half8<DT>(x2, x1, cs, sn, false);
    if (is_q) {
      uint16_t* qrow = static_cast<uint16_t*>(a.q) + (t * hq + row) * D;
      reinterpret_cast<u32x4*>(qrow)[c] = y1;
      reinterpret_cast<u32x4*>(qrow + H2)[c] = y2;
    } else {
      uint16_t* krow = static_cast<uint16_t*>(a.k_cache) + dst_row;
      __builtin_nontemporal_store(y1, reinterpret_cast<u32x4*>(krow) + c);
      __builtin_nontemporal_store(y2, reinterpret_cast<u32x4*>(krow + H2) + c);
    }
  }
}

PA_LAYOUT_PROBE(rope_reshape)

hipError_t launch_rope_reshape(const RopeReshapeArgs& a, int dtype, int head_dim, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.num_tokens > INT32_MAX) return hipErrorInvalidValue;
  const int hq = a.q ? a.num_heads : 0;
  const int64_t items = (int64_t)(hq + 2 * a.num_kv_heads) * (head_dim / 16);
  const int threads = (int)(items >= 1024 ? 1024 : (items + 63) / 64 * 64);
  const dim3 grid((unsigned)a.num_tokens), block(threads);
  if (dtype == DT_BF16) {
    if (head_dim == 128) launch((rope_reshape_kernel<DT_BF16, 128>), grid, block, 0, s, a);
    else if (head_dim == 64) launch((rope_reshape_kernel<DT_BF16, 64>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 128) launch((rope_reshape_kernel<DT_F16, 128>), grid, block, 0, s, a);
    else if (head_dim == 64) launch((rope_reshape_kernel<DT_F16, 64>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
