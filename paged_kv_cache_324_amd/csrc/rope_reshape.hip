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
// threads read and write whole contiguous rows.
// Value items copy their two chunks to the cache bit for bit.  A token whose position is outside the
// table changes nothing; a negative or out-of-pool slot skips the cache write
// (the query is still rotated).
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

// One workgroup per U consecutive tokens (blockDim = a token's item count
// rounded up to whole wavefronts, at most 1024; a token with more items loops).
// A thread takes the same item of each of the U tokens and loads all their
// positions, slots and rows before computing and storing any, so it keeps U
// rows in flight; each token's table entries are read as it is rotated.
template <int DT, int D, int U>
__global__ __launch_bounds__(1024) void rope_reshape_kernel(RopeReshapeArgs a) {
  constexpr int P = D / 16;          // items per row
  constexpr int H2 = D / 2;          // elements per half
  const int hq = a.q ? a.num_heads : 0;
  const int items = (hq + 2 * a.num_kv_heads) * P;
  int64_t tk[U], slot[U], pos[U];
  bool rope_ok[U], cache_ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    tk[u] = (int64_t)blockIdx.x * U + u;
    const bool in = tk[u] < a.num_tokens;
    const int64_t tt = in ? tk[u] : 0;
    pos[u] = in ? a.positions[tt] : -1;
    const int64_t slot_raw = in ? a.slot_mapping[tt] : -1;
    if (threadIdx.x == 0 && in && pos[u] >= 0 && pos[u] < a.max_position)
      report_index_error(a.index_errors, slot_raw >= a.num_slots, kErrSlot, slot_raw);
    rope_ok[u] = pos[u] >= 0 && pos[u] < a.max_position;   // else the token is left alone
    cache_ok[u] = rope_ok[u] && slot_raw >= 0 && slot_raw < a.num_slots;  // else padding / outside the pool
    slot[u] = cache_ok[u] ? slot_raw : 0;
    if (!rope_ok[u]) pos[u] = 0;   // table row 0 is read and not used
    if (!in) tk[u] = 0;
  }
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int row = it / P;
    const int c = it - row * P;
    const bool is_q = row < hq;
    const int kr = row - hq;                           // key rows, then value rows
    const bool is_v = !is_q && kr >= a.num_kv_heads;
    const int kvh = is_v ? kr - a.num_kv_heads : kr;
    u32x4 x1[U], x2[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint16_t* src =
          is_q ? static_cast<const uint16_t*>(a.q) + (tk[u] * hq + row) * D
               : static_cast<const uint16_t*>(is_v ? a.value : a.key) + (tk[u] * a.num_kv_heads + kvh) * D;
      x1[u] = is_v ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + c)
                   : reinterpret_cast<const u32x4*>(src)[c];
      x2[u] = is_v ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + H2) + c)
                   : reinterpret_cast<const u32x4*>(src + H2)[c];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool write = is_q ? rope_ok[u] : cache_ok[u];
      if (!write) continue;
      const int64_t dst_row = (slot[u] * a.num_kv_heads + kvh) * D;   // element offset in a cache
      if (is_v) {
        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.v_cache) + dst_row);
        __builtin_nontemporal_store(x1[u], dst + c);
        __builtin_nontemporal_store(x2[u], dst + P + c);
        continue;
      }
      const float4* cp = reinterpret_cast<const float4*>(a.cos + pos[u] * H2 + 8 * c);
      const float4* sp = reinterpret_cast<const float4*>(a.sin + pos[u] * H2 + 8 * c);
      const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
      const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      const u32x4 y1 = rope_half8<DT>(x1[u], x2[u], cs, sn, true);
      const u32x4 y2 = rope_half8<DT>(x2[u], x1[u], cs, sn, false);
      if (is_q) {
        uint16_t* qrow = static_cast<uint16_t*>(a.q) + (tk[u] * hq + row) * D;
        reinterpret_cast<u32x4*>(qrow)[c] = y1;
        reinterpret_cast<u32x4*>(qrow + H2)[c] = y2;
      } else {
        uint16_t* krow = static_cast<uint16_t*>(a.k_cache) + dst_row;
        __builtin_nontemporal_store(y1, reinterpret_cast<u32x4*>(krow) + c);
        __builtin_nontemporal_store(y2, reinterpret_cast<u32x4*>(krow + H2) + c);
      }
    }
  }
}

PA_LAYOUT_PROBE(rope_reshape)

template <int DT, int D>
void launch_rope_u(const RopeReshapeArgs& a, int u, dim3 block, hipStream_t s) {
  const dim3 grid((unsigned)((a.num_tokens + u - 1) / u));
  switch (u) {
    case 1: launch((rope_reshape_kernel<DT, D, 1>), grid, block, 0, s, a); break;
    default: launch((rope_reshape_kernel<DT, D, 2>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_rope_reshape(const RopeReshapeArgs& a, int dtype, int head_dim, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.num_tokens > INT32_MAX) return hipErrorInvalidValue;
  const int hq = a.q ? a.num_heads : 0;
  const int64_t items = (int64_t)(hq + 2 * a.num_kv_heads) * (head_dim / 16);
  const int threads = (int)(items >= 1024 ? 1024 : (items + 63) / 64 * 64);
  // Tokens per workgroup: two once that keeps at least 512 workgroups (the
  // chunked-prefill chunk of 4096 tokens: 21.0 -> 19.3 us; four took 24.5 us,
  // at 89 VGPRs and five wavefronts per SIMD).
  const int u = a.num_tokens >= 2048 ? 2 : 1;
  const dim3 block(threads);
  if (dtype == DT_BF16) {
    if (head_dim == 128) launch_rope_u<DT_BF16, 128>(a, u, block, s);
    else if (head_dim == 64) launch_rope_u<DT_BF16, 64>(a, u, block, s);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 128) launch_rope_u<DT_F16, 128>(a, u, block, s);
    else if (head_dim == 64) launch_rope_u<DT_F16, 64>(a, u, block, s);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
