// reshape_and_cache: scatter this step's new K/V rows into their cache slots.
//
// The cache keeps each block as (block_size, num_kv_heads, head_dim) (page
// "Nano-vLLM-Ascend", section 2.1, Block structure), so all heads of one token
// form one contiguous num_kv_heads * head_dim row, and flat slot s starts at
// element s * num_kv_heads * head_dim.  A thread moves one 16-byte chunk of a
// token: consecutive threads cover one token's K row, then its V row, so every
// wavefront reads and writes whole contiguous rows.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

// One workgroup per U groups of tokens: a group is TPB = max(1, 256 / per_token)
// tokens of per_token = 2 row_chunks 16-byte chunks each (K row then V row);
// when a token has more than 256 chunks its workgroup loops over them.  Each
// thread issues the loads of its chunk in all U groups (slot and row, the
// row read even for a skipped token: it lies in the input) before any store,
// so a thread keeps U rows in flight and the copy costs one memory round trip
// before its stores, not U.  Every index is 32-bit within the workgroup.
template <int U>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ReshapeArgs a) {
  const int per_token = 2 * a.row_chunks;
  const int tpb = per_token >= 256 ? 1 : 256 / per_token;
  const int span = tpb * per_token;
  for (int local = threadIdx.x; local < span; local += 256) {
    const int lt = local / per_token;
    const int rem = local - lt * per_token;
    const bool is_v = rem >= a.row_chunks;
    const int chunk = is_v ? rem - a.row_chunks : rem;
    int64_t slot[U];
    u32x4 row[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tk = ((int64_t)blockIdx.x * U + u) * tpb + lt;
      const bool in = tk < a.num_tokens;
      const int64_t t = in ? tk : 0;  // past the last token: token 0's row, not stored
      slot[u] = in ? a.slot_mapping[t] : -1;
      row[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(is_v ? a.value : a.key) +
                                          t * a.row_chunks + chunk);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      asm volatile("" : "+v"(row[u]));  // keeps every row load ahead of the slot tests
      report_index_error(a.index_errors, slot[u] >= a.num_slots, kErrSlot, slot[u]);
      if (slot[u] < 0 || slot[u] >= a.num_slots) continue;  // padding token / outside the pool
      u32x4* dst = reinterpret_cast<u32x4*>(is_v ? a.v_cache : a.k_cache) +
                   slot[u] * a.row_chunks + chunk;
      __builtin_nontemporal_store(row[u], dst);
    }
  }
}

PA_LAYOUT_PROBE(reshape_and_cache)

hipError_t launch_reshape_and_cache(const ReshapeArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  const int per_token = 2 * a.row_chunks;
  const int64_t tpb = per_token >= 256 ? 1 : 256 / per_token;
  const int64_t groups = (a.num_tokens + tpb - 1) / tpb;
  // Groups per workgroup: as many (up to 16) as keep at least 256 workgroups, one
  // per compute unit; a copy of 4096 tokens x 8 heads x 128 dims took 8.9 us with
  // one group per workgroup and 6.6 us with sixteen.
  int u = 1;
  while (u < 16 && groups / (2 * u) >= 256) u *= 2;
  const int64_t blocks = (groups + u - 1) / u;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  switch (u) {
    case 1: launch(reshape_and_cache_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
    case 2: launch(reshape_and_cache_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
    case 4: launch(reshape_and_cache_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
    case 8: launch(reshape_and_cache_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
    default: launch(reshape_and_cache_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace pa
