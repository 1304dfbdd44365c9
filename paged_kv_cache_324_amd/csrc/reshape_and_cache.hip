// reshape_and_cache: scatter this step's new K/V rows into their cache slots.
//
// The cache keeps each block as (block_size, num_kv_heads, head_dim) (page
// "Nano-vLLM-Ascend", section 2.1, Block structure), so all heads of one token
// form one contiguous num_kv_heads * head_dim row, and flat slot s starts at
// element s * num_kv_heads * head_dim.  Each thread moves one 16-byte chunk:
// consecutive threads cover one token's K row, then its V row, so every
// wavefront reads and writes whole contiguous rows.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

// One workgroup per group of tokens: TPB = max(1, 256 / per_token) tokens of
// per_token = 2 row_chunks 16-byte chunks each (K row then V row); when a
// token has more than 256 chunks its workgroup loops over them.  The slot is
// read once per token and every index is 32-bit within the workgroup.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ReshapeArgs a) {
  const int per_token = 2 * a.row_chunks;
  const int tpb = per_token >= 256 ? 1 : 256 / per_token;
  const int64_t tbase = (int64_t)blockIdx.x * tpb;
  const int span = tpb * per_token;
  for (int local = threadIdx.x; local < span; local += 256) {
    const int lt = local / per_token;
    const int rem = local - lt * per_token;
    const int64_t t = tbase + lt;
    if (t >= a.num_tokens) break;
    const bool is_v = rem >= a.row_chunks;
    const int chunk = is_v ? rem - a.row_chunks : rem;
    const u32x4* src = reinterpret_cast<const u32x4*>(is_v ? a.value : a.key) +
                       t * a.row_chunks + chunk;
    // The slot and the row are independent: both loads are issued before either
    // is used (the row is read even for a skipped token; it lies in the input),
    // so the copy costs one memory round trip before its store, not two.
    const int64_t slot = a.slot_mapping[t];
    u32x4 row = __builtin_nontemporal_load(src);
    asm volatile("" : "+v"(row));  // keeps the row load ahead of the slot test (no sinking)
    report_index_error(a.index_errors, slot >= a.num_slots, kErrSlot, slot);
    if (slot < 0 || slot >= a.num_slots) continue;  // padding token / outside the pool
    u32x4* dst = reinterpret_cast<u32x4*>(is_v ? a.v_cache : a.k_cache) +
                 slot * a.row_chunks + chunk;
    __builtin_nontemporal_store(row, dst);
  }
}

PA_LAYOUT_PROBE(reshape_and_cache)

hipError_t launch_reshape_and_cache(const ReshapeArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  const int per_token = 2 * a.row_chunks;
  const int64_t tpb = per_token >= 256 ? 1 : 256 / per_token;
  const int64_t blocks = (a.num_tokens + tpb - 1) / tpb;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  launch(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
