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

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ReshapeArgs a) {
  const int64_t per_token = 2 * (int64_t)a.row_chunks;
  const int64_t total = a.num_tokens * per_token;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t t = idx / per_token;
    const int rem = (int)(idx - t * per_token);
    const bool is_v = rem >= a.row_chunks;
    const int chunk = is_v ? rem - a.row_chunks : rem;
    const int64_t slot = a.slot_mapping[t];
    if (slot < 0 || slot >= a.num_slots) continue;  // padding token / outside the pool
    const u32x4* src = reinterpret_cast<const u32x4*>(is_v ? a.value : a.key) +
                       t * a.row_chunks + chunk;
    u32x4* dst = reinterpret_cast<u32x4*>(is_v ? a.v_cache : a.k_cache) +
                 slot * a.row_chunks + chunk;
    __builtin_nontemporal_store(__builtin_nontemporal_load(src), dst);
  }
}

hipError_t launch_reshape_and_cache(const ReshapeArgs& a, hipStream_t s) {
  const int64_t total = a.num_tokens * 2 * (int64_t)a.row_chunks;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
