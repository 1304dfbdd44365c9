// copy_blocks: the copy-on-write step of the block manager.  A block that two
// sequences share (reference count > 1) and one of them is about to write is
// first copied whole to a private block (page "Nano-vLLM-Ascend", section 2.1,
// Block with reference count; page "vLLM-Ascend ...", section 4, block
// sharing).  A cache block is block_size * num_kv_heads * head_dim contiguous
// 16-bit elements, so a copy is a flat move of `block_chunks` 16-byte chunks
// for K and the same for V; each thread moves one chunk per step of a
// grid-stride loop over all (pair, K/V, chunk).
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int64_t per_pair = 2 * a.block_chunks;
  const int64_t total = a.num_copies * per_pair;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t i = idx / per_pair;
    const int64_t rem = idx - i * per_pair;
    const bool is_v = rem >= a.block_chunks;
    const int64_t chunk = is_v ? rem - a.block_chunks : rem;
    const int64_t src = a.src[i], dst = a.dst[i];
    if (chunk == 0 && !is_v) {
      report_index_error(a.index_errors, src < 0 || src >= a.num_blocks, kErrBlockId, src);
      report_index_error(a.index_errors, dst < 0 || dst >= a.num_blocks, kErrBlockId, dst);
    }
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks || src == dst) continue;
    u32x4* cache = static_cast<u32x4*>(is_v ? a.v_cache : a.k_cache);
    cache[dst * a.block_chunks + chunk] = cache[src * a.block_chunks + chunk];
  }
}

PA_LAYOUT_PROBE(copy_blocks)

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s) {
  const int64_t total = a.num_copies * 2 * a.block_chunks;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  launch(copy_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
