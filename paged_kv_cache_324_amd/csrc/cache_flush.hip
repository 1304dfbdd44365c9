// cache_flush: a measuring aid, not a step of attention.  A streaming read of a
// caller buffer larger than the Infinity Cache leaves every L2 and the MALL
// holding its own clean lines, so the next kernel finds none of its operands
// cached and, the read having written nothing, no dirty line waits to be
// written back during it.  Each workgroup reads one contiguous share of the
// buffer, 16 KiB a step (four 16-byte chunks per thread, a 4 KiB run per load
// instruction); the words are folded into a register that is stored only
// through a null sink, so the loads stay and nothing is written.
#include "pa_kernels.h"

namespace pa {

__global__ __launch_bounds__(256) void cache_flush_kernel(const uint4* __restrict__ p, int64_t n,
                                                          uint32_t* sink) {
  const int64_t share = (n + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * share;
  const int64_t hi = lo + share < n ? lo + share : n;
  uint32_t acc = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + 768 < hi; i += 1024) {
    const uint4 a = p[i], b = p[i + 256], c = p[i + 512], d = p[i + 768];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < hi; i += 256) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (sink) sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_cache_flush(const void* buf, int64_t chunks, hipStream_t s) {
  if (chunks == 0) return hipSuccess;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 256 * 8) blocks = 256 * 8;   // eight workgroups per compute unit
  launch(cache_flush_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
         static_cast<const uint4*>(buf), chunks, static_cast<uint32_t*>(nullptr));
  return hipGetLastError();
}

}  // namespace pa
