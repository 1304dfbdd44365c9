// cache_flush: a measuring aid, not a step of attention.  A streaming read of a
// caller buffer larger than the Infinity Cache leaves every L2 and the MALL
// holding its own clean lines, so the next kernel finds none of its operands
// cached and, the read having written nothing, no dirty line waits to be
// written back during it.  Each workgroup reads one contiguous share of the
// buffer, 16 KiB a step (four 16-byte chunks per thread, a 4 KiB run per load
// instruction); the words are folded into a register that is stored only
// through a null sink, so the loads stay and nothing is written.
//
// stream_read: the same walk with non-temporal loads, which do not allocate
// lines in the caches for the data they bring.  Timed over a buffer much larger
// than the Infinity Cache, it gives the device's streaming read rate from HBM.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

template <bool NT>
__device__ __forceinline__ u32x4 read16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__device__ __forceinline__ void read_walk(const u32x4* __restrict__ p, int64_t n, uint32_t* sink) {
  const int64_t share = (n + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * share;
  const int64_t hi = lo + share < n ? lo + share : n;
  uint32_t acc = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + 768 < hi; i += 1024) {
    const u32x4 a = read16<NT>(p + i), b = read16<NT>(p + i + 256), c = read16<NT>(p + i + 512),
                d = read16<NT>(p + i + 768);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < hi; i += 256) {
    const u32x4 a = read16<NT>(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (sink) sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void cache_flush_kernel(const u32x4* __restrict__ p, int64_t n,
                                                          uint32_t* sink) {
  read_walk<false>(p, n, sink);
}

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n,
                                                          uint32_t* sink) {
  read_walk<true>(p, n, sink);
}

hipError_t launch_cache_flush(const void* buf, int64_t chunks, bool non_temporal, hipStream_t s) {
  if (chunks == 0) return hipSuccess;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 256 * 8) blocks = 256 * 8;   // eight workgroups per compute unit
  const u32x4* p = static_cast<const u32x4*>(buf);
  if (non_temporal)
    launch(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, chunks,
           static_cast<uint32_t*>(nullptr));
  else
    launch(cache_flush_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, chunks,
           static_cast<uint32_t*>(nullptr));
  return hipGetLastError();
}

}  // namespace pa
