// reshape_and_cache_int8: scatter this step's new K/V rows into an INT8 KV
// cache, quantising each (token, KV head) row symmetrically: scale = amax /
// 127 over the row's head_dim values, code = rint(x / scale) (ties to even),
// all in IEEE float32, an all-zero row giving scale 0 and codes 0.  INT8 is
// the KV-cache compression the pages propose next (page "Nano-vLLM-Ascend",
// section 4.3; page "vLLM-Ascend ...", section 5, which names the score
// precision as the risk; per-row scales keep every row's error within half a
// step of that row's own range).
//
// Layout, head-major within a block: codes int8 [num_blocks][num_kv_heads]
// [block_size][head_dim], scales float32 [num_blocks][num_kv_heads]
// [block_size], so one head's rows of a block are one contiguous run.  One row
// is handled by D / 8 consecutive lanes, each holding 8 inputs (16 bytes) and
// writing 8 codes.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

template <int DT, int D>
__global__ __launch_bounds__(256) void reshape_int8_kernel(ReshapeInt8Args a) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t rows = a.num_tokens * a.num_kv_heads * 2;
  const int64_t rows_per_grid = (int64_t)gridDim.x * (256 / LPR);
  const int sub = threadIdx.x % LPR;
  for (int64_t r = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR; r < rows;
       r += rows_per_grid) {
    // r = (token * Hkv + head) * 2 + is_v; the whole 16-lane (or 8-lane) group
    // shares r, so it leaves the loop together.
    const int64_t th = r >> 1;
    const bool is_v = r & 1;
    const int64_t t = th / a.num_kv_heads;
    const int head = (int)(th - t * a.num_kv_heads);
    // The slot and the row are independent loads, both issued before either is
    // used (one memory round trip, not two); the row lies in the input even for
    // a skipped token.
    const int64_t slot = a.slot_mapping[t];
    u32x4 x = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(is_v ? a.value : a.key) +
                                             th * D)[sub];
    asm volatile("" : "+v"(x));  // keeps the row load ahead of the slot test (no sinking)
    report_index_error(a.index_errors, slot >= a.num_slots, kErrSlot, slot);
    if (slot < 0 || slot >= a.num_slots) continue;  // padding token / outside the pool
    float f[8] = {lo_f32<DT>(x.x), hi_f32<DT>(x.x), lo_f32<DT>(x.y), hi_f32<DT>(x.y),
                  lo_f32<DT>(x.z), hi_f32<DT>(x.z), lo_f32<DT>(x.w), hi_f32<DT>(x.w)};
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float scale = amax / 127.0f;
    uint32_t packed[2] = {0u, 0u};
    if (scale > 0.f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = (int)__builtin_rintf(f[e] / scale);
        packed[e >> 2] |= ((uint32_t)c & 0xFFu) << (8 * (e & 3));
      }
    }
    const int64_t blk = slot / a.block_size;
    const int off = (int)(slot - blk * a.block_size);
    int8_t* codes = static_cast<int8_t*>(is_v ? a.v_codes : a.k_codes);
    *reinterpret_cast<uint2*>(codes + ((blk * a.num_kv_heads + head) * a.block_size + off) * D + 8 * sub) =
        make_uint2(packed[0], packed[1]);
    if (sub == 0) {
      float* scales = is_v ? a.v_scales : a.k_scales;
      scales[(blk * a.num_kv_heads + head) * a.block_size + off] = scale;
    }
  }
}

PA_LAYOUT_PROBE(reshape_int8)

hipError_t launch_reshape_int8(const ReshapeInt8Args& a, int dtype, int head_dim, hipStream_t s) {
  const int64_t rows = a.num_tokens * a.num_kv_heads * 2;
  if (rows == 0) return hipSuccess;
  const int rows_per_block = 256 / (head_dim / 8);
  int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  const dim3 grid((unsigned)blocks), block(256);
  if (dtype == DT_BF16) {
    if (head_dim == 128) launch((reshape_int8_kernel<DT_BF16, 128>), grid, block, 0, s, a);
    else launch((reshape_int8_kernel<DT_BF16, 64>), grid, block, 0, s, a);
  } else {
    if (head_dim == 128) launch((reshape_int8_kernel<DT_F16, 128>), grid, block, 0, s, a);
    else launch((reshape_int8_kernel<DT_F16, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pa
