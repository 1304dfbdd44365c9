// merge_partials: combine attention rows computed over disjoint sets of keys.
//
// Context parallelism splits one sequence's context across devices (page
// "vllm-ascend architecture", sections 1.1 and 3.1); each shard attends over
// its own keys and reports, per (sequence, query head), its normalised output
// o_n and the log2-domain max m_n and sum l_n of its softmax.  Exact merge:
//   M = max_n m_n,  w_n = l_n 2^(m_n - M),  out = sum_n w_n o_n / sum_n w_n,
// over the shards with l_n > 0 (a shard without keys of the sequence reports
// l_n = 0 and is left out; its o_n and m_n are never used in arithmetic).  A
// row that no shard holds keys for gets zeros and (M, sum) = (-inf, 0).
//
// One wavefront per row; each lane owns D/64 consecutive dimensions of o.  The
// first eight shards' outputs and lane n's (m_n, l_n) are loaded in one round;
// the max and the weights follow by cross-lane operations (shards past 64, if
// any, are read again one by one), and the shards are summed in batches of
// eight.  The merged (M, sum w) can be written too, so merges
// compose (shards of shards).  HBM-bound: num_shards * (D * 2 + 8) bytes read
// and D * 2 (+ 8) written per row.
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

template <int DT, int D>
__global__ __launch_bounds__(64) void merge_partials_kernel(const MergePartialsArgs a) {
  constexpr int E = D / 64;
  constexpr int NB = 8;
  typedef float floatE __attribute__((ext_vector_type(E)));
  typedef typename std::conditional<E == 2, uint32_t, uint16_t>::type RawE;
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int N = a.num_shards;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + row;
  const RawE* po = reinterpret_cast<const RawE*>(static_cast<const uint16_t*>(a.part_o) + row * D) + lane;
  const int64_t ostride = a.num_rows * (D / E);  // RawE words between shards

  // One round of loads: the first batch of outputs together with every
  // lane's own (m, l) (shard = lane).
  RawE pv[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) pv[j] = j < N ? po[j * ostride] : RawE(0);
  const float2 own = lane < N ? ml[lane * a.num_rows] : make_float2(0.f, 0.f);

  float M = own.y > 0.f ? own.x : -__builtin_inff();
  for (int n = lane + 64; n < N; n += 64) {  // only with more than 64 shards
    const float2 v = ml[n * a.num_rows];
    if (v.y > 0.f) M = fmaxf(M, v.x);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const bool any = M != -__builtin_inff();
  // Lane n's weight w_n (shards below 64); shards with l <= 0 (or NaN) weigh 0.
  const float w_own = (any && own.y > 0.f) ? own.y * fast_exp2(own.x - M) : 0.f;

  floatE acc = {};
  float den = 0.f;
  for (int n0 = 0; any && n0 < N; n0 += NB) {
    if (n0 > 0) {
#pragma unroll
      for (int j = 0; j < NB; ++j) pv[j] = n0 + j < N ? po[(n0 + j) * ostride] : RawE(0);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + j;
      float w = 0.f;
      if (n < 64) {
        w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_own), n));
      } else if (n < N) {
        const float2 v = ml[n * a.num_rows];
        w = v.y > 0.f ? v.y * fast_exp2(v.x - M) : 0.f;
      }
      if (n < N && w > 0.f) {
        floatE f;
        f[0] = lo_f32<DT>((uint32_t)pv[j]);
        if constexpr (E == 2) f[1] = hi_f32<DT>((uint32_t)pv[j]);
        acc += w * f;
        den += w;
      }
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  uint16_t* out = static_cast<uint16_t*>(a.out) + row * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) out[e] = to_u16<DT>(acc[e] * inv);
  if (a.out_ml && lane == 0) reinterpret_cast<float2*>(a.out_ml)[row] = make_float2(M, den);
}

PA_LAYOUT_PROBE(merge_partials)

hipError_t launch_merge_partials(const MergePartialsArgs& a, int dtype, int head_dim,
                                 hipStream_t s) {
  const dim3 grid((unsigned)a.num_rows), block(64);
  if (dtype == DT_BF16) {
    if (head_dim == 128) launch((merge_partials_kernel<DT_BF16, 128>), grid, block, 0, s, a);
    else if (head_dim == 64) launch((merge_partials_kernel<DT_BF16, 64>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 128) launch((merge_partials_kernel<DT_F16, 128>), grid, block, 0, s, a);
    else if (head_dim == 64) launch((merge_partials_kernel<DT_F16, 64>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
