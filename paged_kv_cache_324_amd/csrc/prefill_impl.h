// Chunked prefill over a paged KV cache on gfx950 matrix cores (MFMA).
//
// What is computed: sequence i brings n_i new query tokens that follow
// c_i = context_lens[i] - n_i cached tokens; new token t attends to logical
// keys 0 .. c_i + t (bottom-right causal alignment, its own key included):
//   out[t][h] = sum_j softmax_j(scale * q[t][h] . K_j) V_j.
// This is the attention of page "Nano-vLLM-Ascend" (section 2.2.1) over the
// paged layout of section 2.1, run over one chunk of a long prefill at a time
// (page "vllm-ascend architecture", sections 1.1 and 3.1).
//
// Work decomposition.  One workgroup (4 wavefronts) per (sequence, KV head,
// query tile).  A tile holds QT = 128 / G query tokens of all G query heads
// that read the KV head, i.e. 128 rows; wavefront w owns rows 32w .. 32w+31
// (row r = head (r / QT), token (r % QT)), so every K/V tile staged in LDS
// serves 4 x 32 query rows.
//
// Both products are computed transposed so that a lane always owns one query
// row (lane l -> row l % 32 of its wavefront):
//   S^T = K Q^T  (32x32x16 MFMA: A = 32 keys x 16 dims from LDS, B = Q^T held
//                 in registers for the whole kernel),
//   O^T = V^T P^T (A = 32 dims x 16 keys of V^T from LDS, B = P^T straight
//                 from the softmax registers).
// In the 32x32 accumulator layout lane l holds column l % 32 and rows
// 8 (j / 4) + 4 (l / 32) + (j % 4), j = 0..15.  For S^T the column is the
// lane's query, so a row maximum or sum is a reduction over the lane's own
// values plus one exchange with lane l ^ 32.  For the PV product the K index
// of the MFMA runs over keys in the order the S^T accumulator already holds
// them -- half h of the wavefront supplies keys {4h..4h+3, 8+4h..8+4h+3} of
// each 16-key step -- and the V^T operand is read from LDS in that same key
// order, which leaves the sum unchanged.
//
// Softmax statistics are fp32 (page "vLLM-Ascend ...", section 3.1, problem
// 2); the probabilities are rounded to the input dtype for the PV product.
#pragma once

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

constexpr int kPrefillD = 128;
constexpr int kPrefillKeys = 64;                   // keys per KV tile
constexpr int kPrefillKStride = kPrefillD * 2 + 16;  // LDS bytes per key row of the K tile
constexpr int kPrefillVStride = kPrefillKeys * 2 + 8;  // LDS bytes per dim row of the V^T tile
constexpr float kPrefillEmptyMax = -1.0e30f;

template <int DT, int BS, int G>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillArgs a) {
  constexpr int D = kPrefillD;
  constexpr int NK = kPrefillKeys;
  constexpr int QT = 128 / G;
  constexpr int KSTR = kPrefillKStride;
  constexpr int VSTR = kPrefillVStride;
  __shared__ __attribute__((aligned(16))) unsigned char s_k[NK * KSTR];
  __shared__ __attribute__((aligned(16))) unsigned char s_v[D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;

  // Heaviest tiles first: the last query tiles of a chunk see the most keys.
  const int per_tile = a.num_seqs * a.num_kv_heads;
  const int qt = a.q_tiles - 1 - (int)(blockIdx.x / per_tile);
  const int rest = blockIdx.x % per_tile;
  const int rank = rest / a.num_kv_heads;
  const int kvh = rest - rank * a.num_kv_heads;
  const int seq = a.seq_order ? a.seq_order[rank] : rank;
  if (seq < 0 || seq >= a.num_seqs) return;

  const int s0 = a.query_start_loc[seq];
  const int n = min(a.query_start_loc[seq + 1] - s0, a.max_query_len);
  int L = a.context_lens[seq];
  L = max(0, min(L, a.max_blocks * BS));
  const int c = L - n;  // cached tokens before the chunk (negative: caller error)
  const int t0 = qt * QT;
  if (n <= 0 || t0 >= n) return;
  if (s0 < 0 || (int64_t)s0 + n > a.num_tokens) return;  // malformed query_start_loc: skip

  // This lane's query row.
  const int row = wave * 32 + (lane & 31);
  const int g = row / QT;
  const int t = t0 + row % QT;
  const bool row_valid = t < n;
  const int h = kvh * G + g;
  const int vis = min(L, c + t + 1);  // keys visible to this row
  // Keys any row of the workgroup / of this wavefront can see.
  const int tile_last = min(t0 + QT, n) - 1;
  const int kv_end = max(0, min(L, c + tile_last + 1));
  const int wave_t_last = min(t0 + ((wave * 32 + 31) % QT), n - 1);
  const int wave_end = max(0, min(L, c + wave_t_last + 1));

  // Q^T fragments: for dim step ks, lane l holds q[row][16 ks + 8 half .. +7].
  u32x4 qf[D / 16];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)(s0 + (row_valid ? t : 0)) * a.num_heads + h) * D);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 v = qp[ks * 2 + half];
      qf[ks] = row_valid ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m = kPrefillEmptyMax, lsum = 0.f;

  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks;
  const int32_t nb32 = a.num_blocks > INT32_MAX ? INT32_MAX : (int32_t)a.num_blocks;
  const size_t row_bytes = (size_t)a.num_kv_heads * D * 2;
  const unsigned char* kbase = static_cast<const unsigned char*>(a.k_cache) + (size_t)kvh * D * 2;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.v_cache) + (size_t)kvh * D * 2;
  const int ld_key = tid >> 4;    // staging: key row tid/16 (+16 per round), 16-byte chunk tid%16
  const int ld_chunk = tid & 15;

  for (int kv0 = 0; kv0 < kv_end; kv0 += NK) {
    // ---- stage the K tile (row-major) and the V tile (transposed) in LDS
    u32x4 kr[4], vr[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int j = kv0 + it * 16 + ld_key;
      kr[it] = u32x4{0u, 0u, 0u, 0u};
      vr[it] = u32x4{0u, 0u, 0u, 0u};
      if (j < L) {
        const int32_t blk = bt[j / BS];
        if (blk >= 0 && blk < nb32) {
          const size_t off = ((size_t)(uint32_t)blk * BS + (j % BS)) * row_bytes + ld_chunk * 16;
          kr[it] = *reinterpret_cast<const u32x4*>(kbase + off);
          vr[it] = *reinterpret_cast<const u32x4*>(vbase + off);
        }
      }
    }
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int key = it * 16 + ld_key;
      *reinterpret_cast<u32x4*>(s_k + key * KSTR + ld_chunk * 16) = kr[it];
      const uint32_t w[4] = {vr[it].x, vr[it].y, vr[it].z, vr[it].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t x = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
        *reinterpret_cast<uint16_t*>(s_v + (ld_chunk * 8 + e) * VSTR + key * 2) = x;
      }
    }
    __syncthreads();
    if (kv0 >= wave_end) continue;  // nothing in this tile is visible to this wavefront

    // ---- S^T = K Q^T for the tile's two 32-key halves
    f32x16 s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      s[sub] = f32x16{};
      const unsigned char* kp = s_k + (sub * 32 + (lane & 31)) * KSTR + half * 16;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kp + ks * 32);
        s[sub] = mfma32x32x16<DT>(kf, qf[ks], s[sub]);
      }
    }

    // ---- scale, mask, online softmax (this lane's query; partner lane l^32)
    float mx = kPrefillEmptyMax;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kv0 + sub * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
        const float v = key < vis ? s[sub][j] * a.scale_log2 : -__builtin_inff();
        s[sub][j] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    float psum = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = fast_exp2(s[sub][j] - m_new);
        s[sub][j] = p;
        psum += p;
      }
    }
    psum += __shfl_xor(psum, 32);
    lsum = fmaf(lsum, alpha, psum);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;

    // ---- O^T += V^T P^T over the tile's four 16-key steps
#pragma unroll
    for (int kk = 0; kk < NK / 16; ++kk) {
      const f32x16& ps = s[kk >> 1];
      const int jb = 8 * (kk & 1);
      const u32x4 pf = {pack2<DT>(ps[jb + 0], ps[jb + 1]), pack2<DT>(ps[jb + 2], ps[jb + 3]),
                        pack2<DT>(ps[jb + 4], ps[jb + 5]), pack2<DT>(ps[jb + 6], ps[jb + 7])};
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const unsigned char* vp = s_v + (dt * 32 + (lane & 31)) * VSTR + (16 * kk + 4 * half) * 2;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 16);
        o[dt] = mfma32x32x16<DT>(u32x4{lo.x, lo.y, hi.x, hi.y}, pf, o[dt]);
      }
    }
  }

  // ---- normalise and store: lane holds dims 32 dt + 8 (j/4) + 4 half + (j%4)
  if (!row_valid) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // no visible key: zero row
  uint16_t* op = static_cast<uint16_t*>(a.out) + ((int64_t)(s0 + t) * a.num_heads + h) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const int d = dt * 32 + 8 * jq + 4 * half;
      const u32x2 v = {pack2<DT>(o[dt][4 * jq + 0] * inv, o[dt][4 * jq + 1] * inv),
                       pack2<DT>(o[dt][4 * jq + 2] * inv, o[dt][4 * jq + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + d) = v;
    }
  }
}

template <int DT, int BS, int G>
hipError_t launch_prefill_t(const PrefillArgs& a0, hipStream_t s) {
  PrefillArgs a = a0;
  constexpr int QT = 128 / G;
  a.q_tiles = (a.max_query_len + QT - 1) / QT;
  const int64_t grid = (int64_t)a.q_tiles * a.num_seqs * a.num_kv_heads;
  if (grid == 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<DT, BS, G>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int BS>
hipError_t launch_prefill_g(const PrefillArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_prefill_t<DT, BS, 1>(a, s);
    case 2: return launch_prefill_t<DT, BS, 2>(a, s);
    case 4: return launch_prefill_t<DT, BS, 4>(a, s);
    case 8: return launch_prefill_t<DT, BS, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_prefill_dt(const PrefillArgs& a, int block_size, int group, hipStream_t s) {
  switch (block_size) {
    case 16: return launch_prefill_g<DT, 16>(a, group, s);
    case 32: return launch_prefill_g<DT, 32>(a, group, s);
    case 256: return launch_prefill_g<DT, 256>(a, group, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
