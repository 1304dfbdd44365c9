// Paged-attention decode for gfx950: partition kernel + partition merge kernel.
//
// What is computed: for each sequence i and query head h,
//   out[i][h] = sum_j softmax_j(scale * q[i][h] . K_j) V_j,  j < context_lens[i],
// the attention of page "Nano-vLLM-Ascend" (section 2.2.1) with K_j / V_j read
// through the block table (section 2.1) and the softmax statistics kept in
// fp32 (page "vLLM-Ascend ...", section 3.1, problem 2).
//
// Work decomposition.  One workgroup (4 wavefronts) per (sequence, KV head,
// context partition).  All G = Hq/Hkv query heads that read the KV head are
// served by the same workgroup, so every K/V byte is fetched once per step.
//
// Loads.  A token's row for one KV head is head_dim * 2 bytes (256 B at
// D = 128) and each lane fetches 16 B of it, so LPR = D/8 lanes cover a row and
// one wavefront instruction covers RPW = 64/LPR consecutive token rows of one
// block.  Loads go through a raw buffer resource whose base is the block (a
// scalar value: the block id is uniform across the wavefront) and whose size
// ends at the partition's last valid row: rows past the context, blocks past
// the table and out-of-range block ids all read as zero without a memory
// access.  PF steps of K and V are kept in flight per lane.
//
// Softmax.  Each group of LPR lanes (a "row slot") runs its own online softmax
// over the tokens it sees (fp32 running max m and sum l, in the log2 domain so
// the exponential is a single v_exp_f32).  Scores are reduced across the LPR
// lanes with DPP row operations.  At the end the row slots of a wavefront are
// merged with cross-lane shuffles and the four wavefronts through LDS.
//
// Partitions.  With partition_size > 0 a long context is cut into partitions
// of that many tokens.  A partition writes its normalised output o_p and its
// (m_p, l_p); the merge kernel then forms
//   M = max_p m_p,  w_p = l_p 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
// Sequences that fit one partition write `out` directly.
#pragma once

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

constexpr int kDecodeWaves = 4;
constexpr float kEmptyMax = -1.0e30f;  // finite "no token yet" max: keeps 2^(m - m') finite

__device__ __forceinline__ int clamp_context(const DecodeArgs& a, int seq) {
  const int L = a.context_lens[seq];
  return L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
}

template <int DT, int D, int BS, int G, int PF>
__global__ __launch_bounds__(256) void decode_partition_kernel(const DecodeArgs a) {
  constexpr int LPR = D / 8;           // lanes per token row
  constexpr int RPW = 64 / LPR;        // token rows per wavefront load
  constexpr int NW = kDecodeWaves;
  constexpr int TPS = NW * RPW;        // tokens per workgroup step
  static_assert(BS % RPW == 0, "a wavefront's rows must lie in one block");

  __shared__ float s_acc[NW][G][D];
  __shared__ float s_ml[NW][G][2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR;
  const int c = lane % LPR;

  int wg = blockIdx.x;
  const int part = wg % a.num_parts;
  wg /= a.num_parts;
  const int kvh = wg % a.num_kv_heads;
  const int seq = wg / a.num_kv_heads;
  const int h0 = kvh * G;

  const int L = clamp_context(a, seq);
  const int t0 = part * a.part_tokens;
  if (L == 0) {
    if (part == 0) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + ((int64_t)seq * a.num_heads + h0) * D;
      for (int idx = threadIdx.x; idx < G * D; idx += 256) o[idx] = 0;
    }
    return;
  }
  if (t0 >= L) return;
  const int t1 = min(L, t0 + a.part_tokens);
  const int nparts_seq = 1 + (L - 1) / a.part_tokens;
  const int nblk = (L + BS - 1) / BS;

  const uint32_t row_stride = (uint32_t)a.num_kv_heads * D * 2;
  const uint64_t block_bytes = (uint64_t)BS * row_stride;
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)kvh * D * 2;
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)kvh * D * 2;
  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks;
  const uint32_t lane_off = (uint32_t)r * row_stride + (uint32_t)c * 16;

  uint32_t qv[G][4];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) +
                                                     ((int64_t)seq * a.num_heads + h0) * D) + c;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const u32x4 t = qp[g * (D / 8)];
      qv[g][0] = t.x; qv[g][1] = t.y; qv[g][2] = t.z; qv[g][3] = t.w;
    }
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kEmptyMax;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  // Scalar addressing of the block holding this wavefront's rows at step s.
  struct Where { uint64_t boff; uint32_t nrec; uint32_t voff; };
  auto where = [&](int s) -> Where {
    const int tb = t0 + s * TPS + wave * RPW;
    const int lb = tb / BS;
    const int nv = min(BS, t1 - lb * BS);
    int blk = bt[min(lb, nblk - 1)];
    const bool ok = nv > 0 && blk >= 0 && (int64_t)blk < a.num_blocks;
    Where w;
    w.nrec = ok ? (uint32_t)(nv - 1) * row_stride + D * 2 : 0u;
    w.boff = ok ? (uint64_t)blk * block_bytes : 0ull;
    w.voff = (uint32_t)(tb - lb * BS) * row_stride + lane_off;
    return w;
  };

  const int nsteps = (t1 - t0 + TPS - 1) / TPS;
  u32x4 kb[PF], vb[PF];
  Where wh[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    wh[u] = where(u);
    kb[u] = buffer_load16(make_rsrc(kbase + wh[u].boff, wh[u].nrec), wh[u].voff);
    vb[u] = buffer_load16(make_rsrc(vbase + wh[u].boff, wh[u].nrec), wh[u].voff);
  }

  for (int s0 = 0; s0 < nsteps; s0 += PF) {
    float sc[PF][G];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const bool valid = t0 + (s0 + u) * TPS + wave * RPW + r < t1;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = dot2<DT>(qv[g][0], kb[u].x, 0.f);
        d = dot2<DT>(qv[g][1], kb[u].y, d);
        d = dot2<DT>(qv[g][2], kb[u].z, d);
        d = dot2<DT>(qv[g][3], kb[u].w, d);
        d = group_sum<LPR>(d);
        sc[u][g] = valid ? d * a.scale_log2 : -__builtin_inff();
      }
    }
    // K registers are free: start the next group's K loads.
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      wh[u] = where(s0 + PF + u);
      kb[u] = buffer_load16(make_rsrc(kbase + wh[u].boff, wh[u].nrec), wh[u].voff);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < PF; ++u) mx = fmaxf(mx, sc[u][g]);
      const float alpha = fast_exp2(m[g] - mx);
      m[g] = mx;
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      float vf[8];
      vf[0] = lo_f32<DT>(vb[u].x); vf[1] = hi_f32<DT>(vb[u].x);
      vf[2] = lo_f32<DT>(vb[u].y); vf[3] = hi_f32<DT>(vb[u].y);
      vf[4] = lo_f32<DT>(vb[u].z); vf[5] = hi_f32<DT>(vb[u].z);
      vf[6] = lo_f32<DT>(vb[u].w); vf[7] = hi_f32<DT>(vb[u].w);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = fast_exp2(sc[u][g] - m[g]);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
      }
      vb[u] = buffer_load16(make_rsrc(vbase + wh[u].boff, wh[u].nrec), wh[u].voff);
    }
  }

  // Merge the row slots of this wavefront (lanes with equal c).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = m[g];
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float w = fast_exp2(m[g] - M);
    float ls = l[g] * w;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] *= w;
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      ls += __shfl_xor(ls, o);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] += __shfl_xor(acc[g][e], o);
    }
    m[g] = M;
    l[g] = ls;
  }
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][g][c * 8 + e] = acc[g][e];
      if (c == 0) {
        s_ml[wave][g][0] = m[g];
        s_ml[wave][g][1] = l[g];
      }
    }
  }
  __syncthreads();

  // Merge the wavefronts and write the partition (or final) result.
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = s_ml[0][g][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[w][g][0]);
    float den = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(s_ml[w][g][0] - M);
      den = fmaf(s_ml[w][g][1], f, den);
      o = fmaf(s_acc[w][g][d], f, o);
    }
    const float val = o / den;
    const int h = h0 + g;
    if (nparts_seq == 1) {
      static_cast<uint16_t*>(a.out)[((int64_t)seq * a.num_heads + h) * D + d] = to_u16<DT>(val);
    } else {
      const int64_t pidx = ((int64_t)seq * a.num_heads + h) * a.num_parts + part;
      a.part_out[pidx * D + d] = val;
      if (d == 0) {
        a.part_ml[pidx * 2] = M;
        a.part_ml[pidx * 2 + 1] = den;
      }
    }
  }
}

// One wavefront per (sequence, query head): merge that row's partitions.
template <int DT, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const DecodeArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const int h = blockIdx.x % a.num_heads;
  const int seq = blockIdx.x / a.num_heads;
  const int L = clamp_context(a, seq);
  const int n = L > 0 ? 1 + (L - 1) / a.part_tokens : 0;
  if (n <= 1) return;  // single-partition rows were written by the partition kernel
  const int64_t base = ((int64_t)seq * a.num_heads + h) * a.num_parts;
  const float* ml = a.part_ml + base * 2;
  float M = -__builtin_inff();
  for (int p = 0; p < n; ++p) M = fmaxf(M, ml[2 * p]);
  float den = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int p = 0; p < n; ++p) {
    const float w = ml[2 * p + 1] * fast_exp2(ml[2 * p] - M);
    den += w;
    const float* po = a.part_out + (base + p) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = fmaf(w, po[lane + 64 * e], o[e]);
  }
  uint16_t* out = static_cast<uint16_t*>(a.out) + ((int64_t)seq * a.num_heads + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) out[lane + 64 * e] = to_u16<DT>(o[e] / den);
}

template <int DT, int D, int BS, int G>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  constexpr int PF = (G <= 2) ? 8 : 4;
  const unsigned grid = (unsigned)((int64_t)a.num_seqs * a.num_kv_heads * a.num_parts);
  hipLaunchKernelGGL((decode_partition_kernel<DT, D, BS, G, PF>), dim3(grid), dim3(256), 0, s, a);
  if (a.num_parts > 1) {
    hipLaunchKernelGGL((decode_merge_kernel<DT, D>), dim3((unsigned)(a.num_seqs * a.num_heads)),
                       dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

template <int DT, int D, int BS>
hipError_t launch_decode_g(const DecodeArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_decode_t<DT, D, BS, 1>(a, s);
    case 2: return launch_decode_t<DT, D, BS, 2>(a, s);
    case 4: return launch_decode_t<DT, D, BS, 4>(a, s);
    case 8: return launch_decode_t<DT, D, BS, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t launch_decode_bs(const DecodeArgs& a, int block_size, int group, hipStream_t s) {
  switch (block_size) {
    case 16: return launch_decode_g<DT, D, 16>(a, group, s);
    case 32: return launch_decode_g<DT, D, 32>(a, group, s);
    case 256: return launch_decode_g<DT, D, 256>(a, group, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_decode_dt(const DecodeArgs& a, int head_dim, int block_size, int group,
                            hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_decode_bs<DT, 64>(a, block_size, group, s);
    case 128: return launch_decode_bs<DT, 128>(a, block_size, group, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
