// Paged-attention decode for gfx950: partition kernel + partition merge kernel.
//
// What is computed: for each sequence i and query head h,
//   out[i][h] = sum_j softmax_j(scale * q[i][h] . K_j) V_j,  j < context_lens[i],
// the attention of page "Nano-vLLM-Ascend" (section 2.2.1) with K_j / V_j read
// through the block table (section 2.1) and the softmax statistics kept in
// fp32 (page "vLLM-Ascend ...", section 3.1, problem 2).
//
// Work decomposition.  One workgroup (NW wavefronts, see DecodeShape) per
// (sequence, KV head, context partition).  All G = Hq/Hkv query heads that read the KV head are
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
// merged with cross-lane shuffles and the NW wavefronts through LDS.
//
// Partitions.  With partition_size > 0 a long context is cut into partitions
// of that many tokens.  A partition writes its normalised output o_p and its
// (m_p, l_p); the merge kernel then forms
//   M = max_p m_p,  w_p = l_p 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
// Sequences that fit one partition write `out` directly.
//
// Partial mode (out_ml set).  Every row also reports its (m, l), the merge
// writes the merged (M, sum_p w_p), and an empty context gives (-inf, 0), so
// the rows of several calls over disjoint key sets can be merged afterwards
// by the same rule (merge_partials.hip).
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

#ifndef PA_DECODE_AUX
#define PA_DECODE_AUX kCachePolicyNT
#endif

// Launch shape of decode_partition_kernel for G query heads per KV head.
// G <= 2 (G = 2 only at head_dim 64: at head_dim 128 the matrix-core kernel
// runs): eight wavefronts per workgroup and four steps of K and V in flight
// per lane, within 128 VGPRs, so that a SIMD holds four wavefronts and a
// compute unit two workgroups (on the Qwen3-shaped batch, when it ran here,
// this measured 3.5% faster than four wavefronts with eight steps each: the
// same bytes in flight per workgroup, and the same two-round longest-first
// dispatch).
// G = 4 or 8 (head_dim 64; at head_dim 128 the matrix-core kernel runs):
// four wavefronts, four steps, two wavefronts per SIMD.
// Wavefronts per decode_mfma_kernel workgroup: eight when a workgroup streams
// at least kMfmaLongSpan tokens (its partition, or the whole context when
// unsplit), four otherwise.  Eight halve the workgroups a compute unit holds
// (175 VGPRs: two wavefronts per SIMD) and double each one's loads in flight,
// which pays when spans are long and uneven (Llama-2-shaped batch, 4k-8k
// contexts unsplit: 310 -> 293 us) but not for short partitions, whose
// workgroups are dominated by their prologue and merge (512-token
// partitions: 165 -> 192 us; 2048: 174 -> 179 us; 4096: equal).
constexpr int kMfmaLongSpan = 4096;
// Two wavefronts when contexts are cut into partitions of at most this many
// tokens: each wavefront then takes more of its partition's few steps
// (context-parallel shard at partition 256: 31.5 -> 30.8 us; long split-K at
// 512: 165.6 -> 164.3 us).
constexpr int kMfmaShortPartition = 512;
// Persistent workgroups (decode_mfma_kernel's PERSIST): with eight wavefronts,
// when the work items outnumber the compute units; with two, when they number
// at least twice the resident workgroups.  Each workgroup then pairs long items
// with short ones and skips a launch per item (Llama-2-shaped batches 266 ->
// 260 / 265 -> 258 us, long split-K 150 -> 148 us).  With four wavefronts (the
// Qwen3-shaped batch) it measured 1% slower, and a grid that is not larger than
// the resident workgroups gains nothing from it: both keep one item per
// workgroup.

template <int G>
struct DecodeShape {
  static constexpr int waves = G <= 2 ? 8 : 4;
  static constexpr int pf = 4;
  static constexpr int waves_per_eu = G <= 2 ? 4 : 2;
};
constexpr int kTableCap = 256;  // block ids staged in LDS per chunk of a partition
constexpr float kEmptyMax = -1.0e30f;  // finite "no token yet" max: keeps 2^(m - m') finite

__device__ __forceinline__ int clamp_context(const DecodeArgs& a, int seq) {
  const int L = a.context_lens[seq];
  report_index_error(a.index_errors, L < 0 || L > a.max_context_len, kErrContextLen, L);
  return L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
}

// A sequence with no context: zero output rows for the G heads of a KV head
// (and, in partial mode, an empty (max, sum) = (-inf, 0)).
template <int D, int G>
__device__ __forceinline__ void write_empty_rows(const DecodeArgs& a, int seq, int h0) {
  const int64_t row0 = (int64_t)seq * a.num_heads + h0;
  uint16_t* o = static_cast<uint16_t*>(a.out) + row0 * D;
  for (int idx = threadIdx.x; idx < G * D; idx += (int)blockDim.x) o[idx] = 0;
  if (a.out_ml && (int)threadIdx.x < G)
    reinterpret_cast<float2*>(a.out_ml)[row0 + threadIdx.x] = make_float2(-__builtin_inff(), 0.f);
}

// Where a partition's (max, sum) go: the workspace when the sequence has
// several partitions, the caller's out_ml in partial mode when it has one,
// nowhere otherwise.
__device__ __forceinline__ float2* row_ml_target(const DecodeArgs& a, int nparts_seq, int seq,
                                                 int h0, int64_t prow) {
  if (nparts_seq > 1) return reinterpret_cast<float2*>(a.part_ml) + prow;
  if (a.out_ml) return reinterpret_cast<float2*>(a.out_ml) + (int64_t)seq * a.num_heads + h0;
  return nullptr;
}

template <int DT, int D, int BS, int G, int NW, int PF, int WAVES_PER_EU, int LOAD_AUX, bool ROPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WAVES_PER_EU, 8)))
void decode_partition_kernel(const DecodeArgs a) {
  constexpr int LPR = D / 8;           // lanes per token row
  constexpr int RPW = 64 / LPR;        // token rows per wavefront load
  constexpr int TPS = NW * RPW;        // tokens per workgroup step
  static_assert(BS % RPW == 0, "a wavefront's rows must lie in one block");
  static_assert(PF >= 1 && PF <= 64, "lane u of a wavefront addresses step u of a group");

  __shared__ float s_acc[NW][G][D];
  __shared__ float s_ml[NW][G][2];
  __shared__ int32_t s_tbl[kTableCap];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR;
  const int c = lane % LPR;

  // Partition-major order: every sequence's first partition is dispatched
  // before any second partition, so long contexts start early and the
  // workgroups of partitions past a short context (which exit at once) come
  // last.
  // Within a partition index, sequences are visited in `seq_order` when one
  // is given (longest first lets the dispatcher balance the CUs like
  // longest-processing-time list scheduling).
  const int per_part = a.num_seqs * a.num_kv_heads;
  const int part = blockIdx.x / per_part;
  const int rest = blockIdx.x - part * per_part;
  const int rank = rest / a.num_kv_heads;
  const int kvh = rest - rank * a.num_kv_heads;
  const int seq = a.seq_order ? a.seq_order[rank] : rank;
  if (seq < 0 || seq >= a.num_seqs) return;  // not a permutation entry: nothing to do
  const int h0 = kvh * G;

  // Issue the independent loads of the prologue together: the context
  // length (scalar), this workgroup's queries, and the block ids of the first
  // chunk (speculatively, before the length is known; every id read lies in
  // the sequence's table row).
  const int t0 = part * a.part_tokens;
  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks;
  const int lb_first = t0 / BS;
  const int32_t tbl_first =
      lb_first + (int)threadIdx.x < a.max_blocks ? bt[lb_first + threadIdx.x] : -1;
  // Rotary tables of the step's position (fused rotary step): lane c of a row
  // slot rotates dims 8 (c % (LPR/2)) .. + 7 of its half with the same dims of
  // the other half, held by lane c ^ (LPR/2).
  float rcs[8], rsn[8];
  bool rope_ok = false;
  if constexpr (ROPE) {
    const int64_t pos = a.positions[seq];
    rope_ok = pos >= 0 && pos < a.max_position;
    const int cr = (threadIdx.x & 63) % LPR;
    rope_row8(a.rope_cos, rope_ok ? pos : 0, D / 2, 8 * (cr % (LPR / 2)), rcs);
    rope_row8(a.rope_sin, rope_ok ? pos : 0, D / 2, 8 * (cr % (LPR / 2)), rsn);
  }
  uint32_t qv[G][4];
  {
    const int c = (threadIdx.x & 63) % LPR;
    const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) +
                                                     ((int64_t)seq * a.num_heads + h0) * D) + c;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const u32x4 t = qp[g * (D / 8)];
      qv[g][0] = t.x; qv[g][1] = t.y; qv[g][2] = t.z; qv[g][3] = t.w;
    }
  }
  const int L = clamp_context(a, seq);
  if (L == 0) {
    if (part == 0) write_empty_rows<D, G>(a, seq, h0);
    return;
  }
  if (t0 >= L) return;
  const int t1 = min(L, t0 + a.part_tokens);
  const int nparts_seq = 1 + (L - 1) / a.part_tokens;
  // Fused step: the partition holding position L-1 reads only the cached
  // tokens before it and takes the new token's rows from key_new/value_new
  // (fetched now, used after the cached tokens).
  const bool new_here = a.key_new != nullptr && t1 == L;
  const int t1c = new_here ? L - 1 : t1;
  u32x4 k_new = {0u, 0u, 0u, 0u}, v_new = {0u, 0u, 0u, 0u};
  if (new_here && wave == 0 && r == 0) {
    const int64_t row = ((int64_t)seq * a.num_kv_heads + kvh) * D;
    k_new = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.key_new) + row)[c];
    v_new = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.value_new) + row)[c];
  }
  if constexpr (ROPE) {
    if (new_here && wave == 0) {  // rotate the new key (row slot 0 holds it)
      const u32x4 partner = {(uint32_t)__shfl_xor((int)k_new.x, LPR / 2),
                             (uint32_t)__shfl_xor((int)k_new.y, LPR / 2),
                             (uint32_t)__shfl_xor((int)k_new.z, LPR / 2),
                             (uint32_t)__shfl_xor((int)k_new.w, LPR / 2)};
      if (rope_ok && r == 0) k_new = rope_half8<DT>(k_new, partner, rcs, rsn, c < LPR / 2);
    }
  }

  if constexpr (ROPE) {  // rotate the queries (used from the first step on)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const u32x4 own = {qv[g][0], qv[g][1], qv[g][2], qv[g][3]};
      const u32x4 partner = {(uint32_t)__shfl_xor((int)own.x, LPR / 2),
                             (uint32_t)__shfl_xor((int)own.y, LPR / 2),
                             (uint32_t)__shfl_xor((int)own.z, LPR / 2),
                             (uint32_t)__shfl_xor((int)own.w, LPR / 2)};
      if (rope_ok) {
        const u32x4 y = rope_half8<DT>(own, partner, rcs, rsn, c < LPR / 2);
        qv[g][0] = y.x; qv[g][1] = y.y; qv[g][2] = y.z; qv[g][3] = y.w;
      }
    }
  }

  const uint32_t row_stride = (uint32_t)a.num_kv_heads * D * 2;
  const uint64_t block_bytes = (uint64_t)BS * row_stride;
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)kvh * D * 2;
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)kvh * D * 2;
  const uint32_t lane_off = (uint32_t)r * row_stride + (uint32_t)c * 16;  // within a step

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kEmptyMax;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  // The partition is walked in chunks of at most kTableCap blocks whose ids are
  // first staged in LDS; each step then reads its block id with one uniform
  // LDS read instead of a dependent scalar load.
  const int32_t nb32 = a.num_blocks > INT32_MAX ? INT32_MAX : (int32_t)a.num_blocks;
  constexpr int kChunkTokens = kTableCap * BS;
  for (int c0 = t0; c0 < t1c; c0 += kChunkTokens) {
    const int c1 = min(t1c, c0 + kChunkTokens);
    const int lb0 = c0 / BS;
    const int nchunk_blk = (c1 - c0 + BS - 1) / BS;
    static_assert(kTableCap <= 64 * NW, "one table entry per thread");
    __syncthreads();  // previous chunk's table reads are done
    if ((int)threadIdx.x < nchunk_blk) {
      const int32_t blk = c0 == t0 ? tbl_first : bt[lb0 + threadIdx.x];
      report_index_error(a.index_errors, blk < 0 || blk >= nb32, kErrBlockId, blk);
      s_tbl[threadIdx.x] = (blk >= 0 && blk < nb32) ? blk : -1;
    }
    __syncthreads();

    // Addressing of a group of PF steps: lane u (mod PF) works out step
    // sbase + u -- the block holding the wavefront's rows, the byte offset of
    // its first row, and how many bytes from there are valid -- with one LDS
    // read for the whole group.  Each step then takes its values with
    // v_readlane into scalar registers (all operands non-negative; BS and TPS
    // are powers of two).
    const uint32_t wave_t0 = (uint32_t)c0 + (uint32_t)wave * RPW;
    struct Group { uint32_t lo, hi, nrec; };
    auto group_where = [&](int sbase) -> Group {
      const uint32_t tb = wave_t0 + (uint32_t)(sbase + lane % PF) * TPS;
      const uint32_t lb = tb / BS;
      const uint32_t o = tb % BS;                        // first row inside the block
      const int nvr = min(BS, c1 - (int)(lb * BS)) - (int)o;  // valid rows from there
      const int32_t blk = s_tbl[min((int)lb - lb0, nchunk_blk - 1)];
      const bool ok = nvr > 0 && blk >= 0;
      const uint64_t off = ok ? (uint64_t)(uint32_t)blk * block_bytes + o * row_stride : 0ull;
      Group g;
      g.lo = (uint32_t)off;
      g.hi = (uint32_t)(off >> 32);
      g.nrec = ok ? (uint32_t)(nvr - 1) * row_stride + D * 2 : 0u;
      return g;
    };
    auto load = [&](const char* base, const Group& g, int u) -> u32x4 {
      const uint64_t off = ((uint64_t)__builtin_amdgcn_readlane(g.hi, u) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane(g.lo, u);
      const uint32_t nrec = __builtin_amdgcn_readlane(g.nrec, u);
      return buffer_load16<LOAD_AUX>(make_rsrc(base + off, nrec), lane_off);
    };

    // Loads are issued K first, then V, in every group, so that the wait for
    // a group's K leaves its V loads in flight, and the wait for each V leaves
    // the next group's K loads in flight.
    const int nsteps = (c1 - c0 + TPS - 1) / TPS;
    u32x4 kb[PF], vb[PF];
    Group gcur = group_where(0);
#pragma unroll
    for (int u = 0; u < PF; ++u) kb[u] = load(kbase, gcur, u);
#pragma unroll
    for (int u = 0; u < PF; ++u) vb[u] = load(vbase, gcur, u);
    Group gnext = group_where(PF);

    for (int s0 = 0; s0 < nsteps; s0 += PF) {
      float sc[PF][G];
      const bool full = c0 + (s0 + PF) * TPS <= c1;  // no masked row in this group
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const bool valid = full || (c0 + (s0 + u) * TPS + wave * RPW + r < c1);
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
      // K registers are free: start the next group's K loads here, before the
      // softmax and PV work (the scheduler may not sink them past it).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < PF; ++u) kb[u] = load(kbase, gnext, u);
      __builtin_amdgcn_sched_barrier(0);
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
        vb[u] = load(vbase, gnext, u);
      }
      gnext = group_where(s0 + 2 * PF);  // its LDS read overlaps the next group's scores
    }
  }

  if (new_here && wave == 0) {
    // Row slot 0 of wavefront 0 takes the new token; in the other row slots
    // the score is -inf, which leaves their state unchanged.
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = dot2<DT>(qv[g][0], k_new.x, 0.f);
      d = dot2<DT>(qv[g][1], k_new.y, d);
      d = dot2<DT>(qv[g][2], k_new.z, d);
      d = dot2<DT>(qv[g][3], k_new.w, d);
      d = group_sum<LPR>(d);
      const float sc = r == 0 ? d * a.scale_log2 : -__builtin_inff();
      const float mx = fmaxf(m[g], sc);
      const float alpha = fast_exp2(m[g] - mx), p = fast_exp2(sc - mx);
      m[g] = mx;
      l[g] = fmaf(l[g], alpha, p);
      acc[g][0] = fmaf(acc[g][0], alpha, p * lo_f32<DT>(v_new.x));
      acc[g][1] = fmaf(acc[g][1], alpha, p * hi_f32<DT>(v_new.x));
      acc[g][2] = fmaf(acc[g][2], alpha, p * lo_f32<DT>(v_new.y));
      acc[g][3] = fmaf(acc[g][3], alpha, p * hi_f32<DT>(v_new.y));
      acc[g][4] = fmaf(acc[g][4], alpha, p * lo_f32<DT>(v_new.z));
      acc[g][5] = fmaf(acc[g][5], alpha, p * hi_f32<DT>(v_new.z));
      acc[g][6] = fmaf(acc[g][6], alpha, p * lo_f32<DT>(v_new.w));
      acc[g][7] = fmaf(acc[g][7], alpha, p * hi_f32<DT>(v_new.w));
    }
    const int64_t slot = a.slot_mapping[seq];
    if (lane == 0) report_index_error(a.index_errors, slot >= a.num_slots, kErrSlot, slot);
    if (r == 0 && slot >= 0 && slot < a.num_slots) {
      const int64_t dst = (slot * a.num_kv_heads + kvh) * D;
      reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.k_cache_w) + dst)[c] = k_new;
      reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.v_cache_w) + dst)[c] = v_new;
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

  // Merge the wavefronts and write the partition (or final) result.  A
  // partition's rows of the G heads are contiguous in part_out.
  const int64_t prow = ((int64_t)seq * a.num_parts + part) * a.num_heads + h0;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) {
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
    if (nparts_seq == 1) {
      static_cast<uint16_t*>(a.out)[((int64_t)seq * a.num_heads + h0 + g) * D + d] = to_u16<DT>(val);
    } else {
      a.part_out[prow * D + idx] = to_u16<DT>(val);
    }
  }
  float2* mlp = row_ml_target(a, nparts_seq, seq, h0, prow);
  if (mlp && (int)threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = s_ml[0][g][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[w][g][0]);
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) den = fmaf(s_ml[w][g][1], fast_exp2(s_ml[w][g][0] - M), den);
    mlp[g] = make_float2(M, den);
  }
}

// One wavefront per (sequence, query head): merge that row's partitions.
// Rows are visited through `seq_order` like the partition kernel's workgroups,
// so a sequence the order leaves out is neither read nor written.
// Lane p folds the (m, l) of partitions p, p+64, ...; each lane owns D/64
// consecutive dimensions of the partial outputs.  The outputs of the first 64
// partitions and all (m, l) are loaded before the context length is known;
// entries of partitions past the context are never used.
template <int DT, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const DecodeArgs a) {
  constexpr int E = D / 64;
  constexpr int PA = 64;
  typedef float floatE __attribute__((ext_vector_type(E)));
  // A lane's E partial-output elements (cache dtype) as one raw word.
  typedef typename std::conditional<E == 2, uint32_t, uint16_t>::type RawE;
  auto widen = [](RawE r) -> floatE {
    floatE f;
    f[0] = lo_f32<DT>((uint32_t)r);
    if constexpr (E == 2) f[1] = hi_f32<DT>((uint32_t)r);
    return f;
  };
  const int lane = threadIdx.x;
  const int h = blockIdx.x % a.num_heads;
  const int rank = blockIdx.x / a.num_heads;
  const int seq = a.seq_order ? a.seq_order[rank] : rank;
  if (seq < 0 || seq >= a.num_seqs) return;
  const int P = a.num_parts;
  // Partition p of this row is entry (seq * P + p) * num_heads + h.
  const int64_t base = (int64_t)seq * P * a.num_heads + h;
  const int64_t pstride = a.num_heads;
  const RawE* po = reinterpret_cast<const RawE*>(a.part_out + base * D + lane * E);
  const int64_t rstride = pstride * (D / E);  // RawE words between partitions
  const float2* pml = reinterpret_cast<const float2*>(a.part_ml) + base;
  // The first PA partitions' outputs are all requested at once (indices
  // clamped to the last partition of the grid, always inside the workspace),
  // so up to PA partitions cost one memory round trip.
  RawE pv[PA];
#pragma unroll
  for (int j = 0; j < PA; ++j) pv[j] = po[min(j, P - 1) * rstride];
  const float2 ml_own = lane < P ? pml[lane * pstride] : make_float2(0.f, 0.f);
  const float m_own = ml_own.x, l_own = ml_own.y;

  const int L = clamp_context(a, seq);
  const int n = L > 0 ? 1 + (L - 1) / a.part_tokens : 0;
  if (n <= 1) return;  // single-partition rows were written by the partition kernel

  float mp = -__builtin_inff(), lp = 0.f;
  if (lane < n) { mp = m_own; lp = l_own; }
  for (int p = lane + 64; p < n; p += 64) {  // only with more than 64 partitions
    const float2 ml2 = pml[p * pstride];
    const float m2 = ml2.x, l2 = ml2.y;
    const float mn = fmaxf(mp, m2);           // finite: partition p holds a token
    lp = lp * fast_exp2(mp - mn) + l2 * fast_exp2(m2 - mn);
    mp = mn;
  }
  float M = mp;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float w_own = lane < n ? lp * fast_exp2(mp - M) : 0.f;  // lane p's weight if n <= 64
  float den = w_own;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);

  floatE acc = {};
#pragma unroll
  for (int j = 0; j < PA; ++j) {
    if (j < n) {
      float w;
      if (n <= 64) {
        w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_own), j));
      } else {
        const float2 mlp = pml[j * pstride];
        w = mlp.y * fast_exp2(mlp.x - M);
      }
      acc += w * widen(pv[j]);
    }
  }
  for (int p = PA; p < n; ++p) {  // only with more than PA partitions
    const float2 mlp = pml[p * pstride];
    acc += (mlp.y * fast_exp2(mlp.x - M)) * widen(po[p * rstride]);
  }
  uint16_t* out = static_cast<uint16_t*>(a.out) + ((int64_t)seq * a.num_heads + h) * D + lane * E;
  const float inv = 1.0f / den;
#pragma unroll
  for (int e = 0; e < E; ++e) out[e] = to_u16<DT>(acc[e] * inv);
  if (a.out_ml && lane == 0)
    reinterpret_cast<float2*>(a.out_ml)[(int64_t)seq * a.num_heads + h] = make_float2(M, den);
}

template <int DT, int BS, int G, int NW, bool ROPE, bool PERSIST>
__global__ void decode_mfma_kernel(const DecodeArgs a);

// Matrix cores take the score/value products once a KV head serves 2 or more
// query heads (head_dim 128): the matrix-core kernel's whole-row loads then
// stream faster than the vector kernel even with 14 of its 16 MFMA columns
// idle (Qwen3-shaped batch, G = 2: 98.6 -> 95.5 us per step).  With one query
// head per KV head the vector kernel keeps it (6.4 TB/s on uniform contexts).
template <int D, int G>
constexpr bool decode_uses_mfma() {
  return D == 128 && G >= 2;
}

template <int DT, int D, int BS, int G, bool ROPE>
void launch_partitions(const DecodeArgs& a, unsigned grid, hipStream_t s) {
  using Shape = DecodeShape<G>;
  if constexpr (decode_uses_mfma<D, G>()) {
    // Workgroups resident at once: two wavefronts per SIMD, four SIMDs per unit.
    const unsigned cus = a.num_cus > 0 ? (unsigned)a.num_cus : 256u;
    if (a.part_tokens >= kMfmaLongSpan) {
      if (grid > cus)
        launch((decode_mfma_kernel<DT, BS, G, 8, ROPE, true>), dim3(cus), dim3(512), 0, s, a);
      else
        launch((decode_mfma_kernel<DT, BS, G, 8, ROPE, false>), dim3(grid), dim3(512), 0, s, a);
    } else if (a.num_parts > 1 && a.part_tokens <= kMfmaShortPartition) {
      if (grid >= 8 * cus)
        launch((decode_mfma_kernel<DT, BS, G, 2, ROPE, true>), dim3(4 * cus), dim3(128), 0, s, a);
      else
        launch((decode_mfma_kernel<DT, BS, G, 2, ROPE, false>), dim3(grid), dim3(128), 0, s, a);
    } else {
      launch((decode_mfma_kernel<DT, BS, G, 4, ROPE, false>), dim3(grid), dim3(256), 0, s, a);
    }
  } else {
    launch((decode_partition_kernel<DT, D, BS, G, Shape::waves, Shape::pf, Shape::waves_per_eu,
                                    PA_DECODE_AUX, ROPE>),
           dim3(grid), dim3(64 * Shape::waves), 0, s, a);
  }
}

// The partition merge (a6) of a split decode, when some context spans several
// partitions.
template <int DT, int D>
void launch_merge(const DecodeArgs& a, hipStream_t s) {
  if (a.num_parts > 1) {
    launch((decode_merge_kernel<DT, D>), dim3((unsigned)(a.num_seqs * a.num_heads)), dim3(64),
           0, s, a);
  }
}

template <int DT, int D, int BS, int G>
hipError_t launch_decode_t(const DecodeArgs& a, int phases, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.num_seqs * a.num_kv_heads * a.num_parts);
  if (phases & kPhasePartitions) {
    if (a.rope_cos) {
      launch_partitions<DT, D, BS, G, true>(a, grid, s);
    } else {
      launch_partitions<DT, D, BS, G, false>(a, grid, s);
    }
  }
  if (phases & kPhaseMerge) launch_merge<DT, D>(a, s);
  return hipGetLastError();
}

template <int DT, int D, int BS>
hipError_t launch_decode_g(const DecodeArgs& a, int group, int phases, hipStream_t s) {
  switch (group) {
    case 1: return launch_decode_t<DT, D, BS, 1>(a, phases, s);
    case 2: return launch_decode_t<DT, D, BS, 2>(a, phases, s);
    case 4: return launch_decode_t<DT, D, BS, 4>(a, phases, s);
    case 8: return launch_decode_t<DT, D, BS, 8>(a, phases, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t launch_decode_bs(const DecodeArgs& a, int block_size, int group, int phases,
                            hipStream_t s) {
  if (phases == kPhaseMerge) {  // the merge alone does not depend on the cache's shape
    launch_merge<DT, D>(a, s);
    return hipGetLastError();
  }
  switch (block_size) {
    case 16: return launch_decode_g<DT, D, 16>(a, group, phases, s);
    case 32: return launch_decode_g<DT, D, 32>(a, group, phases, s);
    case 256: return launch_decode_g<DT, D, 256>(a, group, phases, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_decode_dt(const DecodeArgs& a, int head_dim, int block_size, int group,
                            int phases, hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_decode_bs<DT, 64>(a, block_size, group, phases, s);
    case 128: return launch_decode_bs<DT, 128>(a, block_size, group, phases, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
