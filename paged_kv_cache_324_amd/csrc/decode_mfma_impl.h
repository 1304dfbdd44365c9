// Paged-attention decode on matrix cores, for 2..16 query heads per KV head.
//
// Same computation, inputs, outputs and partition scheme as
// decode_partition_kernel (decode_impl.h): out[i][h] = softmax(scale q K^T) V
// over the paged context (page "Nano-vLLM-Ascend", sections 2.1 and 2.2.1),
// with fp32 softmax statistics (page "vLLM-Ascend ...", section 3.1, problem
// 2).  With G query heads per KV head the score and value products are small
// dense contractions ([G x 128] x [128 x keys] and back), so they run on MFMA
// instead of fp32 vector ALUs, which keeps GQA-8 decode bound by HBM rather
// than by VALU issue.
//
// One workgroup (NW wavefronts) per (sequence, KV head, context partition),
// or, for grids larger than the resident workgroups (PERSIST), a resident
// grid whose workgroups take several such items in turn.  The partition is
// cut into 32-key steps taken round-robin by the NW wavefronts:
//   S^T = K Q^T   16x16x32 MFMA, two 16-key groups per step.  A = K rows
//                 (16 keys x 32 dims).  K and V rows are loaded whole, four
//                 256-byte rows per load instruction, through buffer
//                 resources based at the group's block (16 keys never
//                 straddle a block) whose size ends at the last valid key;
//                 K goes through this wavefront's LDS K buffer, from which
//                 lane l reads key l % 16, dims 32 ks + 8 (l/16) ...  (Loading
//                 the A fragments straight from the cache made each load
//                 instruction span 16 rows 2 KB apart, eight 4 KB pages, and
//                 stalled the L1 address translation: 10% slower on Llama-2-
//                 shaped batches, 11% on split long contexts.)  B = Q^T, the G
//                 heads in columns 0..G-1.
//   softmax       lane l owns head l % 16 and 4 keys of each group; the max
//                 adds two lane exchanges (l ^ 16, l ^ 32).  Rescaling of O is
//                 lazy (only when a maximum grows by more than 2^8).
//   O^T += V^T P^T  16x16x16 MFMA over each group's 16 keys.  V rows are
//                 loaded into registers with K, stored to this wavefront's LDS
//                 V buffer and read back transposed (ds_read_b64_tr_b16); P^T is
//                 the softmax registers rounded to the input dtype.
//   row sum       one more 16x16x16 MFMA per group, ones P^T: the sum, in
//                 fp32, of exactly the rounded p the value product consumes,
//                 so numerator and denominator weigh every key alike.
// As soon as a step's K and V have left their registers (both in LDS) the
// same registers take the loads of the wavefront's next step, whose
// block ids were loaded a step earlier still; so one step per wavefront is
// always in flight.
// At the end the NW wavefronts' (m, l, O) are merged through LDS and the
// partition writes `out` (unsplit context) or its normalised partial for the
// merge kernel.
#pragma once

#include "decode_impl.h"
#include "mfma.h"

namespace pa {

constexpr int kMdRow = 256;                 // bytes of one key row (head_dim 128)
constexpr int kMdStepKeys = 32;             // keys per wavefront step
constexpr int kMdStep = kMdStepKeys * kMdRow;
constexpr float kMdLazyRescale = 8.0f;

// V rows of a step are stored with 16-byte chunk c of row r at c ^ ((2 r) & 15):
// the transposed reads (8 rows x chunks {2 dt, 2 dt + 1} per half wavefront)
// then touch 16 distinct bank groups.
__device__ __forceinline__ int md_vswz(int r) { return (2 * r) & 15; }
// K rows likewise with chunk c of row r at c ^ (r & 7): the score operands (16
// rows, one 16-byte chunk each per quarter wavefront) then read 8 distinct bank
// groups per 8 lanes.
__device__ __forceinline__ int md_kswz(int r) { return r & 7; }

// One work item: (partition, sequence rank, KV head) number `item` of the grid's
// order.
template <int DT, int BS, int G, int NW, bool ROPE>
__device__ __forceinline__ void decode_mfma_item(const DecodeArgs& a, const int item) {
  constexpr int D = 128;
  static_assert(G >= 1 && G <= 16, "heads of a group fill the 16 MFMA columns");
  static_assert(BS % 16 == 0, "a 16-key group lies in one block");
  // One V buffer per wavefront; at the end the same bytes hold that
  // wavefront's fp32 O^T (16 heads x 128 dims) for the merge.
  __shared__ __attribute__((aligned(16))) unsigned char s_v[NW][kMdStep];  // 8 KB per wavefront
  __shared__ __attribute__((aligned(16))) unsigned char s_k[NW][kMdStep];
  __shared__ float s_ml[NW * 16 * 2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;   // head (score / output column)
  const int quad = lane >> 4;  // which 4 keys / dims of a group this lane holds

  // Partition-major order (every sequence's first partition before any
  // second one); within a partition index, sequences in `seq_order` when one
  // is given.
  const int per_part = a.num_seqs * a.num_kv_heads;
  const int part = item / per_part;
  const int rest = item - part * per_part;
  const int rank = rest / a.num_kv_heads;
  const int kvh = rest - rank * a.num_kv_heads;
  const int seq = a.seq_order ? a.seq_order[rank] : rank;
  if (seq < 0 || seq >= a.num_seqs) return;
  const int h0 = kvh * G;
  const int t0 = part * a.part_tokens;  // a block boundary

  // Prologue loads are issued together: the block ids of this wavefront's
  // first two steps (speculatively, before the context length is known;
  // reads are clamped to the sequence's table row), the queries and the
  // length.
  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks;
  const int lbA = t0 / BS;
  // Lane l holds the block id of 16-key group (l & 1) of step s.
  auto load_ids = [&](int s) -> int32_t {
    return bt[min(lbA + (kMdStepKeys * s + 16 * (lane & 1)) / BS, a.max_blocks - 1)];
  };
  const int32_t ids_first = load_ids(wave);
  int32_t ids_next = load_ids(wave + NW);

  // Q^T fragments: column = head col, dims 32 ks + 8 quad .. + 7.  Columns
  // past G repeat head h0 (finite scores in columns of their own, never
  // written out), so no select has to wait for the loads.
  u32x4 qf[4];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)seq * a.num_heads + h0 + (col < G ? col : 0)) * D);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = qp[4 * ks + quad];
  }
  // Fused rotary step: fragment ks holds 16-byte chunk 4 ks + quad, so chunks
  // j and j + 8 (dims 8 j .. + 7 of the two halves) are fragments ks and ks + 2
  // of the same lane; table entries of pair index 8 (4 ks + quad), ks = 0, 1.
  // The table rows are read where they are used (for q, then for the new key),
  // so they hold no registers across the context loop.
  int64_t rope_pos = 0;
  bool rope_ok = false;
  if constexpr (ROPE) {
    rope_pos = a.positions[seq];
    rope_ok = rope_pos >= 0 && rope_pos < a.max_position;
  }
  auto rotate_frags = [&](u32x4 (&f)[4]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float rcs[8], rsn[8];
      rope_row8(a.rope_cos, rope_pos, D / 2, 8 * (4 * ks + quad), rcs);
      rope_row8(a.rope_sin, rope_pos, D / 2, 8 * (4 * ks + quad), rsn);
      const u32x4 x1 = f[ks], x2 = f[ks + 2];
      f[ks] = rope_half8<DT>(x1, x2, rcs, rsn, true);
      f[ks + 2] = rope_half8<DT>(x2, x1, rcs, rsn, false);
    }
  };

  const int L = clamp_context(a, seq);
  if (L == 0) {
    if (part == 0) write_empty_rows<D, G>(a, seq, h0);
    return;
  }
  if (t0 >= L) return;
  const int t1 = (int)min((int64_t)L, (int64_t)t0 + a.part_tokens);
  const int nparts_seq = 1 + (L - 1) / a.part_tokens;

  // Fused step: the partition holding position L-1 streams the cached tokens
  // before it, takes that position's K/V from key_new/value_new in a one-key
  // step of its own, and stores them bit for bit at the slot.
  const bool new_here = a.key_new != nullptr && t1 == L;
  const int t1c = new_here ? L - 1 : t1;  // end of the cached range
  const int64_t new_row = ((int64_t)seq * a.num_kv_heads + kvh) * D;
  if (new_here && wave == 0 && lane < 32) {
    const int64_t slot = a.slot_mapping[seq];
    if (lane == 0) report_index_error(a.index_errors, slot >= a.num_slots, kErrSlot, slot);
    if (slot >= 0 && slot < a.num_slots) {
      const void* src = lane < 16 ? a.key_new : a.value_new;
      void* dst = lane < 16 ? a.k_cache_w : a.v_cache_w;
      const u32x4* srow = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + new_row);
      u32x4 chunk = srow[col];
      if constexpr (ROPE) {
        if (lane < 16 && rope_ok) {  // the stored key is the rotated one
          float cs[8], sn[8];
          rope_row8(a.rope_cos, rope_pos, D / 2, 8 * (col & 7), cs);
          rope_row8(a.rope_sin, rope_pos, D / 2, 8 * (col & 7), sn);
          chunk = rope_half8<DT>(chunk, srow[col ^ 8], cs, sn, col < 8);
        }
      }
      reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + (slot * a.num_kv_heads + kvh) * D)[col] =
          chunk;
    }
  }

  if constexpr (ROPE) {
    if (rope_ok) rotate_frags(qf);
  }

  const int32_t nb32 = a.num_blocks > INT32_MAX ? INT32_MAX : (int32_t)a.num_blocks;
  const uint32_t row_bytes = (uint32_t)a.num_kv_heads * D * 2;
  const uint64_t block_bytes = (uint64_t)BS * row_bytes;
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)kvh * D * 2;
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)kvh * D * 2;

  float m = kEmptyMax;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{};
  // Row sums of the rounded P: every accumulator row holds its column's sum.
  f32x4 lacc = f32x4{};
  const uint32_t one2 = pack2<DT>(1.f, 1.f);
  const u32x2 ones = {one2, one2};
  unsigned char* const sv = s_v[wave];
  unsigned char* const sk = s_k[wave];
  u32x4 kf[2][4], kr[2][4], vr[2][4];

  // The K and V rows this lane will store (row 4 i + quad of each group,
  // chunk col ^ swizzle), for step s; `ids` holds the step's block ids.  Past
  // the cached range the resources have size 0: loads return zeros without
  // touching memory.
  auto issue = [&](int s, int32_t ids) {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      const int g0 = t0 + kMdStepKeys * s + 16 * gr;
      const int lb = g0 / BS;
      const int32_t blk = __builtin_amdgcn_readlane(ids, gr);
      const int nv = min(16, t1c - g0);
      const bool ok = nv > 0 && blk >= 0 && blk < nb32;
      report_index_error(a.index_errors, nv > 0 && !ok, kErrBlockId, blk);
      const uint64_t off = ok ? (uint64_t)(uint32_t)blk * block_bytes +
                                    (uint64_t)(g0 - lb * BS) * row_bytes
                              : 0ull;
      const uint32_t nrec = ok ? (uint32_t)(nv - 1) * row_bytes + D * 2 : 0u;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + off, nrec);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + off, nrec);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * i + quad;
        kr[gr][i] = buffer_load16<kCachePolicyNT>(
            rk, (uint32_t)rr * row_bytes + (uint32_t)((col ^ md_kswz(16 * gr + rr)) * 16));
        vr[gr][i] = buffer_load16<kCachePolicyNT>(
            rv, (uint32_t)rr * row_bytes + (uint32_t)((col ^ md_vswz(16 * gr + rr)) * 16));
      }
    }
  };

  auto store_v = [&]() {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(sv + (16 * gr + 4 * i + quad) * kMdRow + col * 16) = vr[gr][i];
  };
  auto store_k = [&]() {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(sk + (16 * gr + 4 * i + quad) * kMdRow + col * 16) = kr[gr][i];
  };
  // Score operands from the K rows in LDS: lane (key col, quad) takes chunk
  // 4 ks + quad of key 16 gr + col.
  auto load_kf = [&]() {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      const int r = 16 * gr + col;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kf[gr][ks] = *reinterpret_cast<const u32x4*>(
            sk + r * kMdRow + (((4 * ks + quad) ^ md_kswz(r)) * 16));
    }
  };

  auto scores = [&](f32x4 (&sc)[2]) {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      sc[gr] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[gr] = mfma16x16x32<DT>(kf[gr][ks], qf[ks], sc[gr]);
    }
  };

  // Softmax update and O^T += V^T P^T for the step at key kb, keys < kend.
  auto accumulate = [&](f32x4 (&sc)[2], int kb, int kend) {
    if (kb + kMdStepKeys > kend) {  // partial step: keys past the range score -inf
#pragma unroll
      for (int gr = 0; gr < 2; ++gr)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + 16 * gr + 4 * quad + i >= kend) sc[gr][i] = -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = max_xor32(max_xor16(mx)) * a.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m + kMdLazyRescale)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      lacc *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
    }
#pragma unroll
    for (int gr = 0; gr < 2; ++gr)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[gr][i] = fast_exp2(fmaf(sc[gr][i], a.scale_log2, -m));
    // O^T[d][head] += V^T[d][key] P^T[key][head], 16 dims x 16 keys per MFMA;
    // the row sum takes the same rounded P^T.
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      const u32x2 pf = {pack2<DT>(sc[gr][0], sc[gr][1]), pack2<DT>(sc[gr][2], sc[gr][3])};
      lacc = mfma16x16x16<DT>(ones, pf, lacc);
      const int rr = 16 * gr + 4 * quad + (col >> 2);
      const unsigned char* rowp = sv + rr * kMdRow + 8 * (col & 1);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int chunk = 2 * dt + ((col & 3) >> 1);
        const u32x2 vf = lds_read_tr16(rowp + ((chunk ^ md_vswz(rr)) * 16));
        o[dt] = mfma16x16x16<DT>(vf, pf, o[dt]);
      }
    }
  };

  // Merge the NW wavefronts' (m, l, O) and write the partition.
  auto merge = [&]() {
    float* s_o = reinterpret_cast<float*>(sv);  // this wavefront's [16][128]
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[col * D + 16 * dt + 4 * quad + i] = o[dt][i];
    if (quad == 0) {
      s_ml[(wave * 16 + col) * 2] = m;
      s_ml[(wave * 16 + col) * 2 + 1] = lacc[0];
    }
    __syncthreads();
    const float* s_all = reinterpret_cast<const float*>(&s_v[0][0]);  // [NW][16][128]
    // The partition's rows of the G heads are contiguous in part_out.
    const int64_t prow = ((int64_t)seq * a.num_parts + part) * a.num_heads + h0;
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) {
      const int g = idx / D;
      const int d = idx - g * D;
      float M = s_ml[g * 2];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[(w * 16 + g) * 2]);
      float den = 0.f, ov = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2(s_ml[(w * 16 + g) * 2] - M);
        den = fmaf(s_ml[(w * 16 + g) * 2 + 1], f, den);
        ov = fmaf(s_all[(w * 16 + g) * D + d], f, ov);
      }
      const float val = ov / den;
      if (nparts_seq == 1) {
        static_cast<uint16_t*>(a.out)[((int64_t)seq * a.num_heads + h0 + g) * D + d] = to_u16<DT>(val);
      } else {
        a.part_out[prow * D + idx] = to_u16<DT>(val);
      }
    }
    float2* mlp = row_ml_target(a, nparts_seq, seq, h0, prow);
    if (mlp && (int)threadIdx.x < G) {
      const int g = threadIdx.x;
      float M = s_ml[g * 2];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[(w * 16 + g) * 2]);
      float den = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w)
        den = fmaf(s_ml[(w * 16 + g) * 2 + 1], fast_exp2(s_ml[(w * 16 + g) * 2] - M), den);
      mlp[g] = make_float2(M, den);
    }
  };

  const int nsteps = (t1c - t0 + kMdStepKeys - 1) / kMdStepKeys;
  int s = wave;
  if (s < nsteps) {
    issue(s, ids_first);
    for (; s < nsteps; s += NW) {
      // The ids of step s + 2 NW go out before the K/V of step s + NW, so waiting
      // for ids never waits for K/V; loads past the partition are harmless
      // (clamped ids, size-0 resources), so every step sees the same loads in
      // flight.
      const int32_t ids_after = load_ids(s + 2 * NW);
      store_k();
      store_v();
      load_kf();
      f32x4 sc[2];
      scores(sc);
      issue(s + NW, ids_next);
      ids_next = ids_after;
      accumulate(sc, t0 + kMdStepKeys * s, t1c);
    }
  }
  if (new_here && wave == nsteps % NW) {
    // The new token, on the wavefront with the fewest steps: row 0 of a
    // step whose buffer resources span just its rows of key_new / value_new,
    // so every other row loads as zeros (and scores -inf).
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(static_cast<const uint16_t*>(a.key_new) + new_row, D * 2);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(static_cast<const uint16_t*>(a.value_new) + new_row, D * 2);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[0][ks] = buffer_load16<0>(rk, (uint32_t)col * row_bytes + (uint32_t)(4 * ks + quad) * 16);
      kf[1][ks] = u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (ROPE) {
      if (rope_ok) rotate_frags(kf[0]);  // rows other than 0 are zeros and stay zeros
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * i + quad;
      vr[0][i] = buffer_load16<0>(rv, (uint32_t)rr * row_bytes + (uint32_t)((col ^ md_vswz(rr)) * 16));
      vr[1][i] = u32x4{0u, 0u, 0u, 0u};
    }
    store_v();
    f32x4 sc[2];
    scores(sc);
    accumulate(sc, L - 1, L);
  }
  merge();
}

// One work item per workgroup, or (PERSIST) a grid of W workgroups each taking
// items b, 2W - 1 - b, 2W + b, 4W - 1 - b, ...: in the longest-first order that
// pairs long items with short ones, and saves a workgroup launch per item.
template <int DT, int BS, int G, int NW, bool ROPE, bool PERSIST>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_mfma_kernel(const DecodeArgs a) {
  if constexpr (!PERSIST) {
    decode_mfma_item<DT, BS, G, NW, ROPE>(a, (int)blockIdx.x);
  } else {
    const int n = a.num_seqs * a.num_kv_heads * a.num_parts;
    const int W = (int)gridDim.x;
    for (int k = 0;; ++k) {
      const int item = (k & 1) ? (k + 1) * W - 1 - (int)blockIdx.x : k * W + (int)blockIdx.x;
      if (item >= n) break;
      decode_mfma_item<DT, BS, G, NW, ROPE>(a, item);
      __syncthreads();  // the next item reuses the LDS buffers
    }
  }
}

}  // namespace pa
