// Paged-attention decode on matrix cores, for 4..16 query heads per KV head.
//
// Same computation, inputs, grid order and partition scheme as
// decode_partition_kernel (decode_impl.h): out[i][h] = softmax(scale q K^T) V
// over the paged context (page "Nano-vLLM-Ascend", sections 2.1 and 2.2.1),
// with fp32 softmax statistics (page "vLLM-Ascend ...", section 3.1, problem
// 2).  With G query heads per KV head the score and value products are small
// dense contractions ([G x 128] x [128 x keys] and back), so they run on MFMA
// instead of fp32 vector ALUs, which keeps GQA-8 decode bound by HBM rather
// than by VALU issue.
//
// One workgroup (4 wavefronts) per (sequence, KV head, context partition).
// The partition is cut into 32-key steps taken round-robin by the four
// wavefronts; each wavefront streams its own steps with no barrier:
//   S^T = K Q^T   16x16x32 MFMA, two 16-key groups per step.  A = K rows
//                 (16 keys x 32 dims), loaded straight from the cache into
//                 registers: lane l takes key l % 16, dims 32 ks + 8 (l/16) ..,
//                 through a buffer resource based at the group's block (16
//                 keys never straddle a block) whose size ends at the last
//                 valid key.  B = Q^T, the G heads in columns 0..G-1.
//   softmax       lane l owns head l % 16 and 4 keys of each group; max and
//                 sum add two lane exchanges (l ^ 16, l ^ 32).  Rescaling of
//                 O is lazy (only when a maximum grows by more than 2^8).
//   O^T += V^T P^T  16x16x16 MFMA over each group's 16 keys.  V rows are
//                 loaded into registers with K, stored to this wavefront's LDS
//                 buffer just before use and read back transposed
//                 (ds_read_b64_tr_b16); P^T is the softmax registers.
// K and V of the wavefront's next step are in flight while a step computes;
// block ids come from an LDS copy of the table, so no wait on the table ever
// drains the prefetch.
// At the end the four wavefronts' (m, l, O) are merged through LDS; a
// partition either writes `out` or its normalised partial for the merge kernel.
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

template <int DT, int BS, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_mfma_kernel(const DecodeArgs a) {
  constexpr int D = 128;
  static_assert(G >= 1 && G <= 16, "heads of a group fill the 16 MFMA columns");
  static_assert(BS % 16 == 0, "a 16-key group lies in one block");
  __shared__ __attribute__((aligned(16))) unsigned char s_v[4][kMdStep];  // 32 KB, one per wave
  __shared__ int32_t s_tbl[kTableCap];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;   // head (score / output column)
  const int quad = lane >> 4;  // which 4 keys / dims of a group this lane holds

  const int per_part = a.num_seqs * a.num_kv_heads;
  const int part = blockIdx.x / per_part;
  const int rest = blockIdx.x - part * per_part;
  const int rank = rest / a.num_kv_heads;
  const int kvh = rest - rank * a.num_kv_heads;
  const int seq = a.seq_order ? a.seq_order[rank] : rank;
  if (seq < 0 || seq >= a.num_seqs) return;
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

  // Q^T fragments: column = head col (zero past G), dims 32 ks + 8 quad .. + 7.
  u32x4 qf[4];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)seq * a.num_heads + h0 + (col < G ? col : 0)) * D);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 v = qp[4 * ks + quad];
      qf[ks] = col < G ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // Fused step: the partition holding position L-1 takes that position's
  // K/V from key_new/value_new (patched into the registers of the one step
  // that holds it) and stores them bit for bit at the sequence's slot.
  const bool new_here = a.key_new != nullptr && t1 == L;
  const int64_t new_row = ((int64_t)seq * a.num_kv_heads + kvh) * D;
  if (new_here && wave == 0 && lane < 32) {
    const int64_t slot = a.slot_mapping[seq];
    if (slot >= 0 && slot < a.num_slots) {
      const void* src = lane < 16 ? a.key_new : a.value_new;
      void* dst = lane < 16 ? a.k_cache_w : a.v_cache_w;
      reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + (slot * a.num_kv_heads + kvh) * D)[col] =
          reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + new_row)[col];
    }
  }

  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks;
  const int32_t nb32 = a.num_blocks > INT32_MAX ? INT32_MAX : (int32_t)a.num_blocks;
  const uint32_t row_bytes = (uint32_t)a.num_kv_heads * D * 2;
  const uint64_t block_bytes = (uint64_t)BS * row_bytes;
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)kvh * D * 2;
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)kvh * D * 2;

  float m = kEmptyMax, lsum = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{};
  unsigned char* const sv = s_v[wave];

  auto compute = [&](int kb, const u32x4 (&kf)[2][4], int kend) {
    f32x4 sc[2];
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      sc[gr] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[gr] = mfma16x16x32<DT>(kf[gr][ks], qf[ks], sc[gr]);
    }
    if (kb + kMdStepKeys > kend) {  // last, partial step: keys past the range score -inf
#pragma unroll
      for (int gr = 0; gr < 2; ++gr)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + 16 * gr + 4 * quad + i >= kend) sc[gr][i] = -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m + kMdLazyRescale)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int gr = 0; gr < 2; ++gr)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(fmaf(sc[gr][i], a.scale_log2, -m));
        sc[gr][i] = p;
        psum += p;
      }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    lsum += psum;
    // O^T[d][head] += V^T[d][key] P^T[key][head], 16 dims x 16 keys per MFMA.
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      const u32x2 pf = {pack2<DT>(sc[gr][0], sc[gr][1]), pack2<DT>(sc[gr][2], sc[gr][3])};
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

  // The partition is walked in chunks of at most kTableCap blocks whose ids
  // are staged in LDS; within a chunk wavefront w takes the 32-key steps
  // w, w + 4, ... and keeps the next one in flight while it computes.
  constexpr int kChunkTokens = kTableCap * BS;
  for (int c0 = t0; c0 < t1; c0 += kChunkTokens) {
    const int c1 = min(t1, c0 + kChunkTokens);
    const int lb0 = c0 / BS;
    const int nchunk_blk = (c1 - c0 + BS - 1) / BS;
    __syncthreads();  // previous chunk's table reads are done
    if ((int)threadIdx.x < nchunk_blk) {
      const int32_t blk = bt[lb0 + threadIdx.x];
      s_tbl[threadIdx.x] = (blk >= 0 && blk < nb32) ? blk : -1;
    }
    __syncthreads();

    // K fragments to registers (lane: key col, dims 32 ks + 8 quad ..) and the
    // V rows this lane will store (row 4 i + quad of each group, chunk col ^
    // swizzle), for the step at key kb.
    auto issue = [&](int kb, u32x4 (&kf)[2][4], u32x4 (&vr)[2][4]) {
#pragma unroll
      for (int gr = 0; gr < 2; ++gr) {
        const int g0 = kb + 16 * gr;
        const int lb = g0 / BS;
        const int32_t blk = __builtin_amdgcn_readfirstlane(s_tbl[min(lb - lb0, nchunk_blk - 1)]);
        const int nv = min(16, c1 - g0);
        const bool ok = nv > 0 && blk >= 0;
        const uint64_t off = ok ? (uint64_t)(uint32_t)blk * block_bytes +
                                      (uint64_t)(g0 - lb * BS) * row_bytes
                                : 0ull;
        const uint32_t nrec = ok ? (uint32_t)(nv - 1) * row_bytes + D * 2 : 0u;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + off, nrec);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + off, nrec);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kf[gr][ks] = buffer_load16<kCachePolicyNT>(
              rk, (uint32_t)col * row_bytes + (uint32_t)(4 * ks + quad) * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * i + quad;
          vr[gr][i] = buffer_load16<kCachePolicyNT>(
              rv, (uint32_t)rr * row_bytes + (uint32_t)((col ^ md_vswz(16 * gr + rr)) * 16));
        }
      }
    };
    auto store_v = [&](const u32x4 (&vr)[2][4]) {
#pragma unroll
      for (int gr = 0; gr < 2; ++gr)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(sv + (16 * gr + 4 * i + quad) * kMdRow + col * 16) = vr[gr][i];
    };

    // The look-ahead issue is unconditional: past the end its buffer
    // resources have size 0, so the loads return zeros without touching
    // memory, and every step sees the same count of loads in flight (a
    // conditional issue would make the compiler wait for all of them).
    auto patch_new = [&](int kb, u32x4 (&kf)[2][4], u32x4 (&vr)[2][4]) {
      const int r = L - 1 - kb;  // 0..31: the new token's row in this step
      const u32x4* kn = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.key_new) + new_row);
      const u32x4* vn = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.value_new) + new_row);
#pragma unroll
      for (int gr = 0; gr < 2; ++gr) {
        if ((r >> 4) != gr) continue;
        const int rr = r & 15;
        if (col == rr) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) kf[gr][ks] = kn[4 * ks + quad];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * i + quad == rr) vr[gr][i] = vn[col ^ md_vswz(16 * gr + rr)];
      }
    };
    auto holds_new = [&](int kb) { return new_here && L - 1 >= kb && L - 1 < kb + kMdStepKeys; };

    const int nsteps = (c1 - c0 + kMdStepKeys - 1) / kMdStepKeys;
    u32x4 kfa[2][4], kfb[2][4], vra[2][4], vrb[2][4];
    int s = wave;
    if (s < nsteps) issue(c0 + kMdStepKeys * s, kfa, vra);
    while (s < nsteps) {
      issue(c0 + kMdStepKeys * (s + 4), kfb, vrb);
      if (holds_new(c0 + kMdStepKeys * s)) patch_new(c0 + kMdStepKeys * s, kfa, vra);
      store_v(vra);
      compute(c0 + kMdStepKeys * s, kfa, c1);
      s += 4;
      if (s >= nsteps) break;
      issue(c0 + kMdStepKeys * (s + 4), kfa, vra);
      if (holds_new(c0 + kMdStepKeys * s)) patch_new(c0 + kMdStepKeys * s, kfb, vrb);
      store_v(vrb);
      compute(c0 + kMdStepKeys * s, kfb, c1);
      s += 4;
    }
  }

  // ---- merge the four wavefronts through LDS (reusing the V buffers)
  __syncthreads();
  float* s_o = reinterpret_cast<float*>(&s_v[0][0]);           // [4][16][128], 32 KB
  float* s_ml = reinterpret_cast<float*>(&s_tbl[0]);           // [4][16][2]
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[(wave * 16 + col) * D + 16 * dt + 4 * quad + i] = o[dt][i];
  if (quad == 0) {
    s_ml[(wave * 16 + col) * 2] = m;
    s_ml[(wave * 16 + col) * 2 + 1] = lsum;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = s_ml[g * 2];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_ml[(w * 16 + g) * 2]);
    float den = 0.f, ov = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = fast_exp2(s_ml[(w * 16 + g) * 2] - M);
      den = fmaf(s_ml[(w * 16 + g) * 2 + 1], f, den);
      ov = fmaf(s_o[(w * 16 + g) * D + d], f, ov);
    }
    const float val = ov / den;
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

}  // namespace pa
