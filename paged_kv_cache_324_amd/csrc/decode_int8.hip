// Paged-attention decode over an INT8 KV cache (head_dim 64 and 128).
//
// Same computation as the 16-bit decode kernels, over the dequantised cache:
// out[i][h] = softmax(scale q K'^T) V' with K'[j] = code_K[j] * sK[j] and
// V'[j] = code_V[j] * sV[j] per token j and KV head (page "Nano-vLLM-Ascend",
// sections 2.1 and 2.2.1; fp32 softmax statistics, page "vLLM-Ascend ...",
// section 3.1, problem 2; INT8 as the next KV-cache compression, page
// "Nano-vLLM-Ascend", section 4.3, and page "vLLM-Ascend ...", section 5).
// Caches, head-major within a block: codes int8 [num_blocks][num_kv_heads]
// [block_size][128], scales float32 [num_blocks][num_kv_heads][block_size]
// (pa_reshape_and_cache_int8): a 16-key group of one head is one contiguous
// 16 D-byte run (the token-major 16-bit layout would leave 16 runs of D bytes).
//
// The structure is that of decode_mfma_kernel (decode_mfma_impl.h): one
// workgroup of 2, 4 or 8 wavefronts per (sequence, KV head, partition), 32-key steps
// taken round-robin, scores S^T = K Q^T on 16x16x32 MFMA and O^T += V^T P^T on
// 16x16x16 MFMA from a transposed LDS tile, a merge of the wavefronts through
// LDS.  What differs:
//   * a key row is D bytes.  Key rows are loaded whole, like value rows
//     (1024 / D rows per load instruction), and staged in the wavefront's LDS
//     K tile as codes; lane (key col, quad) reads back the D / 4 codes of dims
//     (D / 4) quad .. + D / 4 - 1 and MFMA step ks (of D / 32) takes dims
//     (D / 4) quad + 8 ks .. + 7; the query fragments follow the same dim
//     order (a dot product does not depend on the order of its terms).
//     (Loading those operand slices straight from the cache, 16 rows a quarter
//     of a line each per instruction, streamed 14% slower: 4.9 TB/s with no
//     arithmetic at all on the Qwen3-shaped batch);
//   * key codes are exact in fp16 and bf16 (|code| <= 127), so each is
//     converted in registers to the query's 16-bit type and the key scale
//     multiplies the fp32 score;
//   * V rows arrive as 16-byte chunks of 16 codes and are written to LDS as
//     two 16-byte chunks of 16-bit values, in the swizzled layout the
//     transposed reads expect: each value dequantised, code x scale rounded to
//     fp32 and then once to the query's 16-bit type (the operand type of the
//     value product);
//   * p is rounded to the 16-bit type for the value product, and the row sum
//     is a ones MFMA over the same rounded p (as in the 16-bit matrix-core
//     kernel), so numerator and denominator weigh every key alike;
//   * a step carries half the bytes, so each wavefront keeps two steps in
//     flight (two register sets) instead of one.
#include "decode_impl.h"
#include "mfma.h"

namespace pa {

constexpr int kI8StepKeys = 32;
constexpr float kI8LazyRescale = 8.0f;

// Swizzle of the 16-byte chunks of a converted V row in LDS (2 D bytes, D / 8
// chunks): chunk c of row r is stored at c ^ i8_vswz<D>(r), so that the
// transposed reads (4 consecutive rows x 2 adjacent chunks per 16 lanes) touch
// 16 distinct bank groups: with 256-byte rows each row spans the 64 banks and
// (2 r) & 15 gives 4 consecutive rows disjoint chunk pairs; with 128-byte rows
// two rows span the banks and ((r >> 1) ^ (r & 2)) & 7 gives rows r0 and r0 + 2
// (r0 % 4 = 0) disjoint pairs.
template <int D>
__device__ __forceinline__ int i8_vswz(int r) {
  if constexpr (D == 128) {
    return (2 * r) & 15;
  } else {
    return ((r >> 1) ^ (r & 2)) & 7;
  }
}

// Swizzle of the 16-byte chunks of a K code row in LDS (D bytes, D / 16
// chunks): chunk c of row r is stored at c ^ i8_kswz<D>(r), so that the score
// operand reads (16 rows, one chunk each per 16 lanes) touch 16 distinct bank
// groups: a 128-byte row puts rows r and r + 2 in the same half of the banks,
// a 64-byte row rows r and r + 4 in the same quarter.
template <int D>
__device__ __forceinline__ int i8_kswz(int r) {
  if constexpr (D == 128) {
    return (r ^ (r >> 3)) & 7;
  } else {
    return (r >> 2) & 3;
  }
}

// Codes b[2k], b[2k+1] of a dword (signed bytes) as a packed 16-bit pair, exactly.
template <int DT>
__device__ __forceinline__ uint32_t i8_pair(uint32_t w, int k) {
  const float lo = (float)(int8_t)(w >> (16 * k));
  const float hi = (float)(int8_t)(w >> (16 * k + 8));
  return pack2<DT>(lo, hi);
}

template <int DT>
__device__ __forceinline__ u32x4 i8_to_16(uint32_t w0, uint32_t w1) {
  return u32x4{i8_pair<DT>(w0, 0), i8_pair<DT>(w0, 1), i8_pair<DT>(w1, 0), i8_pair<DT>(w1, 1)};
}

// The four codes of a dword dequantised with row scale s, as two packed 16-bit
// pairs: code x s rounded once to fp32, then to the 16-bit type (nearest
// even).  Each code is read as the unsigned byte code + 128 of w ^ 0x80808080
// (one byte-to-float conversion) and the product formed as
// fma(code + 128, s, nb) with nb = -128 s (exact), which equals code x s up to
// that single rounding.
template <int DT>
__device__ __forceinline__ u32x2 i8x4_dequant(uint32_t w, float s, float nb) {
  const uint32_t u = w ^ 0x80808080u;
  const float f0 = fmaf((float)(u & 0xFFu), s, nb);
  const float f1 = fmaf((float)((u >> 8) & 0xFFu), s, nb);
  const float f2 = fmaf((float)((u >> 16) & 0xFFu), s, nb);
  const float f3 = fmaf((float)(u >> 24), s, nb);
  return u32x2{pack2<DT>(f0, f1), pack2<DT>(f2, f3)};
}

template <int DT, int D, int BS, int G, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_int8_kernel(const DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static_assert(G >= 1 && G <= 16, "heads of a group fill the 16 MFMA columns");
  static_assert(BS % 16 == 0, "a 16-key group lies in one block");
  constexpr int ROW = 2 * D;           // bytes of a converted (16-bit) V row in LDS
  constexpr int KS = D / 32;           // 16x16x32 score steps per key
  constexpr int KC = D / 64;           // 16-byte code chunks a lane loads per key
  constexpr int LPRV = D / 16;         // lanes per V code row (16 codes each)
  constexpr int RPLV = 64 / LPRV;      // V rows per load instruction
  constexpr int NJ = 16 / RPLV;        // V loads per 16-key group
  constexpr int LPRN = D / 8;          // lanes per 16-bit row of the new token
  // One V buffer of 32 rows per wavefront; at the end the same bytes hold that
  // wavefront's fp32 O^T (16 heads x D dims) for the merge.
  __shared__ __attribute__((aligned(16))) unsigned char s_v[NW][kI8StepKeys * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char s_k[NW][kI8StepKeys * D];  // raw K codes
  __shared__ float s_ml[NW * 16 * 2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int quad = lane >> 4;

  const int per_part = a.num_seqs * a.num_kv_heads;
  const int part = blockIdx.x / per_part;
  const int rest = blockIdx.x - part * per_part;
  const int rank = rest / a.num_kv_heads;
  const int kvh = rest - rank * a.num_kv_heads;
  const int seq = a.seq_order ? a.seq_order[rank] : rank;
  if (seq < 0 || seq >= a.num_seqs) return;
  const int h0 = kvh * G;
  const int t0 = part * a.part_tokens;

  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks;
  const int lbA = t0 / BS;
  auto load_ids = [&](int s) -> int32_t {
    return bt[min(lbA + (kI8StepKeys * s + 16 * (lane & 1)) / BS, a.max_blocks - 1)];
  };
  const int32_t ids_first = load_ids(wave);
  const int32_t ids_second = load_ids(wave + NW);
  int32_t ids_next = load_ids(wave + 2 * NW);

  // Q^T fragment for step ks: head col (columns past G repeat head h0), dims
  // (D / 4) quad + 8 ks .. + 7, the order the key codes are loaded in.
  u32x4 qf[KS];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)seq * a.num_heads + h0 + (col < G ? col : 0)) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qp[KS * quad + ks];
  }

  const int L = clamp_context(a, seq);
  if (L == 0) {
    if (part == 0) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + ((int64_t)seq * a.num_heads + h0) * D;
      for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) o[idx] = 0;
    }
    return;
  }
  if (t0 >= L) return;
  const int t1 = (int)min((int64_t)L, (int64_t)t0 + a.part_tokens);
  const int nparts_seq = 1 + (L - 1) / a.part_tokens;
  // Fused step: the partition holding position L-1 reads only the cached
  // positions before it; the new token is quantised and attended below.
  const bool new_here = a.key_new != nullptr && t1 == L;
  const int t1c = new_here ? L - 1 : t1;

  const int32_t nb32 = a.num_blocks > INT32_MAX ? INT32_MAX : (int32_t)a.num_blocks;
  const uint32_t row_bytes = (uint32_t)D;  // consecutive keys of one head
  const uint64_t block_bytes = (uint64_t)a.num_kv_heads * BS * D;
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)kvh * BS * D;
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)kvh * BS * D;
  const char* ksbase = reinterpret_cast<const char*>(a.k_scales) + (size_t)kvh * BS * 4;
  const char* vsbase = reinterpret_cast<const char*>(a.v_scales) + (size_t)kvh * BS * 4;
  const uint64_t sblock_bytes = (uint64_t)a.num_kv_heads * BS * 4;

  float m = kEmptyMax;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{};
  f32x4 lacc = f32x4{};  // row sums of the rounded P (every row holds its column's sum)
  const uint32_t one2 = pack2<DT>(1.f, 1.f);
  const u32x2 ones = {one2, one2};
  unsigned char* const sv = s_v[wave];
  unsigned char* const sk = s_k[wave];
  // Two register sets of codes and scales: the steps s + 4 and s + 8 of a
  // wavefront are in flight while step s computes.  ksc: the key scales of
  // keys 4 quad .. + 3 of each group (the keys whose scores this lane holds);
  // vrs: the value scale of the V row this lane stages (see store_v).
  struct Regs {
    u32x4 kr[2][NJ], vr[2][NJ], ksc[2];
    float vrs[2][NJ];
  };
  Regs ra, rb;

  // Codes and scales of step s (ids: the step's block ids, lane l holds group
  // l & 1).  Past the partition the resources have size 0 (zeros, no memory).
  auto issue = [&](int s, int32_t ids, Regs& r) {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      const int g0 = t0 + kI8StepKeys * s + 16 * gr;
      const int lb = g0 / BS;
      const int32_t blk = __builtin_amdgcn_readlane(ids, gr);
      const int nv = min(16, t1c - g0);
      const bool ok = nv > 0 && blk >= 0 && blk < nb32;
      report_index_error(a.index_errors, nv > 0 && !ok, kErrBlockId, blk);
      const int off_in_blk = g0 - lb * BS;
      const uint64_t off = ok ? (uint64_t)(uint32_t)blk * block_bytes + (uint64_t)off_in_blk * row_bytes : 0ull;
      const uint32_t nrec = ok ? (uint32_t)(nv - 1) * row_bytes + D : 0u;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + off, nrec);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + off, nrec);
      const uint64_t soff = ok ? (uint64_t)(uint32_t)blk * sblock_bytes + (uint64_t)off_in_blk * 4 : 0ull;
      const uint32_t snrec = ok ? (uint32_t)nv * 4 : 0u;
      const __amdgpu_buffer_rsrc_t rks = make_rsrc(ksbase + soff, snrec);
      const __amdgpu_buffer_rsrc_t rvs = make_rsrc(vsbase + soff, snrec);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int kr_row = RPLV * j + lane / LPRV;
        r.kr[gr][j] = buffer_load16<kCachePolicyNT>(
            rk, (uint32_t)kr_row * row_bytes +
                    (uint32_t)(((lane % LPRV) ^ i8_kswz<D>(16 * gr + kr_row)) * 16));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        r.vr[gr][j] = buffer_load16<kCachePolicyNT>(
            rv, (uint32_t)(RPLV * j + lane / LPRV) * row_bytes + (uint32_t)((lane % LPRV) * 16));
      r.ksc[gr] = buffer_load16<kCachePolicyNT>(rks, (uint32_t)(16 * quad));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        r.vrs[gr][j] =
            buffer_load4f<kCachePolicyNT>(rvs, (uint32_t)(4 * (RPLV * j + lane / LPRV)));
    }
  };

  // V codes -> dequantised 16-bit rows of this wavefront's LDS tile (row 16 gr +
  // RPLV j + lane / LPRV of the step, dims 16 (lane % LPRV) .. + 15 = chunks
  // 2 (lane % LPRV), +1), each code times its row's scale.
  auto store_v = [&](const Regs& r) {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int row = 16 * gr + RPLV * j + lane / LPRV;
        const int c = 2 * (lane % LPRV);
        unsigned char* rowp = sv + row * ROW;
        const u32x4 w = r.vr[gr][j];
        const float vs = r.vrs[gr][j], nb = -128.f * vs;
        const u32x2 d0 = i8x4_dequant<DT>(w.x, vs, nb), d1 = i8x4_dequant<DT>(w.y, vs, nb);
        const u32x2 d2 = i8x4_dequant<DT>(w.z, vs, nb), d3 = i8x4_dequant<DT>(w.w, vs, nb);
        *reinterpret_cast<u32x4*>(rowp + ((c ^ i8_vswz<D>(row)) * 16)) =
            u32x4{d0.x, d0.y, d1.x, d1.y};
        *reinterpret_cast<u32x4*>(rowp + (((c + 1) ^ i8_vswz<D>(row)) * 16)) =
            u32x4{d2.x, d2.y, d3.x, d3.y};
      }
  };

  // K code rows to this wavefront's LDS tile as loaded (row 16 gr + RPLV j +
  // lane / LPRV, chunk position lane % LPRV), and back as score operands: lane
  // (key col, quad) takes chunks KC quad .. + KC - 1 of key 16 gr + col, dims
  // (D / 4) quad .. + D / 4 - 1.
  auto store_k = [&](const Regs& r) {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        *reinterpret_cast<u32x4*>(sk + (16 * gr + RPLV * j + lane / LPRV) * D + (lane % LPRV) * 16) =
            r.kr[gr][j];
  };
  auto load_kq = [&](u32x4 (&kq)[2][KC]) {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      const int row = 16 * gr + col;
#pragma unroll
      for (int j = 0; j < KC; ++j)
        kq[gr][j] = *reinterpret_cast<const u32x4*>(sk + row * D + ((KC * quad + j) ^ i8_kswz<D>(row)) * 16);
    }
  };

  auto scores = [&](const u32x4 (&kq)[2][KC], const Regs& r, f32x4 (&sc)[2], f32x4 (&kscale)[2]) {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      sc[gr] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 w = kq[gr][ks >> 1];
        const u32x4 kf = (ks & 1) ? i8_to_16<DT>(w.z, w.w) : i8_to_16<DT>(w.x, w.y);
        sc[gr] = mfma16x16x32<DT>(kf, qf[ks], sc[gr]);
      }
      kscale[gr] = __builtin_bit_cast(f32x4, r.ksc[gr]);
    }
  };

  auto accumulate = [&](f32x4 (&sc)[2], const f32x4 (&kscale)[2], int kb, int kend) {
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) sc[gr] *= kscale[gr];  // key j's score x sK[j]
    if (kb + kI8StepKeys > kend) {
#pragma unroll
      for (int gr = 0; gr < 2; ++gr)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + 16 * gr + 4 * quad + i >= kend) sc[gr][i] = -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = max_xor32(max_xor16(mx)) * a.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m + kI8LazyRescale)) {
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
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      const u32x2 pf = {pack2<DT>(sc[gr][0], sc[gr][1]), pack2<DT>(sc[gr][2], sc[gr][3])};
      lacc = mfma16x16x16<DT>(ones, pf, lacc);
      const int rr = 16 * gr + 4 * quad + (col >> 2);
      const unsigned char* rowp = sv + rr * ROW + 8 * (col & 1);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int chunk = 2 * dt + ((col & 3) >> 1);
        const u32x2 vf = lds_read_tr16(rowp + ((chunk ^ i8_vswz<D>(rr)) * 16));
        o[dt] = mfma16x16x16<DT>(vf, pf, o[dt]);
      }
    }
  };

  // Step s computes from one register set, which then takes step s + 2 NW;
  // the other set holds step s + NW.  Block ids run a step ahead of the loads that
  // use them.  Look-ahead loads are unconditional (clamped ids, size-0
  // resources past the partition), so every step waits for the same loads.
  const int nsteps = (t1c - t0 + kI8StepKeys - 1) / kI8StepKeys;
  // The new token's 16-bit rows (lanes 0 .. LPRN - 1 key, LPRN .. 2 LPRN - 1
  // value, 16 bytes each) are fetched before the cached steps, on the
  // wavefront that attends to it.
  u32x4 new_x = {0u, 0u, 0u, 0u};
  if (new_here && wave == nsteps % NW && lane < 2 * LPRN) {
    const int64_t nrow = ((int64_t)seq * a.num_kv_heads + kvh) * D;
    new_x = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(lane >= LPRN ? a.value_new : a.key_new) + nrow)[lane % LPRN];
  }
  auto step = [&](int s, Regs& r) {
    const int32_t ids_after = load_ids(s + 3 * NW);
    store_k(r);
    store_v(r);
    u32x4 kq[2][KC];
    load_kq(kq);
    f32x4 sc[2], kscale[2];
    scores(kq, r, sc, kscale);
    issue(s + 2 * NW, ids_next, r);
    ids_next = ids_after;
    accumulate(sc, kscale, t0 + kI8StepKeys * s, t1c);
  };
  int s = wave;
  if (s < nsteps) {
    issue(s, ids_first, ra);
    issue(s + NW, ids_second, rb);
    while (true) {
      step(s, ra);
      s += NW;
      if (s >= nsteps) break;
      step(s, rb);
      s += NW;
      if (s >= nsteps) break;
    }
  }

  if (new_here && wave == nsteps % NW) {
    // The new token (position L-1), on the wavefront with the fewest steps.
    // Lanes 0 .. LPRN - 1 quantise its key row and the next LPRN its value row,
    // 8 dimensions each, exactly as pa_reshape_and_cache_int8 does (scale =
    // amax / 127, code = rint(x / scale), IEEE float32); the codes and scales
    // are stored at the token's slot for later steps and attended from
    // registers as a one-key step (every other key of the step is zeros and
    // masked).
    const bool is_v = lane >= LPRN;
    const int qsub = lane % LPRN;
    const u32x4 x = new_x;
    const float f[8] = {lo_f32<DT>(x.x), hi_f32<DT>(x.x), lo_f32<DT>(x.y), hi_f32<DT>(x.y),
                        lo_f32<DT>(x.z), hi_f32<DT>(x.z), lo_f32<DT>(x.w), hi_f32<DT>(x.w)};
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
#pragma unroll
    for (int o2 = LPRN / 2; o2 >= 1; o2 >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o2));  // one row
    const float qscale = amax / 127.0f;
    uint32_t pk[2] = {0u, 0u};
    if (qscale > 0.f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cq = (int)__builtin_rintf(f[e] / qscale);
        pk[e >> 2] |= ((uint32_t)cq & 0xFFu) << (8 * (e & 3));
      }
    }
    const int64_t slot = a.slot_mapping[seq];
    if (lane == 0) report_index_error(a.index_errors, slot >= a.num_slots, kErrSlot, slot);
    if (lane < 2 * LPRN && slot >= 0 && slot < a.num_slots) {
      const int64_t sblk = slot / BS;
      const int64_t srow = (sblk * a.num_kv_heads + kvh) * BS + (slot - sblk * BS);
      int8_t* codes = static_cast<int8_t*>(is_v ? a.v_cache_w : a.k_cache_w);
      *reinterpret_cast<uint2*>(codes + srow * D + 8 * qsub) = make_uint2(pk[0], pk[1]);
      if (qsub == 0) (is_v ? a.v_scales_w : a.k_scales_w)[srow] = qscale;
    }
    // Registers of the one-key step, key 0 of group 0 being the new token: its
    // key codes in the score-operand layout load_kq returns (dims (D / 4) quad
    // .. + D / 4 - 1 on the lanes with col 0, from quantising lanes KS quad ..
    // KS quad + KS - 1, 8 codes each); as issue() loads a cached step, its
    // value codes, dims 16 (lane % LPRV) .. + 15, and its value scale to lanes
    // 0 .. LPRV - 1 (from lanes LPRN + 2 (lane % LPRV) and the next); its key
    // scale to the quad-0 lanes.
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    Regs rn;
    u32x4 kqn[2][KC];
    uint32_t kw[4 * KC], vw[4];
#pragma unroll
    for (int k = 0; k < 4 * KC; ++k) kw[k] = (uint32_t)__shfl((int)pk[k & 1], KS * quad + (k >> 1));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      vw[k] = (uint32_t)__shfl((int)pk[k & 1], LPRN + 2 * (lane % LPRV) + (k >> 1));
    const float ksn = __shfl(qscale, 0), vsn = __shfl(qscale, LPRN);
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      kqn[0][j] = col == 0 ? u32x4{kw[4 * j], kw[4 * j + 1], kw[4 * j + 2], kw[4 * j + 3]} : zero4;
      kqn[1][j] = zero4;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      rn.vr[0][j] = (j == 0 && lane < LPRV) ? u32x4{vw[0], vw[1], vw[2], vw[3]} : zero4;
      rn.vr[1][j] = zero4;
      rn.vrs[0][j] = (j == 0 && lane < LPRV) ? vsn : 0.f;
      rn.vrs[1][j] = 0.f;
    }
    rn.ksc[0] = quad == 0 ? u32x4{__float_as_uint(ksn), 0u, 0u, 0u} : zero4;
    rn.ksc[1] = zero4;
    store_v(rn);
    f32x4 sc[2], kscale[2];
    scores(kqn, rn, sc, kscale);
    accumulate(sc, kscale, L - 1, L);
  }

  // Merge the NW wavefronts' (m, l, O) and write the partition.
  float* s_o = reinterpret_cast<float*>(sv);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[col * D + 16 * dt + 4 * quad + i] = o[dt][i];
  if (quad == 0) {
    s_ml[(wave * 16 + col) * 2] = m;
    s_ml[(wave * 16 + col) * 2 + 1] = lacc[0];
  }
  __syncthreads();
  const float* s_all = reinterpret_cast<const float*>(&s_v[0][0]);
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
  if (nparts_seq > 1 && (int)threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = s_ml[g * 2];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_ml[(w * 16 + g) * 2]);
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      den = fmaf(s_ml[(w * 16 + g) * 2 + 1], fast_exp2(s_ml[(w * 16 + g) * 2] - M), den);
    reinterpret_cast<float2*>(a.part_ml)[prow + g] = make_float2(M, den);
  }
}

PA_LAYOUT_PROBE(decode_int8)

template <int DT, int D, int BS, int G>
hipError_t launch_int8_t(const DecodeArgs& a, int phases, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.num_seqs * a.num_kv_heads * a.num_parts);
  if (phases & kPhaseMerge && !(phases & kPhasePartitions)) {
    launch_merge<DT, D>(a, s);
    return hipGetLastError();
  }
  // Wavefronts per workgroup: eight for spans of kMfmaLongSpan+ tokens (as for the
  // 16-bit matrix-core kernel); one for contexts cut into partitions of at most
  // kMfmaShortPartition tokens, so that a wavefront takes all steps of its short
  // partition and no merge of wavefronts follows (long split-K INT8 decode at
  // 512: four 100.3, two 96.4 then 98.9, one 96.0 us; unsplit contexts of up to
  // 2048 tokens lose with two: 62.1 -> 67.5 us); four otherwise.
  if (a.part_tokens >= kMfmaLongSpan) {
    launch((decode_int8_kernel<DT, D, BS, G, 8>), dim3(grid), dim3(512), 0, s, a);
  } else if (a.num_parts > 1 && a.part_tokens <= kMfmaShortPartition) {
    launch((decode_int8_kernel<DT, D, BS, G, 1>), dim3(grid), dim3(64), 0, s, a);
  } else {
    launch((decode_int8_kernel<DT, D, BS, G, 4>), dim3(grid), dim3(256), 0, s, a);
  }
  if (phases & kPhaseMerge) launch_merge<DT, D>(a, s);
  return hipGetLastError();
}

template <int DT, int D, int BS>
hipError_t launch_int8_g(const DecodeArgs& a, int group, int phases, hipStream_t s) {
  switch (group) {
    case 1: return launch_int8_t<DT, D, BS, 1>(a, phases, s);
    case 2: return launch_int8_t<DT, D, BS, 2>(a, phases, s);
    case 4: return launch_int8_t<DT, D, BS, 4>(a, phases, s);
    case 8: return launch_int8_t<DT, D, BS, 8>(a, phases, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t launch_int8_bs(const DecodeArgs& a, int block_size, int group, int phases,
                          hipStream_t s) {
  switch (block_size) {
    case 16: return launch_int8_g<DT, D, 16>(a, group, phases, s);
    case 32: return launch_int8_g<DT, D, 32>(a, group, phases, s);
    case 256: return launch_int8_g<DT, D, 256>(a, group, phases, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_int8(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                              int group, int phases, hipStream_t s) {
  if (head_dim == 128)
    return dtype == DT_BF16 ? launch_int8_bs<DT_BF16, 128>(a, block_size, group, phases, s)
                            : launch_int8_bs<DT_F16, 128>(a, block_size, group, phases, s);
  if (head_dim == 64)
    return dtype == DT_BF16 ? launch_int8_bs<DT_BF16, 64>(a, block_size, group, phases, s)
                            : launch_int8_bs<DT_F16, 64>(a, block_size, group, phases, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
