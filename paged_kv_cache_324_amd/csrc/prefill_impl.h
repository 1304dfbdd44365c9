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
// row (lane l -> row l % 32 of its wavefront); with head_dim D (64 or 128) a
// 16-key step takes D / 16 score MFMAs per 32 keys and D / 32 value tiles:
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
// 2); the probabilities are rounded to the input dtype for the PV product.  The
// row sum adds exactly those rounded probabilities in fp32, two per
// v_dot2_f32 with a pair of ones (16 per tile; lane l and l ^ 32 each sum their
// half of the keys and are added once at the end).
#pragma once

#include <type_traits>

#include "mfma.h"
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

constexpr int kPrefillKeys = 64;        // keys per KV tile
constexpr float kPrefillEmptyMax = -1.0e30f;
constexpr float kLazyRescale = 8.0f;
constexpr int kXcds = 8;  // workgroups are dispatched round-robin over the 8 XCDs of an MI355X

// A raw buffer resource as its four descriptor words (base, stride 0,
// num_records = bytes, the same flags as make_rsrc), wave-uniform.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu),
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), (uint32_t)kBufferWord3};
}

// LDS byte offset of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 with
// the lds bit): lane l fills LDS bytes [lds_base + 16 l, + 16); lanes past the
// buffer's size write zeros.  Issued as assembly: the compiler cannot tell
// which LDS bytes such a copy writes, so for the builtin it waits for the copy
// before every later LDS read, which would serialise a prefetch with the
// compute it is meant to overlap.  The caller waits (s_waitcnt vmcnt) before
// reading the destination; the compiler's own waits stay correct because the
// counter retires in order.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t lds_base, uint32_t voffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}

// Swizzle of the 16-byte chunks of a tile row: chunk c of row r is stored at
// position c ^ swz<D>(r).
// * D = 128 (256-byte rows, 16 chunks): swz(r) is the two 2-bit fields of r & 15
//   swapped.  Both read patterns then hit 16 distinct 16-byte bank groups: 16
//   consecutive rows at one chunk (the K operand), and 4 consecutive rows
//   (4 r0 .. 4 r0 + 3) at 4 adjacent chunks (4 a .. 4 a + 3, the transposed V
//   operand), since (4 a + i) ^ ((j << 2) | k) = 4 (a ^ j) + (i ^ k).
// * D = 64 (128-byte rows, 8 chunks; two rows span the 64 banks): swz(r) =
//   ((r >> 1) ^ (r & 2)) & 7 runs through all 8 positions over the even rows
//   of 16 consecutive ones and over the odd rows (the K operand), and gives rows
//   r0 and r0 + 2 (r0 % 4 = 0) disjoint pairs of adjacent positions (the
//   transposed V operand reads 4 rows x 2 adjacent chunks per 16 lanes).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return ((row >> 1) ^ (row & 2)) & 7;
  }
}

template <int D>
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return (uint32_t)row * (2 * D) + (uint32_t)((chunk ^ swz<D>(row)) * 16);
}

template <int DT, int D, int BS, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(const PrefillArgs a) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int NK = kPrefillKeys;
  constexpr int QT = 128 / G;
  constexpr int ROW = 2 * D;           // bytes of a key row in LDS
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;        // rows a 1 KB load of 64 lanes covers
  static_assert(BS % 16 == 0, "a wavefront stages 16 keys of one block");
  // [buffer][K or V][64 key rows x 2D bytes]: double-buffered tiles filled straight
  // from the cache by buffer loads into LDS.
  __shared__ __attribute__((aligned(16))) unsigned char s_kv[2][2][NK * ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;

  // XCD-aware order.  Workgroup b runs on XCD b % 8; each XCD takes every 8th
  // (sequence, KV head) group and runs that group's query tiles back to back,
  // so the group's K/V is fetched from HBM once and then served by that
  // XCD's L2.  Groups go heaviest sequence first (seq_order), and within a
  // group the last query tiles (which see the most keys) go first.
  const int xcd = blockIdx.x % kXcds;
  const int kx = blockIdx.x / kXcds;
  const int gi = kx / a.q_tiles;
  const int qt = a.q_tiles - 1 - (kx - gi * a.q_tiles);
  const int group = gi * kXcds + xcd;
  if (group >= a.num_seqs * a.num_kv_heads) return;
  const int rank = group / a.num_kv_heads;
  const int kvh = group - rank * a.num_kv_heads;
  const int seq = a.seq_order ? a.seq_order[rank] : rank;
  if (seq < 0 || seq >= a.num_seqs) return;

  const int s0 = a.query_start_loc[seq];
  const int n_raw = a.query_start_loc[seq + 1] - s0;
  const int n = min(n_raw, a.max_query_len);
  const int L_raw = a.context_lens[seq];
  const int L = max(0, min(L_raw, a.max_blocks * BS));
  const int c = L - n;  // cached tokens before the chunk (negative: caller error)
  const int t0 = qt * QT;
  if (threadIdx.x == 0 && qt == a.q_tiles - 1) {  // once per (sequence, KV head)
    report_index_error(a.index_errors,
                       s0 < 0 || n_raw < 0 || n_raw > a.max_query_len ||
                           (int64_t)s0 + n_raw > a.num_tokens,
                       kErrQueryLoc, s0);
    report_index_error(a.index_errors, L_raw < n_raw || L_raw > a.max_blocks * BS,
                       kErrContextLen, L_raw);
  }
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
        static_cast<const uint16_t*>(a.q) +
        ((int64_t)(s0 + (row_valid ? t : 0)) * a.num_heads + h) * D);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 v = qp[ks * 2 + half];
      qf[ks] = row_valid ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m = kPrefillEmptyMax;
  // This lane's keys of its row's sum of the rounded P (lane l ^ 32 holds the others).
  float lpart = 0.f;
  const uint32_t one2 = pack2<DT>(1.f, 1.f);

  // ---- staging: wavefront w moves keys kv0 + 16 w .. + 15 (one block) of K
  // and of V with 16 / RPL 1 KB buffer loads each; lane l of load i brings key row
  // RPL i + l / CPR, chunk (l % CPR) ^ swz(row), so the tile lands already swizzled.
  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks;
  const int32_t nb32 = a.num_blocks > INT32_MAX ? INT32_MAX : (int32_t)a.num_blocks;
  const uint32_t row_bytes = (uint32_t)a.num_kv_heads * D * 2;
  const uint64_t block_bytes = (uint64_t)BS * row_bytes;
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)kvh * D * 2;
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)kvh * D * 2;
  const int nblk_last = max(0, (L + BS - 1) / BS - 1);
  const int srow = lane / CPR;  // row within a 1 KB load
  // Block ids, lane-parallel: for window w, lane j holds the id of the block
  // this wavefront stages in tile 64 w + j (reads clamped to the context).
  auto load_ids = [&](int w) -> int32_t {
    const int key0 = (64 * w + lane) * NK + 16 * wave;
    return bt[min(key0 / BS, nblk_last)];
  };
  // KIND 0: the K rows, 1: the V rows of the tile at key kv0, into buffer buf.
  auto stage = [&](auto kind, int kv0, int buf, int32_t ids) {
    constexpr int KIND = decltype(kind)::value;
    const int key0 = kv0 + 16 * wave;
    const int lb = key0 / BS;
    const int32_t blk = __builtin_amdgcn_readlane(ids, (kv0 / NK) & 63);
    const int nvalid = min(16, L - key0);
    const bool ok = nvalid > 0 && blk >= 0 && blk < nb32;
    if (KIND == 0) report_index_error(a.index_errors, nvalid > 0 && !ok, kErrBlockId, blk);
    const uint64_t boff = ok ? (uint64_t)(uint32_t)blk * block_bytes +
                                   (uint64_t)(key0 - lb * BS) * row_bytes
                             : 0ull;
    const uint32_t nrec = ok ? (uint32_t)(nvalid - 1) * row_bytes + D * 2 : 0u;
    const u32x4 rs = rsrc_words((KIND == 0 ? kbase : vbase) + boff, nrec);
#pragma unroll
    for (int i = 0; i < 16 / RPL; ++i) {
      const int r = RPL * i + srow;  // 0..15, also the tile row modulo 16
      const uint32_t voff = (uint32_t)r * row_bytes + (uint32_t)(((lane % CPR) ^ swz<D>(r)) * 16);
      lds_dma16(rs, lds_offset(s_kv[buf][KIND] + (16 * wave + RPL * i) * ROW), voff);
    }
  };
  using KRows = std::integral_constant<int, 0>;
  using VRows = std::integral_constant<int, 1>;

  // Operand addressing inside a tile.
  //   S^T = K Q^T, A operand: key row 32 sub + l % 32, dims 16 ks + 8 half .. + 7.
  //   O^T = V^T P^T, A operand by transposed reads: 16-lane group q = l / 16
  //   (half = q / 2, dim half dh = q % 2), position p = l % 16 addresses key row
  //   16 kk + 4 half (+ 8 for the second read) + p / 4 at dims
  //   32 dt + 16 dh + 4 (p % 4) .. + 3, so lane l receives those four keys of
  //   dim 32 dt + l % 32.
  const int p16 = lane & 15;
  const int dh = (lane >> 4) & 1;
  // Those addresses for tile buffer 0, per lane, computed once.  Key rows 32 sub
  // + r and 16 kk + r share r's swizzle (it depends on r % 16 only), so the other
  // halves and steps add immediates (32 sub, 16 kk rows); the buffer flip of each
  // tile adds +-kBuf to all of them.
  constexpr int kBuf = 2 * NK * ROW;   // bytes from tile buffer 0 to buffer 1
  uint32_t koff[D / 16], vlo[D / 32], vhi[D / 32];
  {
    const int r1 = 4 * half + (p16 >> 2);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) koff[ks] = tile_off<D>(lane & 31, 2 * ks + half);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int chunk = 4 * dt + 2 * dh + ((p16 & 3) >> 1);
      vlo[dt] = NK * ROW + tile_off<D>(r1, chunk) + 8 * (p16 & 1);
      vhi[dt] = NK * ROW + tile_off<D>(r1 + 8, chunk) + 8 * (p16 & 1);
    }
  }
  const unsigned char* const lds = &s_kv[0][0][0];

  // Smallest causal limit over the wavefront's rows: tiles below it need no mask.
  int wave_min_vis = vis;
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) wave_min_vis = min(wave_min_vis, __shfl_xor(wave_min_vis, o2));
  wave_min_vis = __builtin_amdgcn_readfirstlane(wave_min_vis);

  // ---- S^T of the tile whose K rows koff addresses, both 32-key halves,
  // their products alternating so that no product waits for the one before
  // it; the operands of D / 32 dim steps are read ahead of the first product
  // (with the order pinned by the caller, see pin_scores).
  auto scores = [&](f32x16 (&sc)[2]) {
    constexpr int AHEAD = D / 32;
    u32x4 kf[2][D / 16];
#pragma unroll
    for (int ks = 0; ks < AHEAD; ++ks) {
      kf[0][ks] = *reinterpret_cast<const u32x4*>(lds + koff[ks]);
      kf[1][ks] = *reinterpret_cast<const u32x4*>(lds + koff[ks] + 32 * ROW);
    }
    sc[0] = f32x16{};
    sc[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      if (ks + AHEAD < D / 16) {
        kf[0][ks + AHEAD] = *reinterpret_cast<const u32x4*>(lds + koff[ks + AHEAD]);
        kf[1][ks + AHEAD] = *reinterpret_cast<const u32x4*>(lds + koff[ks + AHEAD] + 32 * ROW);
      }
      sc[0] = mfma32x32x16<DT>(kf[0][ks], qf[ks], sc[0]);
      sc[1] = mfma32x32x16<DT>(kf[1][ks], qf[ks], sc[1]);
    }
  };
  // scores() alone: D / 16 LDS reads, then (2 products, 2 reads) while reads
  // remain, then the last products.
  auto pin_scores = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (ks + D / 32 < D / 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // ---- causal mask of the tile at key kv0 (this lane's query).  Only tiles
  // that cross some row's limit need it.
  auto mask = [&](f32x16 (&sc)[2], int kv0) {
    if (kv0 + NK > wave_min_vis) {
      // key kv0 + 4 half + c (c = 32 sub + 8 (j / 4) + j % 4) is visible iff c < lim
      const int lim = vis - kv0 - 4 * half;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int c = sub * 32 + 8 * (j >> 2) + (j & 3);
          sc[sub][j] = c < lim ? sc[sub][j] : -__builtin_inff();
        }
      }
    }
  };

  // ---- online softmax of a masked tile, in place, without a branch: the
  // row maximum (this lane and its partner l ^ 32), the lazy update of m
  // (only when some row's maximum grows by more than kLazyRescale, in log2
  // units; until then p <= 2^kLazyRescale, harmless in fp32 and in the 16-bit
  // P), and p = 2^(s scale_log2 - m).  The scale is positive, so the maximum is
  // taken over raw scores and folded into the exponent.  Returns the factor
  // O and l must be rescaled by (1 when m did not move) and whether it moved.
  auto softmax = [&](f32x16 (&sc)[2], bool& moved) -> float {
    float mx = -__builtin_inff();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[sub][j]);
    }
    mx = max_xor32(mx) * a.scale_log2;  // partner lane l ^ 32, by a lane swap
    moved = (__builtin_amdgcn_read_exec() & __builtin_amdgcn_ballot_w64(mx > m + kLazyRescale)) != 0;
    const float m_new = moved ? fmaxf(m, mx) : m;
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[sub][j] = fast_exp2(fmaf(sc[sub][j], a.scale_log2, -m));
    }
    return alpha;
  };

  // ---- O^T += V^T P^T over the tile's four 16-key steps (V rows at vlo/vhi),
  // and the row sum of the same rounded P.  Raised wave priority: of the two
  // wavefronts sharing a SIMD, the one with products ready issues first.
  auto pv = [&](const f32x16 (&sc)[2]) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < NK / 16; ++kk) {
      const f32x16& ps = sc[kk >> 1];
      const int jb = 8 * (kk & 1);
      const u32x4 pf = {pack2<DT>(ps[jb + 0], ps[jb + 1]), pack2<DT>(ps[jb + 2], ps[jb + 3]),
                        pack2<DT>(ps[jb + 4], ps[jb + 5]), pack2<DT>(ps[jb + 6], ps[jb + 7])};
      lpart = dot2<DT>(pf.w, one2, dot2<DT>(pf.z, one2, dot2<DT>(pf.y, one2, dot2<DT>(pf.x, one2, lpart))));
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x2 lo = lds_read_tr16(lds + vlo[dt] + kk * 16 * ROW);
        const u32x2 hi = lds_read_tr16(lds + vhi[dt] + kk * 16 * ROW);
        o[dt] = mfma32x32x16<DT>(u32x4{lo.x, lo.y, hi.x, hi.y}, pf, o[dt]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- pipeline.  Tile i's K and V rows live in buffer i & 1, but in
  // different iterations: iteration i computes S^T of tile i + 1 (its K) while
  // the vector ALU runs tile i's softmax, then tile i's value product (its V).
  // So at the top of iteration i, after one barrier, K of tile i + 2 streams
  // into the buffer tile i's K leaves and V of tile i + 1 into the one tile
  // i - 1's V leaves, each with a whole iteration to arrive.  Block ids come
  // lane-parallel in windows of 64 tiles, loaded a window ahead (one set for
  // the K stream, one for the V stream).
  const int ntiles = (kv_end + NK - 1) / NK;
  const int nw = min(ntiles, (wave_end + NK - 1) / NK);  // tiles this wavefront computes
  int32_t idk = 0, idk_n = 0, idv = 0, idv_n = 0;
  if (ntiles > 0) {
    idk = load_ids(0);
    idk_n = load_ids(1);
    idv = idk;
    idv_n = idk_n;
    stage(KRows{}, 0, 0, idk);
    if (ntiles > 1) stage(KRows{}, NK, 1, idk);
    stage(VRows{}, 0, 0, idv);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x16 sa[2], sb[2];
  if (nw > 0) {
    scores(sa);
    pin_scores();
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] += kBuf;  // K of tile 1

  // One iteration: sc holds tile it's raw scores, sn receives tile it + 1's.
  auto iteration = [&](int it, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 2 < ntiles) {
      if (((it + 2) & 63) == 0) {
        idk = idk_n;
        idk_n = load_ids(((it + 2) >> 6) + 1);
      }
      stage(KRows{}, (it + 2) * NK, it & 1, idk);
    }
    if (it + 1 < ntiles) {
      if (((it + 1) & 63) == 0) {
        idv = idv_n;
        idv_n = load_ids(((it + 1) >> 6) + 1);
      }
      stage(VRows{}, (it + 1) * NK, (it + 1) & 1, idv);
    }
    if (it < nw) {
      mask(sc, it * NK);
      bool moved;
      float alpha;
      if (it + 1 < nw) {
        scores(sn);
        alpha = softmax(sc, moved);
        // Interleave: the next tile's D / 8 products run on the matrix cores
        // while this tile's softmax issues on the vector ALU between them.  The
        // first 20 vector instructions (the row maximum) go before the first
        // product, while its operand reads land; then six per product (10 or 16
        // up front, or 4, 5, 7 or 8 per product, measured 0.3-7% slower).
        __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 1);
        __builtin_amdgcn_sched_group_barrier(0x402, 20, 1);
#pragma unroll
        for (int k = 0; k < D / 8; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x402, 6, 1);
          if ((k & 1) && k / 2 + D / 32 < D / 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
      } else {
        alpha = softmax(sc, moved);
      }
      if (moved) {
        lpart *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
      }
      pv(sc);
    }
    // next iteration: K of tile it + 2 (buffer it & 1), V of tile it + 1
    const int32_t kflip = (it & 1) ? kBuf : -kBuf;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) koff[ks] += kflip;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      vlo[dt] -= kflip;
      vhi[dt] -= kflip;
    }
  };
  for (int it = 0; it < ntiles; it += 2) {
    iteration(it, sa, sb);
    if (it + 1 < ntiles) iteration(it + 1, sb, sa);
  }

  // ---- normalise and store: lane holds dims 32 dt + 8 (j/4) + 4 half + (j%4)
  const float lsum = sum_xor32(lpart);
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

template <int DT, int D, int BS, int G>
hipError_t launch_prefill_t(const PrefillArgs& a0, hipStream_t s) {
  PrefillArgs a = a0;
  constexpr int QT = 128 / G;
  a.q_tiles = (a.max_query_len + QT - 1) / QT;
  const int64_t groups = (int64_t)a.num_seqs * a.num_kv_heads;
  const int64_t grid = (groups + kXcds - 1) / kXcds * kXcds * a.q_tiles;
  if (grid == 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  launch((prefill_kernel<DT, D, BS, G>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int D, int BS>
hipError_t launch_prefill_g(const PrefillArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_prefill_t<DT, D, BS, 1>(a, s);
    case 2: return launch_prefill_t<DT, D, BS, 2>(a, s);
    case 4: return launch_prefill_t<DT, D, BS, 4>(a, s);
    case 8: return launch_prefill_t<DT, D, BS, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t launch_prefill_dt(const PrefillArgs& a, int block_size, int group, hipStream_t s) {
  switch (block_size) {
    case 16: return launch_prefill_g<DT, D, 16>(a, group, s);
    case 32: return launch_prefill_g<DT, D, 32>(a, group, s);
    case 256: return launch_prefill_g<DT, D, 256>(a, group, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
