// Internal launch interface between the C ABI (pa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Index errors a PA_CHECK_INDICES build records on the device instead of
// skipping the access silently: the kinds seen (an OR of the bits) and the
// kind and offending value of the first one.  In other builds the kernels
// never touch it and the pointer in the launch arguments is null.
enum : uint32_t {
  kErrBlockId = 1,      // a block id a context needs lies outside [0, num_blocks)
  kErrSlot = 2,         // a slot at or past num_blocks * block_size (negative = padding, legal)
  kErrContextLen = 4,   // a context length < 0, above max_context_len, or shorter than its chunk
  kErrQueryLoc = 8,     // query_start_loc not within [0, num_tokens], or a chunk above max_query_len
};

struct IndexErrors {
  uint32_t kinds;
  uint32_t first_kind;
  int64_t first_value;
};

struct ReshapeArgs {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int64_t num_slots;   // num_blocks * block_size
  int row_chunks;      // 16-byte chunks in one token's num_kv_heads * head_dim row
  IndexErrors* index_errors;  // PA_CHECK_INDICES builds only; null otherwise
};

struct RopeReshapeArgs {
  void* q;                 // [num_tokens][num_heads][head_dim], rotated in place; or null
  const void* key;         // [num_tokens][num_kv_heads][head_dim]
  const void* value;
  void* k_cache;           // [num_blocks][block_size][num_kv_heads][head_dim]
  void* v_cache;
  const int64_t* positions;  // [num_tokens]
  const float* cos;        // [max_position][head_dim / 2]
  const float* sin;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int64_t num_slots;
  int64_t max_position;
  int num_heads;
  int num_kv_heads;
  IndexErrors* index_errors;  // PA_CHECK_INDICES builds only; null otherwise
};

struct ReshapeInt8Args {
  const void* key;       // [num_tokens][num_kv_heads][head_dim], 16-bit
  const void* value;
  void* k_codes;         // int8 [num_blocks][num_kv_heads][block_size][head_dim]
  void* v_codes;
  float* k_scales;       // [num_blocks][num_kv_heads][block_size]
  float* v_scales;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int64_t num_slots;
  int num_kv_heads;
  int block_size;
  IndexErrors* index_errors;  // PA_CHECK_INDICES builds only; null otherwise
};

struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  const int64_t* src;    // [num_copies] source blocks
  const int64_t* dst;    // [num_copies] destination blocks
  int64_t num_copies;
  int64_t num_blocks;
  int64_t block_chunks;  // 16-byte chunks in one block of one cache
  IndexErrors* index_errors;  // PA_CHECK_INDICES builds only; null otherwise
};

struct DecodeArgs {
#ifdef PA_LAYOUT_SKEW_TEST
  // Only in the layout check's test object: a translation unit compiled
  // against an older DecodeArgs, every later field shifted.
  const void* stale_field;
#endif
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint16_t* part_out;  // [num_seqs][num_parts][num_heads][head_dim], partition-normalised, cache dtype
  float* part_ml;      // [num_seqs][num_parts][num_heads][2]: log2-domain max, sum
  // Partial mode (null otherwise): `out` receives each row's normalised output
  // and out_ml [num_seqs][num_heads][2] its log2-domain max and sum, so that the
  // row can later be merged with rows computed over other keys.
  float* out_ml;
  const int32_t* seq_order;  // optional [num_seqs]: order in which sequences are visited
  // Fused decode step (all null otherwise): this step's token of sequence i is
  // at position context_lens[i] - 1; its K/V rows come from key_new/value_new
  // [num_seqs][num_kv_heads][head_dim] and are also stored at slot_mapping[i].
  const void* key_new;
  const void* value_new;
  const int64_t* slot_mapping;
  void* k_cache_w;
  void* v_cache_w;
  const float* k_scales;  // INT8 caches only: [num_blocks][num_kv_heads][block_size]
  const float* v_scales;
  // INT8 fused step only (null otherwise): where the new token's scales are stored.
  float* k_scales_w;
  float* v_scales_w;
  // Fused rotary embedding (fused step only; null otherwise): the query and the
  // new key of sequence i are rotated by row positions[i] of the float32
  // tables [max_position][head_dim / 2] before use (rows outside the table:
  // no rotation).
  const int64_t* positions;
  const float* rope_cos;
  const float* rope_sin;
  int64_t max_position;
  int64_t num_slots;   // num_blocks * block_size
  int64_t num_blocks;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int max_blocks;
  int max_context_len;
  int num_parts;       // partitions per sequence in the grid
  int part_tokens;     // tokens per partition (>= every context when unsplit)
  int num_cus;         // compute units of the device: how many workgroups fit at once
  float scale_log2;    // scale * log2(e)
  IndexErrors* index_errors;  // PA_CHECK_INDICES builds only; null otherwise
};

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  const int32_t* seq_order;  // optional [num_seqs]: order in which sequences are visited
  int64_t num_blocks;
  int64_t num_tokens;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int max_blocks;
  int max_query_len;
  int q_tiles;         // query tiles per sequence in the grid
  float scale_log2;
  IndexErrors* index_errors;  // PA_CHECK_INDICES builds only; null otherwise
};

hipError_t launch_reshape_and_cache(const ReshapeArgs& a, hipStream_t s);
hipError_t launch_rope_reshape(const RopeReshapeArgs& a, int dtype, int head_dim, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s);
hipError_t launch_reshape_int8(const ReshapeInt8Args& a, int dtype, int head_dim, hipStream_t s);
// Which launches of a decode to enqueue: the partition kernel (a2-a5), the
// partition merge (a6, only when a context spans several partitions), or both.
enum : int { kPhasePartitions = 1, kPhaseMerge = 2, kPhaseAll = 3 };

// INT8 decode: DecodeArgs with k_cache / v_cache pointing at the int8 codes and
// the per-row scales in k_scales / v_scales.
hipError_t launch_decode_int8(const DecodeArgs& a, int dtype, int head_dim, int block_size,
                              int group, int phases, hipStream_t s);

// dtype DT_F16 / DT_BF16; head_dim 64/128; block_size 16/32/256; group 1/2/4/8.
hipError_t launch_decode_f16(const DecodeArgs& a, int head_dim, int block_size, int group,
                             int phases, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, int head_dim, int block_size, int group,
                              int phases, hipStream_t s);

// Merge of partials computed over disjoint key sets (context-parallel shards).
struct MergePartialsArgs {
  void* out;               // [num_rows][head_dim], 16-bit
  float* out_ml;           // optional [num_rows][2]
  const void* part_o;      // [num_shards][num_rows][head_dim], 16-bit
  const float* part_ml;    // [num_shards][num_rows][2]
  int64_t num_rows;        // num_seqs * num_heads
  int num_shards;
};

hipError_t launch_merge_partials(const MergePartialsArgs& a, int dtype, int head_dim,
                                 hipStream_t s);

hipError_t launch_cache_flush(const void* buf, int64_t chunks, bool non_temporal, hipStream_t s);

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int block_size,
                          int group, hipStream_t s);

// ---- kernel timing events --------------------------------------------------
// Events armed on the calling thread by pa_set_kernel_events: the first kernel
// launched after arming records `start` (if any) and every kernel launched
// while armed records `stop` as it ends, from the dispatch's own timestamps.
struct KernelEvents {
  hipEvent_t start;
  hipEvent_t stop;
  bool start_pending;
};
KernelEvents& kernel_events();

// Every kernel of the library is launched through this: hipLaunchKernelGGL,
// or the extended launch that records the armed events.
template <typename... KArgs, typename... Args>
inline void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds_bytes,
                   hipStream_t s, Args... args) {
  KernelEvents& ev = kernel_events();
  hipStreamCaptureStatus capturing = hipStreamCaptureStatusNone;
  if (ev.stop != nullptr) (void)hipStreamIsCapturing(s, &capturing);
  if (ev.stop == nullptr || capturing != hipStreamCaptureStatusNone) {  // no events in a graph
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, s, args...);
    return;
  }
  hipEvent_t start = ev.start_pending ? ev.start : nullptr;
  ev.start_pending = false;
  hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, s, start, ev.stop, 0u, args...);
}

// ---- layout check ----------------------------------------------------------
// The launch-argument structs cross translation units by value, so every unit
// must compile them alike: a kernel object built against an older version of
// this header would read every field after a change at the wrong offset.  Each
// kernel unit exports this fingerprint as it compiled it (PA_LAYOUT_PROBE) and
// the C ABI compares them with its own at load; on a mismatch every entry
// point that launches a kernel fails instead.
constexpr uint64_t layout_mix(uint64_t h, uint64_t v) { return (h ^ v) * 1099511628211ull; }

constexpr uint64_t args_layout() {
  uint64_t h = 1469598103934665603ull;
  const uint64_t parts[] = {
      sizeof(ReshapeArgs), offsetof(ReshapeArgs, num_tokens), offsetof(ReshapeArgs, index_errors),
      sizeof(RopeReshapeArgs), offsetof(RopeReshapeArgs, num_tokens),
      offsetof(RopeReshapeArgs, index_errors),
      sizeof(ReshapeInt8Args), offsetof(ReshapeInt8Args, num_tokens),
      offsetof(ReshapeInt8Args, index_errors),
      sizeof(CopyBlocksArgs), offsetof(CopyBlocksArgs, num_copies),
      offsetof(CopyBlocksArgs, index_errors),
      sizeof(DecodeArgs), offsetof(DecodeArgs, q), offsetof(DecodeArgs, part_out),
      offsetof(DecodeArgs, key_new), offsetof(DecodeArgs, k_scales), offsetof(DecodeArgs, positions),
      offsetof(DecodeArgs, num_slots), offsetof(DecodeArgs, num_seqs), offsetof(DecodeArgs, num_cus),
      offsetof(DecodeArgs, scale_log2), offsetof(DecodeArgs, index_errors),
      sizeof(MergePartialsArgs), offsetof(MergePartialsArgs, num_rows),
      sizeof(PrefillArgs), offsetof(PrefillArgs, num_blocks), offsetof(PrefillArgs, scale_log2),
      offsetof(PrefillArgs, index_errors), sizeof(IndexErrors),
#ifdef PA_CHECK_INDICES
      1,
#else
      0,
#endif
  };
  for (uint64_t v : parts) h = layout_mix(h, v);
  return h;
}

#define PA_LAYOUT_PROBE(unit) \
  uint64_t layout_probe_##unit() { return args_layout(); }

uint64_t layout_probe_reshape_and_cache();
uint64_t layout_probe_rope_reshape();
uint64_t layout_probe_reshape_int8();
uint64_t layout_probe_copy_blocks();
uint64_t layout_probe_decode_f16();
uint64_t layout_probe_decode_bf16();
uint64_t layout_probe_decode_int8();
uint64_t layout_probe_merge_partials();
uint64_t layout_probe_prefill();

}  // namespace pa
