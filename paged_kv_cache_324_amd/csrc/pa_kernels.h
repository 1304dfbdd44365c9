// Internal launch interface between the C ABI (pa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct ReshapeArgs {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int64_t num_slots;   // num_blocks * block_size
  int row_chunks;      // 16-byte chunks in one token's num_kv_heads * head_dim row
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
};

struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  const int64_t* src;    // [num_copies] source blocks
  const int64_t* dst;    // [num_copies] destination blocks
  int64_t num_copies;
  int64_t num_blocks;
  int64_t block_chunks;  // 16-byte chunks in one block of one cache
};

struct DecodeArgs {
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
  float scale_log2;    // scale * log2(e)
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
hipError_t launch_decode_int8(const DecodeArgs& a, int dtype, int block_size, int group,
                              int phases, hipStream_t s);

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

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int block_size,
                          int group, hipStream_t s);

}  // namespace pa
