/*
 * pa.h -- C ABI of libpa.so, paged attention for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  Scaled dot-product attention softmax(q . K^T * scale) . V
 * (page "Nano-vLLM-Ascend", section 2.2.1, the attention listing) over many
 * variable-length sequences whose keys and values live in a paged KV cache:
 * the cache is cut into fixed-size token blocks, a sequence of L tokens holds
 * ceil(L / block_size) blocks, and a per-sequence block table maps logical
 * block j to a physical block (same page, section 2.1, the Block / BlockTable
 * structures and the 16-token worked example).  Block sizes 16, 32 and 256 are
 * supported (16/32: same page, section 2.1 tip; 256: page "vLLM-Ascend ...",
 * section 2.2 tuning table).  Softmax statistics are kept in fp32 (page
 * "vLLM-Ascend ...", section 3.1, problem 2: fp16 accumulation errors fixed by
 * a float softmax).
 *
 * Layouts (all tensors dense, row-major, element type fp16 or bf16 unless
 * stated):
 *   key cache, value cache : [num_blocks][block_size][num_kv_heads][head_dim]
 *                            (the per-block (block_size, num_heads, head_dim)
 *                            layout of the Block structure, page
 *                            "Nano-vLLM-Ascend", section 2.1), one array each.
 *   block_tables           : int32 [num_seqs][max_blocks_per_seq]; entry j of
 *                            row i is the physical block of logical block j of
 *                            sequence i.  Entries at or past
 *                            ceil(context_lens[i] / block_size) are never read.
 *   context_lens           : int32 [num_seqs]; tokens sequence i attends over,
 *                            including the tokens written this step.
 *   slot_mapping           : int64 [num_tokens]; flat slot = block * block_size
 *                            + offset; a negative slot marks a padding token.
 *   Query head h reads KV head h / (num_heads / num_kv_heads).
 *
 * Ownership and threading.  Every pointer argument except `stream` is a device
 * pointer owned by the caller; the library allocates no device memory and keeps
 * no per-call state.  Each call validates its host arguments, enqueues kernels
 * on `stream` (a hipStream_t; NULL = the default stream) and returns without
 * synchronising.  Calls are thread-safe.
 *
 * Errors.  Every entry point returns a pa_status.  Host arguments are checked
 * before any HIP call; a failed check returns PA_ERR_INVALID_ARG or
 * PA_ERR_UNSUPPORTED and enqueues nothing; pa_last_error() then gives a
 * thread-local message.  A kernel launch failure returns PA_ERR_HIP, and so
 * does every call that launches kernels when the library's parts were built
 * from different versions of its sources (a check made once, at load).
 * Device contents are the caller's contract: block ids outside [0,
 * num_blocks), slots at or past num_blocks * block_size and context lengths
 * above max_context_len are skipped or clamped by the kernels (never
 * dereferenced) and leave the affected output undefined.  The checking build
 * of the library (libpa_check.so, compiled with PA_CHECK_INDICES) also records
 * each such case on the device; pa_take_index_errors reports them.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,  /* null pointer, negative size, inconsistent shape */
  PA_ERR_UNSUPPORTED = -2,  /* head_dim / block_size / group / dtype not built  */
  PA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required      */
  PA_ERR_HIP = -4,          /* a HIP launch reported an error                   */
  PA_ERR_NO_BLOCKS = -5,    /* block manager: too few free blocks (pa_blocks.h)  */
  PA_ERR_BAD_INDEX = -6     /* checking build: kernels met out-of-range indices  */
} pa_status;

typedef enum pa_dtype { PA_F16 = 0, PA_BF16 = 1 } pa_dtype;

/* Library version, (major << 16) | minor. */
int pa_version(void);

/* Static description of a status code. */
const char* pa_status_string(int status);

/* Detail of the last failed call on the calling thread ("" if none). */
const char* pa_last_error(void);

/*
 * Index checks (a debugging aid for the caller's block tables and slot
 * mappings; the pages diagnose leaked or corrupted blocks from the block
 * table's reference counts, page "Nano-vLLM-Ascend", section 4.2, problem 3).
 * The library built with PA_CHECK_INDICES (libpa_check.so; same entry points,
 * same results) makes its kernels record, in a per-device error record, every
 * index they would otherwise skip or clamp:
 *   PA_INDEX_ERR_BLOCK_ID     a block id that a context needs (or a copy source
 *                             or destination) outside [0, num_blocks)
 *   PA_INDEX_ERR_SLOT         a slot at or past num_blocks * block_size
 *                             (negative slots are padding, not errors)
 *   PA_INDEX_ERR_CONTEXT_LEN  a context length < 0 or above max_context_len
 *                             (prefill: shorter than its chunk, or past the table)
 *   PA_INDEX_ERR_QUERY_LOC    query_start_loc outside [0, num_tokens], or a chunk
 *                             longer than max_query_len
 * The offending access is still skipped, so nothing faults.
 *
 * pa_check_indices_enabled: 1 in the checking build, 0 otherwise.
 *
 * pa_take_index_errors: waits for `stream` (HOST pointers for the results),
 * returns the kinds recorded on the stream's device since the previous call
 * (an OR of the bits above), the kind and value of the first one, and clears
 * the record.  Returns PA_OK when there were none, PA_ERR_BAD_INDEX when there
 * were; PA_ERR_UNSUPPORTED in a library built without PA_CHECK_INDICES.
 */
enum {
  PA_INDEX_ERR_BLOCK_ID = 1,
  PA_INDEX_ERR_SLOT = 2,
  PA_INDEX_ERR_CONTEXT_LEN = 4,
  PA_INDEX_ERR_QUERY_LOC = 8
};

int pa_check_indices_enabled(void);

int pa_take_index_errors(void* stream, uint32_t* kinds, uint32_t* first_kind,
                         int64_t* first_value);

/*
 * Measuring aids.
 *
 * pa_set_kernel_events arms HIP events (hipEvent_t handles the caller created
 * with timing enabled) on the calling thread.  While armed, every kernel a
 * library call on this thread launches records stop_event as it ends, from
 * the dispatch's own end timestamp (hipExtLaunchKernel); start_event, if not
 * NULL, is recorded by the first kernel launched after arming, as it begins
 * (the runtime may place it in a packet of its own just before that kernel).
 * Arming again replaces both; (NULL, NULL) disarms.  A start event without a
 * stop event is PA_ERR_INVALID_ARG.  A call that launches no kernel leaves the
 * events as they were.  The events stay the caller's and must outlive the
 * launches that record them.  Stop events armed around two calls in turn give,
 * by hipEventElapsedTime, the device time from the end of the first call's
 * last kernel to the end of the second's.  Launches into a stream that is
 * being captured into a HIP graph record no events.
 *
 * pa_cache_flush reads `bytes` bytes of the device buffer `buf` (address and
 * size multiples of 16) on `stream` and writes nothing: read through a buffer
 * larger than the caches, it leaves the L2s and the Infinity Cache holding
 * clean lines of its own, so that a kernel after it finds none of its
 * operands cached.  bytes == 0 is a no-op; a NULL buffer or misaligned
 * address or size is PA_ERR_INVALID_ARG.
 *
 * pa_stream_read is the same read with non-temporal loads, which leave the
 * caches' contents alone (so it is no flush): timed over a buffer several
 * times the Infinity Cache, it gives the device's streaming read rate from
 * HBM, the practical ceiling for kernels that stream their operands once.
 * Same arguments and errors as pa_cache_flush.
 */
int pa_set_kernel_events(void* start_event, void* stop_event);

int pa_cache_flush(const void* buf, size_t bytes, void* stream);

int pa_stream_read(const void* buf, size_t bytes, void* stream);

/*
 * reshape_and_cache: write this step's new keys and values into their cache
 * slots (the fill of fixed-size blocks, page "vLLM-Ascend ...", section 2.2,
 * preprocessing stage; block layout of page "Nano-vLLM-Ascend", section 2.1).
 *
 *   key, value   [num_tokens][num_kv_heads][head_dim]   read
 *   k_cache, v_cache                                     written at the slots
 *   slot_mapping [num_tokens] int64                      read; < 0 = skip token
 *
 * For every token t with 0 <= slot < num_blocks * block_size, the
 * num_kv_heads * head_dim row of token t is copied bit for bit to
 * cache[slot / block_size][slot % block_size].  Duplicate slots in one call
 * are a caller error (which write lands is unspecified).  num_tokens == 0 is a
 * no-op.  Supported: head_dim in {64, 128}, block_size in {16, 32, 256}.
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                         int head_dim, int block_size, int64_t num_blocks, int dtype,
                         void* stream);

/*
 * pa_rope_reshape_and_cache: rotary position embedding fused with
 * pa_reshape_and_cache.  The pages apply the rotary embedding through a
 * primitive of (x, cos, sin) whose backward is the same primitive with -sin
 * (page "Nano-vLLM-Ascend", section 5.1) and name operator fusion as a way to
 * save passes (page "vLLM-Ascend ...", section 5).  Rotation of a row x at
 * position p: with h = head_dim / 2, for i < h
 *   y_i     = x_i c - x_{i+h} s,   y_{i+h} = x_{i+h} c + x_i s,
 *   c = cos_table[p][i], s = sin_table[p][i],
 * each product and the sum or difference rounded to float32 separately (no
 * fused multiply-add) and the result rounded once to dtype, nearest even.
 *
 *   q          NULL, or [num_tokens][num_heads][head_dim]   rotated in place
 *   key, value [num_tokens][num_kv_heads][head_dim]         read
 *   k_cache, v_cache  as for pa_reshape_and_cache           written at the slots
 *   positions  [num_tokens] int64                           read
 *   cos_table, sin_table  float32 [max_position][head_dim/2] read
 *   slot_mapping [num_tokens] int64                         read
 *
 * For each token t with 0 <= positions[t] < max_position: its query rows (if q
 * is given) are rotated in place; if 0 <= slot_mapping[t] < num_blocks *
 * block_size, its rotated key rows go to k_cache and its value rows, unchanged,
 * to v_cache at that slot.  A token with a position outside the table changes
 * nothing.  q must not overlap the other arrays; all device arrays except
 * positions and slot_mapping 16-byte aligned.  num_tokens == 0 is a no-op.
 * Supported: head_dim in {64, 128}, block_size in {16, 32, 256}, dtype PA_F16
 * or PA_BF16.
 */
int pa_rope_reshape_and_cache(void* q, const void* key, const void* value, void* k_cache,
                              void* v_cache, const int64_t* positions, const float* cos_table,
                              const float* sin_table, const int64_t* slot_mapping,
                              int64_t num_tokens, int num_heads, int num_kv_heads, int head_dim,
                              int block_size, int64_t num_blocks, int64_t max_position, int dtype,
                              void* stream);

/*
 * Bytes of device workspace pa_decode needs for these sizes (0 when the
 * context fits one partition, i.e. partition_size == 0 or
 * max_context_len <= partition_size).  Pure host arithmetic.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_heads, int head_dim, int max_context_len,
                                int partition_size);

/*
 * A partition_size for pa_decode / pa_decode_step suited to the current
 * device: 0 (no split) when the num_seqs * num_kv_heads (sequence, KV head)
 * pairs already give every compute unit two workgroups; otherwise a multiple
 * of block_size (at least 512) that cuts max_context_len into enough
 * partitions for about eight workgroups per compute unit.  Every split gives
 * the same attention up to rounding; this one trades the partitions'
 * parallelism against the partial results they write (page "vLLM-Ascend ...",
 * section 3.1: split the long context across cores, then reduce).  Host
 * arithmetic plus a device-attribute query; returns PA_ERR_INVALID_ARG for
 * non-positive counts or a negative length, PA_ERR_UNSUPPORTED for another
 * block size.
 */
int pa_decode_partition_hint(int num_seqs, int num_kv_heads, int max_context_len,
                             int block_size);

/*
 * pa_decode: one query token per sequence attends over its paged context
 * (attention of page "Nano-vLLM-Ascend", section 2.2.1; paging of section
 * 2.1; float softmax of page "vLLM-Ascend ...", section 3.1, problem 2).
 *
 *   out  [num_seqs][num_heads][head_dim]   written (same dtype as q)
 *   q    [num_seqs][num_heads][head_dim]   read
 *   k_cache, v_cache, block_tables, context_lens as described above.
 *
 * out[i][h] = sum_j p_j V_j with p = softmax_j(scale * q[i][h] . K_j) over the
 * logical tokens j < context_lens[i] of sequence i, K_j/V_j taken from KV head
 * h / (num_heads / num_kv_heads).  A sequence with context length 0 gets a
 * zero row.  Context lengths above max_context_len are treated as
 * max_context_len (which must be <= max_blocks_per_seq * block_size).
 *
 * seq_order: NULL, or an int32 [num_seqs] device array holding a permutation
 * of 0..num_seqs-1: the order in which the kernel's workgroups take up the
 * sequences.  It changes no result, only the schedule: longest context first
 * (pa_decode_order) lets the hardware dispatcher balance the compute units.
 * Entries outside [0, num_seqs) are skipped (those outputs are not written).
 *
 * partition_size: 0 = each (sequence, KV head) is processed by one workgroup;
 * otherwise a positive multiple of block_size: the context is split into
 * partitions of that many tokens processed in parallel and merged by a second
 * kernel using each partition's fp32 max and sum and its normalised output
 * (rounded to the cache dtype, as the final output is), which needs
 * pa_decode_workspace_size(...) bytes of `workspace` (device memory, caller
 * owned, 16-byte aligned, no initialisation needed, reused only after the
 * call's kernels finish on `stream`).
 *
 * Supported: num_heads / num_kv_heads in {1, 2, 4, 8}; head_dim in {64, 128};
 * block_size in {16, 32, 256}; dtype PA_F16 or PA_BF16; scale finite and > 0
 * (PA_ERR_INVALID_ARG otherwise: the softmax temperature, 1/sqrt(head_dim) in the
 * pages' attention).
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
              int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
              int64_t num_blocks, int max_blocks_per_seq, int max_context_len, float scale,
              int partition_size, void* workspace, size_t workspace_bytes, int dtype,
              void* stream);

/*
 * The two phases of a split decode as calls of their own.  pa_decode with
 * partition_size > 0 enqueues the partition kernel (each partition's fp32 max,
 * sum and normalised output into the workspace; sequences that fit one
 * partition are written to `out` directly) and then, when some context spans
 * several partitions, the merge of those partitions (the reduction after a
 * split of the context across cores, page "vLLM-Ascend ...", section 3.1).
 *
 * pa_decode_partitions: the first phase alone.  Arguments, rules and
 * supported shapes exactly as for pa_decode; rows of sequences whose context
 * spans several partitions are left unwritten until pa_decode_merge runs.
 *
 * pa_decode_merge: the second phase alone, over the workspace that a
 * preceding split decode on `stream` filled (pa_decode_partitions, or any of
 * pa_decode, pa_decode_step, pa_decode_step_rope, pa_decode_int8,
 * pa_decode_step_int8, which already merge; a repeated merge rewrites the
 * same rows).  num_seqs, num_heads, head_dim, max_context_len,
 * partition_size, context_lens, seq_order, workspace and dtype must be those
 * of that call.  Writes out[i][h] for every sequence i whose context spans
 * more than one partition (and that seq_order lists), nothing else.  A no-op
 * when partition_size == 0 or max_context_len <= partition_size.  Returns
 * PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED (head_dim not 64/128, dtype) or
 * PA_ERR_WORKSPACE (missing, short, not 16-byte aligned) before any HIP call.
 */
int pa_decode_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                         int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                         int max_context_len, float scale, int partition_size, void* workspace,
                         size_t workspace_bytes, int dtype, void* stream);

int pa_decode_merge(void* out, const int32_t* context_lens, const int32_t* seq_order,
                    int num_seqs, int num_heads, int head_dim, int max_context_len,
                    int partition_size, void* workspace, size_t workspace_bytes, int dtype,
                    void* stream);

/*
 * pa_decode_step: one decode step, i.e. pa_reshape_and_cache of one new token
 * per sequence followed by pa_decode, in a single kernel launch.  The new
 * token of sequence i is logical position context_lens[i] - 1; its rows
 * key[i], value[i] ([num_seqs][num_kv_heads][head_dim]) are attended to as
 * that position's K/V and stored bit for bit at cache slot slot_mapping[i]
 * (skipped when the slot is negative or outside the pool).  Cache positions
 * below context_lens[i] - 1 are read from the caches.  Results equal
 * pa_reshape_and_cache followed by pa_decode whenever slot_mapping[i] is the
 * slot of position context_lens[i] - 1 in sequence i's block table; the
 * summation order differs, so bits may differ within rounding.  Other
 * arguments, workspace rules and supported shapes as for pa_decode.
 */
int pa_decode_step(void* out, const void* q, const void* key, const void* value,
                   const int64_t* slot_mapping, void* k_cache, void* v_cache,
                   const int32_t* block_tables, const int32_t* context_lens,
                   const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                   int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                   int max_context_len, float scale, int partition_size, void* workspace,
                   size_t workspace_bytes, int dtype, void* stream);

/*
 * pa_decode_step_scratch: pa_decode_step for callers that cannot allocate
 * device memory (code under HIP-graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and rules as pa_decode_step
 * with partition_size honoured, except that there is no workspace argument:
 * the partial results of split contexts go to a static scratch array of
 * 16 MiB that the library keeps on each device it runs on until the process
 * ends.  The call allocates and frees nothing.  A split whose workspace would
 * exceed 16 MiB (pa_decode_workspace_size) is rejected with PA_ERR_WORKSPACE
 * before any HIP call.  Nothing in the scratch needs clearing (each call
 * writes every byte it later reads), but all calls on one device share it:
 * calls whose kernels overlap on one device (for example on two streams) race
 * and give undefined results; calls ordered on one stream are safe.
 */
int pa_decode_step_scratch(void* out, const void* q, const void* key, const void* value,
                           const int64_t* slot_mapping, void* k_cache, void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, int64_t num_blocks,
                           int max_blocks_per_seq, int max_context_len, float scale,
                           int partition_size, int dtype, void* stream);

/*
 * Context parallelism.  A long sequence's context can be split across devices
 * (page "vllm-ascend architecture", sections 1.1 and 3.1): each device holds
 * some of the sequence's tokens in its own pool, attends over them, and the
 * devices' results are merged exactly.  The unit exchanged is a partial row:
 *
 *   o   [num_seqs][num_heads][head_dim]  softmax-normalised output over the
 *                                        shard's keys (same dtype as q)
 *   ml  [num_seqs][num_heads][2] float32 (m, l): m = the shard's maximum of
 *                                        scale * q . K_j * log2(e) (or a value
 *                                        up to 8 below it), l = sum_j
 *                                        2^(scale * q . K_j * log2(e) - m)
 *
 * (m, l) is fixed only up to (m + c, l * 2^-c); l * 2^m is what a consumer
 * uses.  A shard with no key of a sequence reports (m, l) = (-inf, 0) and a
 * zero o row.
 *
 * pa_decode_partial: pa_decode over the shard's keys (its own block tables and
 * context lengths, counted in the shard's tokens) writing the partial row
 * (out = o, out_ml = ml, 8-byte aligned) instead of a final one.  Arguments,
 * workspace and supported shapes as for pa_decode; out_ml must not be NULL
 * when num_seqs > 0.
 */
int pa_decode_partial(void* out, float* out_ml, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                      int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                      int max_context_len, float scale, int partition_size, void* workspace,
                      size_t workspace_bytes, int dtype, void* stream);

/*
 * pa_merge_partials: merge num_shards partial rows into the attention over the
 * union of the shards' keys:
 *   M = max m_n over shards with l_n > 0,  w_n = l_n 2^(m_n - M),
 *   out = sum_n w_n o_n / sum_n w_n.
 *
 *   out        [num_seqs][num_heads][head_dim]             written (dtype)
 *   out_ml     NULL or [num_seqs][num_heads][2] float32    written: (M, sum_n w_n),
 *              so merged rows are partial rows again and merges compose
 *   partial_o  [num_shards][num_seqs][num_heads][head_dim] read (dtype, 4-byte aligned)
 *   partial_ml [num_shards][num_seqs][num_heads][2]        read (8-byte aligned)
 *
 * Shards with l_n <= 0 (or NaN) are left out without reading their o or m into
 * the arithmetic; a row with no such shard gets zeros and (-inf, 0).  Result
 * rows are rounded once to dtype.  Supported: head_dim in {64, 128}, dtype
 * PA_F16 or PA_BF16, any num_shards >= 1.  num_seqs == 0 is a no-op.
 */
int pa_merge_partials(void* out, float* out_ml, const void* partial_o, const float* partial_ml,
                      int num_shards, int num_seqs, int num_heads, int head_dim, int dtype,
                      void* stream);

/*
 * pa_decode_step_rope: pa_decode_step with the rotary embedding of
 * pa_rope_reshape_and_cache folded in.  The query rows of sequence i and its
 * new key row are rotated by row positions[i] of cos_table / sin_table
 * (float32 [max_position][head_dim / 2], 16-byte aligned) with exactly the
 * arithmetic of pa_rope_reshape_and_cache, then used as in pa_decode_step: the
 * rotated key (and the value, unchanged) is stored at slot_mapping[i] and
 * attended to at position context_lens[i] - 1.  q itself is only read.  A
 * position outside [0, max_position) leaves that sequence's rows unrotated.
 * Results equal pa_rope_reshape_and_cache (on a copy of q) followed by
 * pa_decode_step on the rotated rows, bit for bit; one launch fewer.  Other
 * arguments, workspace rules and supported shapes as for pa_decode_step.
 */
int pa_decode_step_rope(void* out, const void* q, const void* key, const void* value,
                        const int64_t* slot_mapping, const int64_t* positions, const float* cos_table,
                        const float* sin_table, int64_t max_position, void* k_cache, void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                        int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                        int max_context_len, float scale, int partition_size, void* workspace,
                        size_t workspace_bytes, int dtype, void* stream);

/*
 * INT8 KV cache.  KV-cache compression by INT8 quantisation is the next
 * optimisation the pages list (page "Nano-vLLM-Ascend", section 4.3) and the
 * one that raises throughput if the attention scores keep their precision
 * (page "vLLM-Ascend ...", section 5).  Scheme (symmetric, per token and KV
 * head, IEEE float32): scale = max_d |x_d| / 127, code_d = rint(x_d / scale)
 * (ties to even; an all-zero row has scale 0 and codes 0); the value used is
 * code_d * scale.
 *
 *   k_codes, v_codes   : int8 [num_blocks][num_kv_heads][block_size][head_dim]
 *   k_scales, v_scales : float32 [num_blocks][num_kv_heads][block_size]
 *
 * Unlike the 16-bit caches, the INT8 caches are head-major within a block: the
 * block_size rows of one KV head are contiguous, so a decode reads each
 * (block, head) as one run.
 *
 * pa_reshape_and_cache_int8: quantise key/value [num_tokens][num_kv_heads]
 * [head_dim] (16-bit, dtype) into the slots of slot_mapping, as
 * pa_reshape_and_cache (negative or out-of-pool slots are skipped).
 * Supported: head_dim in {64, 128}, block_size in {16, 32, 256}.
 */
int pa_reshape_and_cache_int8(const void* key, const void* value, void* k_codes, void* v_codes,
                              float* k_scales, float* v_scales, const int64_t* slot_mapping,
                              int64_t num_tokens, int num_kv_heads, int head_dim, int block_size,
                              int64_t num_blocks, int dtype, void* stream);

/*
 * pa_decode_int8: pa_decode over an INT8 cache: out[i][h] = softmax(scale *
 * q[i][h] . K'_j) . V'_j with K'_j, V'_j the dequantised rows; q and out are
 * 16-bit (dtype).  Arguments, partitions, workspace (pa_decode_workspace_size)
 * and seq_order as for pa_decode.  Supported: head_dim 64 or 128; num_heads /
 * num_kv_heads in {1, 2, 4, 8}; block_size in {16, 32, 256}.
 */
int pa_decode_int8(void* out, const void* q, const void* k_codes, const void* v_codes,
                   const float* k_scales, const float* v_scales, const int32_t* block_tables,
                   const int32_t* context_lens, const int32_t* seq_order, int num_seqs,
                   int num_heads, int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                   int max_blocks_per_seq, int max_context_len, float scale, int partition_size,
                   void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * pa_decode_step_int8: one decode step over an INT8 cache, i.e.
 * pa_reshape_and_cache_int8 of one new token per sequence followed by
 * pa_decode_int8, in a single kernel launch.  The new token of sequence i is
 * logical position context_lens[i] - 1; its 16-bit rows key[i], value[i]
 * ([num_seqs][num_kv_heads][head_dim], dtype) are quantised per (token, KV
 * head) exactly as pa_reshape_and_cache_int8 quantises a row, stored at cache
 * slot slot_mapping[i] (codes in k_codes / v_codes, scales in k_scales /
 * v_scales; skipped when the slot is negative or outside the pool) and
 * attended to as that position's dequantised K/V.  Cache positions below
 * context_lens[i] - 1 are read from the caches.  Codes and scales written equal
 * pa_reshape_and_cache_int8's bit for bit; the output equals
 * pa_reshape_and_cache_int8 followed by pa_decode_int8 whenever slot_mapping[i]
 * is the slot of position context_lens[i] - 1 in sequence i's block table,
 * within rounding (the summation order differs).  Other arguments, workspace
 * rules and supported shapes as for pa_decode_int8.
 */
int pa_decode_step_int8(void* out, const void* q, const void* key, const void* value,
                        const int64_t* slot_mapping, void* k_codes, void* v_codes, float* k_scales,
                        float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* seq_order, int num_seqs, int num_heads, int num_kv_heads,
                        int head_dim, int block_size, int64_t num_blocks, int max_blocks_per_seq,
                        int max_context_len, float scale, int partition_size, void* workspace,
                        size_t workspace_bytes, int dtype, void* stream);

/*
 * pa_decode_order: host-side helper (HOST pointers, no GPU work).  Writes to
 * order[0..num_seqs) the sequence indices sorted by decreasing
 * context_lens[i], equal lengths in index order -- the longest-first visiting
 * order to pass (after a copy to the device) as seq_order.
 */
int pa_decode_order(const int32_t* context_lens, int num_seqs, int32_t* order);

/*
 * pa_prefill_chunk: chunked prefill over the paged cache (single-device
 * chunking of long prefills, page "vllm-ascend architecture", sections 1.1
 * and 3.1).  Sequence i contributes n_i = query_start_loc[i+1] -
 * query_start_loc[i] new query tokens (rows query_start_loc[i] ..
 * query_start_loc[i+1]-1 of q and out) that follow c_i = context_lens[i] - n_i
 * cached tokens; the new tokens' keys and values must already be in the cache
 * (pa_reshape_and_cache).  New token t attends to logical keys 0 .. c_i + t
 * (its own key included); a row that sees no key (c_i + t < 0, a caller
 * error) is written as zeros.
 *
 *   out, q          [num_tokens][num_heads][head_dim]
 *   query_start_loc int32 [num_seqs + 1], non-decreasing, query_start_loc[0] = 0,
 *                   query_start_loc[num_seqs] = num_tokens
 *   seq_order       NULL or a permutation of 0..num_seqs-1 (visiting order, as
 *                   for pa_decode; longest context first balances best)
 *   max_query_len   >= every n_i (sizes the grid; longer chunks are truncated)
 *
 * QK^T and PV run as 32x32x16 matrix-core (MFMA) tiles with fp32 accumulation;
 * the softmax is fp32 and the probabilities are rounded to the input dtype
 * before the PV product.  Supported: head_dim 64 or 128; block_size 16, 32, 256;
 * num_heads / num_kv_heads in {1, 2, 4, 8}; dtype PA_F16 or PA_BF16; scale finite and
 * > 0 (PA_ERR_INVALID_ARG otherwise).
 */
int pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start_loc, const int32_t* seq_order, int num_seqs,
                     int64_t num_tokens, int num_heads, int num_kv_heads, int head_dim,
                     int block_size, int64_t num_blocks, int max_blocks_per_seq,
                     int max_query_len, float scale, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
