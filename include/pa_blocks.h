/*
 * pa_blocks.h -- host block manager and block copy of libpa.so.
 *
 * The step before the attention path: which physical block of the KV cache
 * holds which tokens of which sequence.  A block holds block_size tokens and
 * a reference count; a sequence's block table maps its logical block j to a
 * physical block (page "Nano-vLLM-Ascend", section 2.1, the Block and
 * BlockTable structures; a 1000-token sequence of 16-token blocks holds
 * ceil(1000 / 16) = 63 blocks, 1008 slots).  Blocks are shared between
 * sequences by reference count (prefix sharing for long contexts, page
 * "vLLM-Ascend ...", section 4); a shared block that one sequence is about to
 * write is first copied to a private block (copy on write).  A block returns to
 * the free pool when its count drops to zero, so a pool whose sequences have
 * all been freed is entirely free again: the reference-count check the pages
 * prescribe for memory leaks (page "Nano-vLLM-Ascend", section 4.2, problem 3)
 * is pa_bm_num_free() == num_blocks.
 *
 * The manager produces exactly the inputs of pa.h: slot mappings for
 * pa_reshape_and_cache / pa_decode_step, block tables and context lengths for
 * pa_decode / pa_prefill_chunk, and the (source, destination) block pairs that
 * pa_copy_blocks must copy before the new tokens are written.
 *
 * Allocation policy (fixed, so results are reproducible): free blocks form a
 * stack that initially pops 0, 1, 2, ...; a freed block is pushed and is the
 * next one handed out.
 *
 * Threading: a manager serialises its own calls (an internal mutex); several
 * managers are independent.  All arrays of the pa_bm_* calls are host memory
 * owned by the caller.  On any error a call changes nothing.
 */
#ifndef PA_BLOCKS_H_
#define PA_BLOCKS_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager of physical blocks 0 .. num_blocks-1 of block_size tokens, all
 * free.  num_blocks in [1, 2^31 - 1], block_size >= 1.  *out receives the
 * handle (owned by the caller, released with pa_bm_destroy). */
int pa_bm_create(int64_t num_blocks, int block_size, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* A new sequence `seq` (any id not in use) holding num_tokens >= 0 tokens, e.g.
 * a prompt: ceil(num_tokens / block_size) blocks are allocated and the slot of
 * token t (block * block_size + t % block_size) is written to slots[t]
 * (slots may be NULL when num_tokens == 0).  PA_ERR_NO_BLOCKS if the pool has
 * too few free blocks. */
int pa_bm_add(pa_block_manager* bm, int64_t seq, int64_t num_tokens, int64_t* slots);

/* A new sequence `child` sharing the first num_tokens tokens of `parent`
 * (0 <= num_tokens <= the parent's tokens): it takes the parent's first
 * ceil(num_tokens / block_size) blocks, each of whose counts goes up by one.
 * No block is allocated. */
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child, int64_t num_tokens);

/* Append n >= 0 tokens to `seq` and write their slots to slots[0 .. n-1].  New
 * blocks are allocated as needed.  If the sequence's last block is partly
 * filled and shared (count > 1), it is first replaced by a fresh private block
 * and the pair (shared block, fresh block) is queued for pa_bm_take_copies:
 * the device copy must run before the new tokens are written to the cache.
 * PA_ERR_NO_BLOCKS if the pool has too few free blocks. */
int pa_bm_append(pa_block_manager* bm, int64_t seq, int64_t n, int64_t* slots);

/* Release `seq`: every block's count goes down by one, blocks reaching zero
 * return to the pool. */
int pa_bm_free(pa_block_manager* bm, int64_t seq);

/* Block tables and context lengths of a batch, in the layout pa_decode reads:
 * row i of block_tables (int32 [num_seqs][max_blocks_per_seq]) holds the
 * blocks of seqs[i] followed by -1 padding, context_lens[i] its token count.
 * PA_ERR_INVALID_ARG if a sequence is unknown or has more blocks than
 * max_blocks_per_seq. */
int pa_bm_tables(pa_block_manager* bm, const int64_t* seqs, int num_seqs,
                 int max_blocks_per_seq, int32_t* block_tables, int32_t* context_lens);

/* Move up to `capacity` queued copy-on-write pairs, oldest first, into
 * src[] / dst[] and return how many were moved (>= 0), or a negative status. */
int64_t pa_bm_take_copies(pa_block_manager* bm, int64_t* src, int64_t* dst, int64_t capacity);

/* Free blocks in the pool; tokens of `seq` (-1 if unknown); count of physical
 * block `block` (-1 if out of range); sequences held. */
int64_t pa_bm_num_free(pa_block_manager* bm);
int64_t pa_bm_num_tokens(pa_block_manager* bm, int64_t seq);
int pa_bm_ref_count(pa_block_manager* bm, int64_t block);
int64_t pa_bm_num_seqs(pa_block_manager* bm);

/* Device: copy whole blocks src[i] -> dst[i], i < num_copies, in both caches
 * ([num_blocks][block_size][num_kv_heads][head_dim], dtype PA_F16 / PA_BF16):
 * the copy-on-write step of the block manager.  src, dst: int64 device arrays.
 * Pairs with an id outside [0, num_blocks) or src == dst are skipped; two
 * pairs with the same destination race (the manager never queues such
 * pairs).  Supported: head_dim in {64, 128}, block_size in {16, 32, 256}. */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* src, const int64_t* dst,
                   int64_t num_copies, int num_kv_heads, int head_dim, int block_size,
                   int64_t num_blocks, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H_ */
