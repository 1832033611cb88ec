/*
 * pa_blocks.h -- KV block management for the paged cache of pa.h: a host-side
 * block manager (libpa.so) and the device block copies it asks for.
 *
 * The "vLLM Project Update" talk (recap of PagedAttention) describes managing
 * the KV cache the way an operating system manages virtual memory: a
 * sequence's logical blocks map through its block table to physical blocks
 * anywhere in the pool, which lets several requests share physical space.
 * The same talk's "prefix caching" update lets a new request reuse the cache
 * blocks of a common prefix (a system prompt) that an earlier request already
 * computed, so only the rest of its prompt is computed.  The "[core] Multi
 * Step Scheduling" pull request runs on the v2 block manager with a host swap
 * space (--swap-space).  This header gives those roles:
 *
 *   - a free-list allocator of the num_blocks physical blocks of one cache,
 *     with append of one token per sequence per step and free;
 *   - sharing by reference count: pa_bm_fork gives a new sequence all of an
 *     existing one's blocks (parallel sampling, beam search); a write into a
 *     shared block first copies it (copy-on-write), the copy reported to the
 *     caller as a (source, destination) block pair for pa_copy_blocks;
 *   - prefix caching (PA_BM_PREFIX_CACHING): a full block whose KV the caller
 *     has written (pa_bm_mark_computed) is registered under the exact token
 *     prefix it completes; a new sequence whose prompt starts with the same
 *     tokens maps those blocks instead of new ones.  A cached block that no
 *     sequence uses any more stays cached until its space is needed; the
 *     least recently released one is evicted first;
 *   - swap-out of a sequence's blocks to a host pool of num_host_blocks and
 *     swap-in back to device blocks, as (source, destination) pairs for
 *     pa_swap_blocks.
 *
 * Conventions
 *   - The manager holds host state only; it never touches device memory.  It
 *     is not thread-safe: one caller thread per manager.  Arrays passed to
 *     pa_bm_* are HOST arrays.  Sequence ids are the caller's (any int64).
 *   - Every pa_bm_* call either succeeds or changes nothing (it validates and
 *     checks capacity before it changes any state); the one exception is an
 *     out-of-memory failure inside pa_bm_mark_computed, which may leave a
 *     leading part of the blocks registered (a consistent state).
 *   - Block ids are int32 in [0, num_blocks); host block ids in
 *     [0, num_host_blocks).  The physical ids chosen are the manager's and are
 *     not part of the contract; what is: a sequence's table maps its positions
 *     to blocks holding its tokens' KV (after the caller's writes and the
 *     copies the manager reported), no block is written through two tables,
 *     and the counts reported (cached tokens, copies, free blocks) follow the
 *     rules above.
 *   - Errors: PA_ERR_NULL, PA_ERR_SHAPE (sizes, positions, table width),
 *     PA_ERR_CAPACITY (not enough free device or host blocks), PA_ERR_SEQUENCE
 *     (unknown id, an id that exists already, a duplicate id within one call,
 *     an operation on a swapped-out sequence or swap-in of a resident one).
 */
#ifndef PA_BLOCKS_H_
#define PA_BLOCKS_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* pa_bm_create flags */
#define PA_BM_PREFIX_CACHING 1u

/*
 * Create a manager of num_blocks device blocks of block_size token slots and
 * num_host_blocks host (swap) blocks.  *out receives the handle; free it with
 * pa_bm_destroy.  block_size >= 1; num_blocks >= 1; num_host_blocks >= 0.
 */
int pa_bm_create(int64_t num_blocks, int32_t block_size, int64_t num_host_blocks, uint32_t flags,
                 pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/*
 * New sequence seq_id with a prompt of num_tokens tokens (tokens: their ids,
 * required with prefix caching, else may be NULL).  It gets
 * ceil(num_tokens / block_size) blocks.  With prefix caching, its leading full
 * blocks whose exact token prefix is cached map to the cached blocks; then
 * *num_cached_tokens (may be NULL) = block_size x their count, and the
 * caller writes only positions num_cached_tokens .. num_tokens - 1 (their
 * slots: pa_bm_slots).  num_tokens = 0 gives an empty sequence.
 */
int pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                       int32_t num_tokens, int32_t* num_cached_tokens);

/*
 * Append one token to each of n distinct sequences (tokens: their ids, needed
 * for prefix caching, else may be NULL).  slots[i] receives the slot of seq
 * i's new token (its position = its length before the call).  A sequence
 * whose last block is full gets a new block; one whose last block is shared
 * with another sequence gets a private copy: the pair (shared block, new
 * block) is appended to copies[2 * k], copies[2 * k + 1] and *num_copies
 * counts the pairs (at most n; copies may be NULL only if n = 0).  Run the
 * copies (pa_copy_blocks) before writing the new tokens' KV.
 */
int pa_bm_append(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* tokens, int32_t n,
                 int64_t* slots, int32_t* copies, int32_t* num_copies);

/* New sequence child sharing every block of parent (reference counts + 1). */
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* Release a sequence (resident or swapped out) and its references. */
int pa_bm_free(pa_block_manager* bm, int64_t seq_id);

/*
 * Register every full block of seq_id whose KV is now written in the prefix
 * cache (a no-op without PA_BM_PREFIX_CACHING).  Call it after the writes of
 * a prompt and whenever appended tokens have filled blocks.  A block whose
 * token prefix is cached already (through another block) stays private.
 */
int pa_bm_mark_computed(pa_block_manager* bm, int64_t seq_id);

/*
 * Slots of positions start .. start + n - 1 of seq_id (0 <= start,
 * start + n <= its length), e.g. the slot mapping of a prompt write.
 */
int pa_bm_slots(const pa_block_manager* bm, int64_t seq_id, int32_t start, int32_t n,
                int64_t* slots);

/*
 * Block tables and context lengths of n resident sequences, ready for
 * pa_decode: block_tables[i * max_blocks_per_seq + j] = block j of seq_ids[i]
 * (-1 past its last block); context_lens[i] = its length.  PA_ERR_SHAPE if a
 * sequence has more than max_blocks_per_seq blocks.
 */
int pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                       int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* context_lens);

/*
 * Swap seq_id's blocks out to host blocks: pairs[2 * j], pairs[2 * j + 1] =
 * (device block, host block) for each of its blocks in order (room for
 * ceil(length / block_size) pairs), *num_pairs their count.  Enqueue their
 * copies (pa_swap_blocks) before any KV write into blocks allocated after
 * this call: the device blocks are released at once (a block still shared
 * stays with its other users) and may be handed out again.
 */
int pa_bm_swap_out(pa_block_manager* bm, int64_t seq_id, int32_t* pairs, int32_t* num_pairs);

/*
 * Swap seq_id back in to new device blocks: pairs = (host block, device
 * block), as for pa_bm_swap_out; its host blocks are released.
 */
int pa_bm_swap_in(pa_block_manager* bm, int64_t seq_id, int32_t* pairs, int32_t* num_pairs);

/* Device blocks an allocation can take now (free + cached but unused). */
int pa_bm_num_free_blocks(const pa_block_manager* bm, int64_t* num_free);
/* Free host (swap) blocks. */
int pa_bm_num_free_host_blocks(const pa_block_manager* bm, int64_t* num_free);
/* Length of a sequence and whether it is resident (1) or swapped out (0). */
int pa_bm_seq_info(const pa_block_manager* bm, int64_t seq_id, int32_t* length,
                   int32_t* resident);
/* Reference count of a device block (sequences mapping it). */
int pa_bm_ref_count(const pa_block_manager* bm, int32_t block, int32_t* refs);

/*
 * pa_copy_blocks -- the device side of copy-on-write: for each pair
 * (src, dst) of `pairs` (a DEVICE int32 array [num_pairs][2]), copy physical
 * block src to block dst in both caches (every head, every slot).  The
 * caches are the pa.h layouts: a block is block_bytes contiguous bytes in
 * each (num_kv_heads * block_size * head_dim * element size).  Destinations
 * must be distinct and no destination may be a source.  block_bytes must be
 * a positive multiple of 16, caches 16-byte aligned; pairs in [0, num_blocks)
 * are a precondition (out-of-range pairs are skipped on the device).
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                   int64_t num_blocks, int64_t block_bytes, void* stream);

/*
 * pa_swap_blocks -- the copies of a swap: for each pair (src, dst) of the
 * HOST int32 array `pairs`, copy block_bytes bytes from src_pool + src *
 * block_bytes to dst_pool + dst * block_bytes, as asynchronous copies on
 * `stream` (runs of consecutive blocks go as one copy).  One pool is a
 * device cache, the other host memory allocated pinned (hipHostMalloc);
 * call once for the key cache and once for the value cache.
 */
int pa_swap_blocks(void* dst_pool, const void* src_pool, const int32_t* pairs, int32_t num_pairs,
                   int64_t block_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H_ */
