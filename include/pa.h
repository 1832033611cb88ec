/*
 * pa.h -- C ABI of the MI355X (gfx950) paged KV-cache library (libpa.so).
 *
 * Two operations make up the decode hot path of paged attention:
 *
 *   pa_cache_write  scatter each new token's key and value rows into
 *                   fixed-size physical cache blocks through a slot mapping
 *                   ("[core] Multi Step Scheduling" pull request, vllm #7000,
 *                   review thread on ops.advance_step: the per-step state is
 *                   slot_mapping, block_tables, seq_lens and block_size).
 *
 *   pa_decode       single-query attention out = softmax(scale * q.K^T).V per
 *                   (sequence, query head), with K/V gathered block by block
 *                   through a per-sequence block table ("vLLM Project Update"
 *                   talk, PagedAttention recap: attention over blocks of the
 *                   KV cache managed like virtual-memory pages).  The result is
 *                   exact attention ("vLLM: Easy, Fast, and Cheap LLM Serving
 *                   with PagedAttention" thread: paging changes where K/V live,
 *                   not what is computed).  Long or uneven contexts are split
 *                   into partitions whose partial results are merged with a
 *                   log-sum-exp reduction (same talk, passage on the second
 *                   PagedAttention kernel, likened there to flash decoding).
 *
 * Conventions
 *   - All tensor arguments are DEVICE pointers to densely packed row-major
 *     arrays unless a stride argument says otherwise.  The caller owns every
 *     buffer; the library allocates no device memory and keeps no state
 *     between calls (one exception: pa_decode_noalloc's static scratch array,
 *     below).  Calls from several host threads are safe.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued: PA_OK means "validated and launched", nothing is waited for,
 *     and no device->host copy is made (grids are sized from the maximum
 *     context, max_blocks_per_seq * block_size, not from context_lens).
 *   - Errors are reported by the return value: a negative pa_status, detected
 *     on the host before anything is launched (or PA_ERR_HIP if a launch
 *     fails).  No C++ exception crosses this interface.
 *   - Cache layout (chosen for gfx950, see each kernel): the tokens of a block
 *     are kept in quads of four consecutive offsets; X = 16 bytes / element
 *     size (8 for f16/bf16, 4 for f32):
 *       key cache   [num_blocks][num_kv_heads][block_size/4][head_dim/X][4][X]
 *       value cache [num_blocks][num_kv_heads][block_size/4][head_dim][4]
 *     Key element e of the token at offset o: quad o/4, chunk e/X, row o%4,
 *     lane e%X.  Value element e of offset o: quad o/4, dim e, row o%4.  So a
 *     quad's 16-byte key chunks and a quad's four values of one dim are
 *     contiguous, and one token's write fills 32 of each 128 bytes it touches.
 *   - Slot s addresses block s / block_size, offset s % block_size.
 *   - Block-table entries and slots are preconditions: entries
 *     block_tables[b][0 .. ceil(L_b/block_size)-1] must lie in
 *     [0, num_blocks); slots must be < num_blocks * block_size.  Entries past a
 *     sequence's last block are never read and may hold anything (e.g. -1).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,      /* IEEE binary32 */
  PA_DTYPE_F16 = 1,      /* IEEE binary16 */
  PA_DTYPE_BF16 = 2,     /* bfloat16 */
  PA_DTYPE_FP8_E4M3 = 3  /* OCP 8-bit float E4M3 (bias 7, 3 significand bits,
                            largest finite 448, no infinities, S.1111.111 NaN);
                            KV caches only, with one scale per cache tensor */
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  PA_ERR_DTYPE = -3,       /* unknown dtype or unsupported dtype combination */
  PA_ERR_UNSUPPORTED = -4, /* head_dim / block_size / group size not built */
  PA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
  PA_ERR_HIP = -6,         /* a HIP launch failed */
  PA_ERR_CAPACITY = -7,    /* block manager: not enough free blocks (nothing changed) */
  PA_ERR_SEQUENCE = -8,    /* block manager: unknown, duplicate or swapped-out sequence */
  PA_ERR_SCRATCH = -9      /* pa_decode_noalloc: the workspace would exceed PA_SCRATCH_BYTES */
} pa_status;

/* pa_decode flags.  Bits 0-1: which decode kernel family to use. */
#define PA_DECODE_AUTO 0u       /* library picks kernel family and waves */
#define PA_DECODE_FORCE_VALU 1u /* vector-ALU kernel (all dtypes) */
#define PA_DECODE_FORCE_MFMA 2u /* matrix-core kernel (f16/bf16 KV only) */
#define PA_DECODE_KERNEL_MASK 3u
/* Bits 2-3: waves per (sequence, kv head, partition) work item; the waves
 * split the item's tokens and merge their partial results on chip.  0 lets
 * the library pick: 4 for partitions of 1024 tokens or more, 2 from 256
 * tokens, else 1. */
#define PA_DECODE_WAVES_1 4u
#define PA_DECODE_WAVES_2 8u
#define PA_DECODE_WAVES_4 12u
#define PA_DECODE_WAVES_MASK 12u
/* Bits 4-5: how a partitioned launch's workgroups find their work items
 * (sequence, kv head, head chunk, partition).  0 lets the library pick.
 *   PA_DECODE_NO_WORK_LIST  one workgroup per possible item, in grid order
 *                           (the items that hold no tokens exit at once);
 *   PA_DECODE_SORTED_GRID   the items that hold tokens, longest first (a
 *                           one-workgroup kernel orders them on the device
 *                           before the decode, in the workspace), taken
 *                           by a persistent grid (as many workgroups as fit
 *                           on the device): with partitions of 1024 tokens
 *                           or more each workgroup takes the next item of
 *                           the order from a counter when it finishes one;
 *                           with shorter partitions the order is dealt in
 *                           fixed snake rounds (round r of workgroup i:
 *                           entry r * workgroups + i, mirrored on odd
 *                           rounds);
 *   PA_DECODE_WORK_LIST     a persistent grid (as many workgroups as fit on
 *                           the device) walking the list of items that hold
 *                           tokens, which each workgroup builds in LDS.
 * A choice that does not apply (one pass; a list or order too large) falls
 * back to grid order.  The library's pick (0): the sorted grid for
 * partitions of 1024 tokens or more; below that, the work list for batches
 * of up to 64 sequences and the sorted grid for larger ones (each where it
 * fits, else the other, else grid order); except in a decode step's launches
 * (pa_decode_step*, pa_decode_order, and a decode with PA_DECODE_ORDERED),
 * which take the sorted grid wherever its order fits, their ordering riding
 * on the launch that writes the step's tokens.  The plan queries
 * (pa_decode_grid, pa_decode_work_list) give a step's grid when flags carry
 * PA_DECODE_ORDERED; pa_decode_workspace_size covers either. */
#define PA_DECODE_NO_WORK_LIST 16u
#define PA_DECODE_SORTED_GRID 32u
#define PA_DECODE_WORK_LIST 48u
#define PA_DECODE_GRID_MASK 48u
/* Bit 6: the workspace already holds this launch's item order: pa_decode_order
 * ran with the same arguments on the same stream after the workspace's last
 * use, so pa_decode / pa_decode_partitions (and the E4M3 forms) launch the
 * decode kernel alone.  Only meaningful where the grid is the sorted one
 * (pa_decode_grid); ignored elsewhere.  Single-query calls only:
 * pa_decode_mq* with num_queries > 1, pa_decode_step* and pa_decode_noalloc
 * give PA_ERR_UNSUPPORTED. */
#define PA_DECODE_ORDERED 64u

/*
 * pa_cache_write -- for every token i in [0, num_tokens) whose
 * slot_mapping[i] >= 0, with block = slot / block_size and o = slot %
 * block_size, copy k[i][h][e] into k_cache[block][h][o/4][e/X][o%4][e%X] and
 * v[i][h][e] into v_cache[block][h][o/4][e][o%4], for all kv heads h and dims
 * e, as raw bits.  Tokens with a negative slot are skipped (padding).  All other
 * cache bytes are left unchanged.
 *
 *   k, v            device, dtype, token i / head h / dim e at
 *                   k[i * k_token_stride + h * head_dim + e]; the heads of a
 *                   token are packed (stride head_dim), tokens may be strided
 *                   (k_token_stride >= num_kv_heads * head_dim, in elements)
 *   slot_mapping    device int64 [num_tokens]
 *   k_cache,v_cache device, dtype, layouts above
 *   dtype           pa_dtype of k, v and both caches (must match; F32, F16 or
 *                   BF16 -- E4M3 caches are written by pa_cache_write_fp8)
 *   head_dim        64, 128 or 256;  block_size: 8, 16, 32 or 64
 * Duplicate non-negative slots within one call race (undefined which wins).
 * num_tokens == 0 is a valid no-op.
 */
int pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                   void* v_cache, int64_t num_tokens, int64_t k_token_stride,
                   int64_t v_token_stride, int32_t num_kv_heads, int32_t head_dim,
                   int64_t num_blocks, int32_t block_size, int32_t dtype, void* stream);

/*
 * pa_cache_write_fp8 -- pa_cache_write into E4M3 caches ("vLLM Project Update"
 * talk, quantization update: an 8-bit floating-point KV cache).  The talk
 * fixes neither format nor scaling; here: OCP E4M3 with one scale per cache
 * tensor.  Element x of k (v), read as src_dtype, is stored as
 * e4m3(x / k_scale) (resp. v_scale): the quotient is the correctly rounded
 * fp32 division, then rounded to the nearest E4M3 value with ties to the even
 * significand; magnitudes beyond 448 (infinities too) saturate to +-448, NaN
 * stays NaN.  Layouts as above with X = 16 (one byte per element).
 *
 *   k, v            device, src_dtype (F32, F16 or BF16), as in pa_cache_write
 *   k_cache,v_cache device, E4M3 bytes
 *   k_scale,v_scale finite, > 0; a cache element stands for stored * scale
 * Other arguments, errors and races as pa_cache_write.
 */
int pa_cache_write_fp8(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                       void* v_cache, int64_t num_tokens, int64_t k_token_stride,
                       int64_t v_token_stride, int32_t num_kv_heads, int32_t head_dim,
                       int64_t num_blocks, int32_t block_size, int32_t src_dtype, float k_scale,
                       float v_scale, void* stream);

/*
 * pa_advance_step -- advance each sequence's decode state by one step on the
 * device, in place ("[core] Multi Step Scheduling" pull request, review
 * thread on ops.advance_step: between steps of a multi-step run the GPU
 * updates next input tokens, positions, sequence lengths and slots from the
 * sampled ids, block tables and block size).  For i < num_queries:
 *     input_tokens[i]    = sampled_token_ids[i]
 *     input_positions[i] = input_positions[i] + 1            (call it p)
 *     seq_lens[i]        = p + 1
 *     slot_mapping[i]    = block_tables[i][p / block_size] * block_size
 *                          + p % block_size
 *                          (-1 when p / block_size >= max_blocks_per_seq or the
 *                          table entry is negative: the block was not allocated
 *                          ahead, and pa_cache_write skips the token)
 * and for num_queries <= i < num_seqs (padding rows) slot_mapping[i] = -1,
 * everything else untouched.  All pointers are device pointers:
 * input_tokens, input_positions, slot_mapping int64 [num_seqs];
 * sampled_token_ids int64 [num_queries]; seq_lens int32 [num_seqs];
 * block_tables int32 [num_seqs][max_blocks_per_seq] (read only).
 * Callers allocate the blocks of the coming steps before launching them.
 */
int pa_advance_step(int32_t num_seqs, int32_t num_queries, int32_t block_size,
                    int64_t* input_tokens, const int64_t* sampled_token_ids,
                    int64_t* input_positions, int32_t* seq_lens, int64_t* slot_mapping,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, void* stream);

/*
 * pa_decode -- out[b][hq][:] = sum_t softmax_t(scale * q[b][hq] . K_t) V_t
 * over the logical positions t in [0, context_lens[b]) of sequence b, where
 * position t is found in physical block block_tables[b][t / block_size] at
 * offset t % block_size, and query head hq reads kv head
 * hq / (num_q_heads / num_kv_heads).
 *
 *   out            device [num_seqs][num_q_heads][head_dim], out_dtype
 *                  (f32, or the kv dtype)
 *   q              device [num_seqs][num_q_heads][head_dim], q_dtype
 *                  (f32, or the kv dtype)
 *   k_cache,v_cache device, kv_dtype, layouts above, num_blocks blocks
 *   block_tables   device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens   device int32 [num_seqs]; 1 <= L <= max_blocks_per_seq *
 *                  block_size (a sequence with L == 0 gets an all-zero row)
 *   scale          softmax scale (typically 1/sqrt(head_dim))
 *   block_size     8, 16, 32 or 64
 *   partition_size 0: the library picks (see pa_decode_partition_size);
 *                  > 0: positions are processed in partitions of this many
 *                  tokens (a multiple of block_size), merged by a
 *                  log-sum-exp reduction; a value >= max_blocks_per_seq *
 *                  block_size means one pass per (sequence, kv head) with no
 *                  reduction and no workspace; at most 65535 partitions of
 *                  max_blocks_per_seq * block_size (PA_ERR_SHAPE beyond)
 *   head_dim       64 or 128;  num_q_heads % num_kv_heads == 0
 *   workspace      device scratch of at least pa_decode_workspace_size(...)
 *                  bytes for the same arguments (may be NULL when that is 0),
 *                  16-byte aligned; its contents on entry do not matter.
 *                  Calls that may run at the same time need distinct
 *                  workspaces.
 *   flags          PA_DECODE_AUTO, or a PA_DECODE_FORCE_* kernel choice OR-ed
 *                  with a PA_DECODE_WAVES_* split and a grid choice
 *                  (PA_DECODE_NO_WORK_LIST, _SORTED_GRID or _WORK_LIST; each
 *                  part may be 0 = library picks); other bits set, or both
 *                  kernel bits, give PA_ERR_UNSUPPORTED
 * The result does not depend on partition_size, the kernel family or the
 * waves per item beyond floating-point rounding (fp32 accumulation
 * throughout).
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              int32_t block_size, int32_t partition_size, int32_t num_seqs, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
              int32_t max_blocks_per_seq, int32_t q_dtype, int32_t kv_dtype, int32_t out_dtype,
              void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * pa_decode in its two phases, for callers that schedule them separately
 * (e.g. to time them, or to merge partition results gathered from elsewhere).
 * Both take exactly pa_decode's arguments and must be given the same ones.
 *
 * pa_decode_partitions: attention over each partition of partition_size
 *   tokens; writes, per (sequence, q head, partition), the running max m
 *   (log2 domain), the sum l and the unnormalised output vector to the
 *   workspace, and writes `out` directly for sequences that fit one partition.
 * pa_decode_merge: for sequences with more than one partition, merges the
 *   workspace entries by log-sum-exp into `out` ("vLLM Project Update" talk,
 *   second PagedAttention kernel, likened there to flash decoding).  Launches
 *   nothing when every sequence fits one partition.
 * pa_decode(...) == pa_decode_partitions(...) followed by pa_decode_merge(...)
 * on the same stream.
 */
int pa_decode_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         int32_t block_size, int32_t partition_size, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int64_t num_blocks, int32_t max_blocks_per_seq, int32_t q_dtype,
                         int32_t kv_dtype, int32_t out_dtype, void* workspace,
                         size_t workspace_bytes, uint32_t flags, void* stream);
int pa_decode_merge(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                    int32_t block_size, int32_t partition_size, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int64_t num_blocks, int32_t max_blocks_per_seq, int32_t q_dtype,
                    int32_t kv_dtype, int32_t out_dtype, void* workspace, size_t workspace_bytes,
                    uint32_t flags, void* stream);

/*
 * pa_decode_step / pa_decode_step_partitions -- one decode step: pa_cache_write
 * of the step's new tokens (k, v, slot_mapping, num_tokens and the strides as
 * there, kv_dtype the cache dtype, 16-bit or fp32) followed by pa_decode (or
 * pa_decode_partitions) over the updated caches, with the same arguments and
 * results as those calls made one after the other on `stream`.  Where the
 * decode orders its work items on the device (PA_DECODE_SORTED_GRID), the
 * write runs in the same launch as the ordering, saving a launch per step.
 * Nothing is launched unless both the write's and the decode's arguments
 * validate (errors as either call).  E4M3 caches: PA_ERR_DTYPE.
 */
int pa_decode_step(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                   int64_t k_token_stride, int64_t v_token_stride, void* out, const void* q,
                   void* k_cache, void* v_cache, const int32_t* block_tables,
                   const int32_t* context_lens, float scale, int32_t block_size,
                   int32_t partition_size, int32_t num_seqs, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                   int32_t max_blocks_per_seq, int32_t q_dtype, int32_t kv_dtype,
                   int32_t out_dtype, void* workspace, size_t workspace_bytes, uint32_t flags,
                   void* stream);
int pa_decode_step_partitions(const void* k, const void* v, const int64_t* slot_mapping,
                              int64_t num_tokens, int64_t k_token_stride, int64_t v_token_stride,
                              void* out, const void* q, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, int32_t block_size, int32_t partition_size,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t q_dtype, int32_t kv_dtype, int32_t out_dtype,
                              void* workspace, size_t workspace_bytes, uint32_t flags,
                              void* stream);

/*
 * pa_decode_order -- the part of a decode step that precedes the decode
 * kernel, in one launch: pa_cache_write of the step's new tokens (k, v,
 * slot_mapping, num_tokens and the strides as in pa_decode_step; num_tokens =
 * 0 for none) and, where the decode runs on the sorted grid, the ordering of
 * its work items into the workspace.  A following pa_decode_partitions (or
 * pa_decode, or the E4M3 forms) with the same arguments and flags |
 * PA_DECODE_ORDERED then launches only the decode kernel; the results equal
 * pa_decode_step's bit for bit.  Callers that time or schedule the decode
 * kernel on its own use this split.  kv_dtype E4M3 is accepted with
 * num_tokens = 0 only (its write needs scales: pa_cache_write_fp8).
 * Arguments, workspace and errors as pa_decode_step.
 */
int pa_decode_order(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                    int64_t k_token_stride, int64_t v_token_stride, void* out, const void* q,
                    void* k_cache, void* v_cache, const int32_t* block_tables,
                    const int32_t* context_lens, float scale, int32_t block_size,
                    int32_t partition_size, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                    int32_t max_blocks_per_seq, int32_t q_dtype, int32_t kv_dtype,
                    int32_t out_dtype, void* workspace, size_t workspace_bytes, uint32_t flags,
                    void* stream);

/*
 * pa_decode_order_fp8 -- pa_decode_order for E4M3 caches: the quantizing
 * write of the step's new tokens (as pa_cache_write_fp8: source rows of
 * src_dtype f32, f16 or bf16, stored value e4m3(x / k_scale) and
 * e4m3(x / v_scale)) and the ordering of the decode's items in one launch.
 * A following pa_decode_fp8_partitions (or pa_decode_fp8) with the same
 * arguments and flags | PA_DECODE_ORDERED launches the decode kernel alone;
 * caches and results equal pa_cache_write_fp8 followed by pa_decode_fp8 bit
 * for bit.  The caches are E4M3 (kv_dtype is implied); k_scale and v_scale
 * are the caches' scales, as the decode takes them.  Errors as
 * pa_cache_write_fp8 for the write's arguments, as pa_decode_fp8 for the rest.
 */
int pa_decode_order_fp8(const void* k, const void* v, const int64_t* slot_mapping,
                        int64_t num_tokens, int64_t k_token_stride, int64_t v_token_stride,
                        int32_t src_dtype, float k_scale, float v_scale, void* out,
                        const void* q, void* k_cache, void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens, float scale,
                        int32_t block_size, int32_t partition_size, int32_t num_seqs,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int64_t num_blocks, int32_t max_blocks_per_seq, int32_t q_dtype,
                        int32_t out_dtype, void* workspace, size_t workspace_bytes,
                        uint32_t flags, void* stream);

/*
 * pa_decode_mq / pa_decode_mq_partitions / pa_decode_mq_merge -- decode of
 * several query tokens per sequence ("vLLM Project Update" talk, roadmap:
 * multi-query attention kernels for speculative decoding, which score the
 * proposed tokens of a sequence in one pass).  q and out are
 * [num_seqs][num_queries][num_q_heads][head_dim]; context_lens[b] counts all
 * of sequence b's tokens including its num_queries new ones, whose K/V are
 * already in the caches: query i sits at position context_lens[b] -
 * num_queries + i and attends to positions 0 .. its own (causal among the
 * new tokens):
 *   out[b][i][hq] = softmax_t(scale * q[b][i][hq] . k_t) . v_t,
 *                   t = 0 .. context_lens[b] - num_queries + i.
 * A query whose position would be negative (context_lens[b] < num_queries)
 * gets a zero row.  num_queries = 1 is pa_decode.  The (query, head) rows of
 * a kv head form the matrix cores' columns: num_queries * heads_per_item <= 32
 * (instantiated widths 1-8, 10, 12, 16 on one 16-column tile, 24 and 32 on
 * two tiles sharing each key/value load); the vector-ALU kernel takes up to 8.
 *   num_queries    1 .. 16
 *   kv_dtype       any cache dtype; k_scale, v_scale as in pa_decode_fp8 (pass
 *                  1 for the unscaled types)
 *   workspace      pa_decode_workspace_size(num_seqs * num_queries, ...) bytes;
 *                  the other plan queries (partition size, waves, grid) also
 *                  take num_seqs * num_queries for a multi-query decode
 * Other arguments, errors and the phase split as pa_decode.
 */
int pa_decode_mq(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                 float k_scale, float v_scale, int32_t block_size, int32_t partition_size,
                 int32_t num_seqs, int32_t num_queries, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                 int32_t max_blocks_per_seq, int32_t q_dtype, int32_t kv_dtype,
                 int32_t out_dtype, void* workspace, size_t workspace_bytes, uint32_t flags,
                 void* stream);
int pa_decode_mq_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            float scale, float k_scale, float v_scale, int32_t block_size,
                            int32_t partition_size, int32_t num_seqs, int32_t num_queries,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int64_t num_blocks, int32_t max_blocks_per_seq, int32_t q_dtype,
                            int32_t kv_dtype, int32_t out_dtype, void* workspace,
                            size_t workspace_bytes, uint32_t flags, void* stream);
int pa_decode_mq_merge(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, float scale,
                       float k_scale, float v_scale, int32_t block_size, int32_t partition_size,
                       int32_t num_seqs, int32_t num_queries, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                       int32_t max_blocks_per_seq, int32_t q_dtype, int32_t kv_dtype,
                       int32_t out_dtype, void* workspace, size_t workspace_bytes,
                       uint32_t flags, void* stream);

/*
 * The decode kernel family pa_decode_mq runs with num_queries query tokens
 * per sequence (as pa_decode_kernel, which is the num_queries = 1 case);
 * PA_ERR_UNSUPPORTED when no kernel holds the query rows.
 */
int32_t pa_decode_mq_kernel(int32_t num_queries, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t q_dtype, int32_t kv_dtype, uint32_t flags);

/*
 * pa_decode_fp8 / pa_decode_fp8_partitions -- pa_decode / pa_decode_partitions
 * over E4M3 caches written by pa_cache_write_fp8: the attention of each query
 * over the cache elements stored * k_scale (keys) and stored * v_scale
 * (values).  pa_decode and pa_decode_partitions reject E4M3 caches
 * (PA_ERR_DTYPE); the merge phase is pa_decode_merge with kv_dtype
 * PA_DTYPE_FP8_E4M3.
 *   q_dtype        F32, F16 or BF16 (BF16 runs on the matrix cores for GQA
 *                  groups; the E4M3 values widen exactly to bfloat16)
 *   out_dtype      F32 or q_dtype
 *   k_scale,v_scale the scales the caches were written with (finite, > 0)
 * All other arguments, the workspace and errors as pa_decode with kv_dtype
 * PA_DTYPE_FP8_E4M3 (use it in the plan queries and the workspace size).
 */
int pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, float scale,
                  float k_scale, float v_scale, int32_t block_size, int32_t partition_size,
                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int64_t num_blocks, int32_t max_blocks_per_seq, int32_t q_dtype,
                  int32_t out_dtype, void* workspace, size_t workspace_bytes, uint32_t flags,
                  void* stream);
int pa_decode_fp8_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             float scale, float k_scale, float v_scale, int32_t block_size,
                             int32_t partition_size, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                             int32_t max_blocks_per_seq, int32_t q_dtype, int32_t out_dtype,
                             void* workspace, size_t workspace_bytes, uint32_t flags,
                             void* stream);

/*
 * The partition size pa_decode uses when called with partition_size == 0 and
 * the same arguments (a pure function of them; no device query).  Returns a
 * negative pa_status for invalid arguments.  Where this size is 2048 tokens or
 * more and the launch runs on the sorted grid (pa_decode_grid) with one query
 * per sequence, the launch refines it on the device from the actual context
 * lengths to half, the same or twice this size (the ordering kernel decides;
 * the result is then that of pa_decode with the refined size passed
 * explicitly), and pa_decode_workspace_size(partition_size = 0) covers the
 * half.  The refinement: a batch whose longest context is at most twice the
 * mean keeps the size; otherwise the largest of the three that is at most a
 * third of one compute unit's share of the token x kv-head work, twice only
 * while the longest context still spans two partitions and twice <= 8192.
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int32_t kv_dtype, uint32_t flags);

/*
 * The partition the last partition_size == 0 launch with these arguments used
 * on `workspace` (the workspace it was given): the device's refinement where
 * the launch refines (see pa_decode_partition_size), read back from the
 * workspace with a copy on `stream` that the call waits for (a diagnostic, not
 * for a hot loop), else pa_decode_partition_size's value.  Meaningful after
 * such a launch on the workspace; a word holding none of the three candidates
 * (p / 2, p, 2p), as a zeroed workspace does, reads as pa_decode_partition_size's
 * value.  Negative pa_status for invalid arguments or a workspace too small for
 * the launch.
 */
int32_t pa_decode_partition_used(const void* workspace, size_t workspace_bytes,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int32_t kv_dtype, uint32_t flags,
                                 void* stream);

/*
 * The decode kernel family pa_decode runs for these arguments:
 * PA_DECODE_FORCE_VALU (1) or PA_DECODE_FORCE_MFMA (2); a negative pa_status
 * for an unsupported combination.  The waves bits of flags are validated but
 * do not affect the family.
 */
int32_t pa_decode_kernel(int32_t num_q_heads, int32_t num_kv_heads, int32_t q_dtype,
                         int32_t kv_dtype, uint32_t flags);

/*
 * The waves per work item (1, 2 or 4) pa_decode uses for these arguments
 * (partition_size as passed to pa_decode, 0 allowed); a negative pa_status
 * for invalid arguments.  A pure function of the arguments.
 */
int32_t pa_decode_waves(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                        int32_t partition_size, int32_t q_dtype, int32_t kv_dtype,
                        uint32_t flags);

/*
 * 1 when pa_decode runs these arguments on a persistent grid over the list of
 * (sequence, partition) items that hold tokens, 0 when it launches one
 * workgroup per possible item; a negative pa_status for invalid arguments.
 */
int32_t pa_decode_work_list(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                            int32_t partition_size, int32_t q_dtype, int32_t kv_dtype,
                            uint32_t flags);

/*
 * The grid pa_decode runs these arguments on: PA_DECODE_NO_WORK_LIST (one
 * workgroup per possible item in grid order; also every one-pass launch),
 * PA_DECODE_SORTED_GRID or PA_DECODE_WORK_LIST; a negative pa_status for
 * invalid arguments.  For pa_decode_mq pass num_seqs * num_queries.
 */
int32_t pa_decode_grid(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                       int32_t partition_size, int32_t q_dtype, int32_t kv_dtype, uint32_t flags);

/*
 * Workspace bytes pa_decode needs for these arguments (partition_size as
 * passed to pa_decode, 0 allowed: then counted for the smallest partition the
 * launch may refine to, see pa_decode_partition_size): per (sequence, q head,
 * partition) the running max and sum, then the partial output vector, each
 * region 256-byte aligned, then on the sorted grid the item order.  0 when a
 * single pass suffices.  Returns 0 for invalid arguments as well; pa_decode reports those.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t partition_size, int32_t kv_dtype, uint32_t flags);

/*
 * pa_check_tables / pa_check_slots -- opt-in debug checks of the ids the hot
 * path takes on trust ("[core] Multi Step Scheduling" pull request: the
 * per-step slot_mapping and block_tables are the scheduler's, and a broken
 * one surfaced there only as a failed assertion after the merge).  The
 * decode and write kernels never read or write out of bounds: a block-table
 * entry of a context outside [0, num_blocks) is clamped into the pool, a
 * context length beyond max_blocks_per_seq * block_size is cut to it (a
 * negative one is an empty sequence), and a slot >= num_blocks * block_size
 * is dropped.  Such a call returns a wrong answer silently.  These checks
 * evaluate exactly those conditions on the device and OR one bit per kind
 * into *status:
 *   PA_CHECK_CONTEXT_LEN  some context_lens[b] < 0 or > max_blocks_per_seq *
 *                         block_size
 *   PA_CHECK_BLOCK_ID     some block_tables[b][j], j < ceil(L_b / block_size)
 *                         (L_b as the kernels cut it), outside [0, num_blocks)
 *   PA_CHECK_SLOT         some slot_mapping[i] >= num_blocks * block_size
 * Entries past a context and negative slots (padding) are not errors.
 * Clean arguments leave *status unchanged; the caller zeroes it before and
 * reads it after (both on `stream`).  Nothing is allocated.
 *   block_tables, context_lens, slot_mapping: device, as in pa_decode /
 *   pa_cache_write; status: device uint32, 4-byte aligned.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (negative sizes, block_size < 1);
 * num_seqs == 0 or num_tokens == 0 is a valid no-op.
 */
#define PA_CHECK_CONTEXT_LEN 1u
#define PA_CHECK_BLOCK_ID 2u
#define PA_CHECK_SLOT 4u
int pa_check_tables(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks,
                    uint32_t* status, void* stream);
int pa_check_slots(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                   int32_t block_size, uint32_t* status, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments, results and kernels as pa_decode with
 * flags, minus the workspace, which is instead a static device array of
 * PA_SCRATCH_BYTES inside the library.  Nothing is allocated by the call (no
 * hipMalloc, no allocating library routine); each GPU the library runs on
 * holds its own copy of the array until the process ends (its address is
 * looked up once per device, on the first call made with that device
 * current).  Contents left by an earlier call do not matter: what must start
 * at zero is cleared by the call's own kernels.
 *   Limit: pa_decode_workspace_size(...) for the same arguments must be at
 *   most PA_SCRATCH_BYTES, else PA_ERR_SCRATCH and nothing is launched (one
 *   pass needs no workspace and is always accepted).
 *   Races: every call on a GPU shares that GPU's array, so two calls that may
 *   run at the same time on one GPU (different streams, or host threads) race
 *   on it; serialise them (one stream) or use pa_decode with workspaces of
 *   their own.
 * E4M3 caches: PA_ERR_DTYPE (as pa_decode).
 */
#define PA_SCRATCH_BYTES (64u << 20) /* 64 MiB */
int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t partition_size, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int64_t num_blocks, int32_t max_blocks_per_seq, int32_t q_dtype,
                      int32_t kv_dtype, int32_t out_dtype, uint32_t flags, void* stream);

/* Static, library-owned text for a pa_status value. */
const char* pa_status_string(int32_t status);

/* ABI version of this header (incremented on incompatible changes). */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
