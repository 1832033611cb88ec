// pa_launch.hpp -- host-side launch interface between the C ABI (pa_api.cpp)
// and the kernel translation units.  Arguments are validated before any of
// these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct CacheWriteArgs {
  const void* k;
  const void* v;
  const int64_t* slots;
  void* k_cache;
  void* v_cache;
  int64_t num_tokens;
  int64_t k_stride;  // elements between tokens of k
  int64_t v_stride;
  int64_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t elem_bytes;  // of the cache: 1 for E4M3 (a quantizing write from src_dtype)
  float k_scale;  // E4M3 caches: stored value = x / scale
  float v_scale;
  int32_t src_dtype;  // E4M3 caches: the source rows' pa_dtype (f32, f16 or bf16)
};

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);
// Quantizing write of f32 / f16 / bf16 rows (src_dtype) into E4M3 caches.
hipError_t launch_cache_write_fp8(const CacheWriteArgs& a, int src_dtype, hipStream_t stream);

// Everything a decode kernel needs; passed by value as the kernel argument.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_ml;   // [B][Hq][P][2] running max (log2 domain) and sum
  float* ws_acc;  // [B][Hq][P][D] unnormalised partial outputs
  float scale_log2;  // scale * k_scale * log2(e)
  float v_scale;     // cache value = stored value * v_scale (1 for the unscaled types)
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;       // num_q_heads / num_kv_heads
  int32_t heads_per_item;  // q heads handled by one work item
  int32_t num_queries;     // query tokens per sequence: q, out are [B][Q][Hq][d]; an item
                           // handles Q x heads_per_item rows (the kernels' template G)
  int32_t block_size;
  int32_t log2_block_size;
  int32_t max_blocks_per_seq;
  int32_t partition_size;  // tokens per partition
  int32_t max_partitions;  // ceil(max_blocks_per_seq * block_size / partition_size)
  int32_t q_dtype;
  int32_t out_dtype;
  int32_t waves;  // waves per work item (1, 2 or 4): they split its chunks
  int32_t list_ints;  // LDS ints of the work list (persistent grid), 0: one workgroup per item
  // One workgroup per possible item: NULL, grid order (sequence, kv head, head
  // chunk fastest, partitions last to first); else workgroup i (linear over
  // the grid) takes entry i / (items per sequence) of this longest-first list
  // of b * max_partitions + partition (-1: nothing left).
  const int32_t* order;
  // With an order: NULL, one workgroup per grid slot; else a persistent grid
  // deals the order dynamically: workgroup i starts with item i, then takes
  // gridDim.x + (the value of this counter, incremented) until the order runs
  // out.  The ordering kernel zeroes it.
  int32_t* order_ctr;
  // With an order and no counter: 0, one workgroup per grid slot; 1, a
  // persistent grid deals the order statically, in snake rounds: round r of
  // workgroup i takes entry r * gridDim.x + i, mirrored (gridDim.x - 1 - i)
  // on odd rounds, until the order runs out.
  int32_t order_static;
  // Where the ordering kernel picks the partition (part_pick), two words it
  // writes for the launches that follow: [0] the partition, [1] the number of
  // entries in the order (a ticket past it ends a workgroup without reading
  // the entry); else NULL.
  int32_t* part_dev;
  // 1: the library's own partition choice (partition_size = 0), refined by the
  // ordering kernel from the actual context lengths -- partition_size / 2,
  // partition_size or 2 * partition_size (max_partitions is counted for the
  // half); the decode and merge kernels read it (partition_of).  0:
  // partition_size is the partition.
  int32_t part_pick;
  int32_t num_cus;  // compute units of the device (the ordering kernel's choice)
};

// The partition a launch uses: the one the ordering kernel picked, when it
// picks, else partition_size.  A stored value outside the three the ordering
// kernel may pick (an ordered launch whose ordering never ran) falls back to
// partition_size, so every partition index stays below max_partitions.
template <class Args>  // DecodeArgs in any address space (kernel arguments included)
__device__ __forceinline__ int partition_of(Args& a) {
  const int p = a.partition_size;
  if (!a.part_dev || !a.part_pick) return p;
  // the kernel writes the workspace, so the compiler loads the word with a
  // vector load; readfirstlane makes it (and everything derived from it)
  // wave-uniform again (measured: 21% slower decode without)
  const int d = __builtin_amdgcn_readfirstlane(*a.part_dev);
  return (d == p / 2 || d == 2 * p) ? d : p;
}

// LDS ints a workgroup needs for the work list of a persistent launch.
__host__ __device__ inline int work_list_lds_ints(int num_seqs, int max_partitions) {
  return 4 * (max_partitions + 2) + 2 * num_seqs;
}

// Launches a decode kernel: with a work list, a persistent grid of as many
// workgroups as fit on the device at once (at most one per possible item);
// without, grid (items_x, max_partitions).  `lds` is the dynamic LDS per
// workgroup.
hipError_t launch_decode_grid(const void* kernel, const DecodeArgs& a, int64_t items_x,
                              size_t lds, hipStream_t s);

// Writes the longest-first item order of a launch (one workgroup) into
// `order` [num_seqs * max_partitions]; with `write` (16-bit or fp32 caches),
// the same launch also runs that cache write.
hipError_t launch_decode_order(const DecodeArgs& a, int32_t* order, const CacheWriteArgs* write,
                               hipStream_t s);

// Vector-ALU decode kernel: any kv dtype, head_dim 64/128, 1..8 q heads per
// work item.  grid = (num_seqs * num_kv_heads * head_chunks, max_partitions),
// a.waves waves per workgroup.
hipError_t launch_decode_valu(const DecodeArgs& a, int kv_dtype, int head_dim, hipStream_t s);

// Matrix-core decode kernel: f16/bf16 KV with q in the same dtype, head_dim
// 64/128, up to 16 q heads per work item (see mfma_supports_heads).
hipError_t launch_decode_mfma(const DecodeArgs& a, int kv_dtype, int head_dim, hipStream_t s);
bool mfma_supports_heads(int heads_per_item);

// Log-sum-exp merge of the partitions of every (sequence, q head) that has
// more than one.
hipError_t launch_decode_reduce(const DecodeArgs& a, int head_dim, hipStream_t s);

struct AdvanceArgs {
  int64_t* input_tokens;
  const int64_t* sampled_token_ids;
  int64_t* input_positions;
  int32_t* seq_lens;
  int64_t* slot_mapping;
  const int32_t* block_tables;
  int32_t num_seqs;
  int32_t num_queries;
  int32_t block_size;
  int32_t max_blocks_per_seq;
};

// One thread per sequence: next token, position, length and slot.
hipError_t launch_advance_step(const AdvanceArgs& a, hipStream_t s);

// The precondition checks (check_ids.hip): OR PA_CHECK_* bits into *status.
hipError_t launch_check_tables(const int32_t* block_tables, const int32_t* context_lens,
                               int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                               int64_t num_blocks, uint32_t* status, hipStream_t s);
hipError_t launch_check_slots(const int64_t* slots, int64_t num_tokens, int64_t capacity,
                              uint32_t* status, hipStream_t s);

}  // namespace pa
