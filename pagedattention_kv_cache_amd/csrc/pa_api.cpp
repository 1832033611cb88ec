// pa_api.cpp -- the C ABI declared in include/pa.h: argument validation,
// partition-size policy, workspace sizing and kernel launches on the caller's
// stream.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "pa.h"
#include "pa_launch.hpp"

namespace {

constexpr int32_t kAbiVersion = 1;

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_DTYPE_F32: return 4;
    case PA_DTYPE_F16: return 2;
    case PA_DTYPE_BF16: return 2;
    case PA_DTYPE_FP8_E4M3: return 1;
    default: return 0;
  }
}

bool valid_block_size(int32_t bs) { return bs == 8 || bs == 16 || bs == 32 || bs == 64; }

int log2_exact(int32_t v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest divisor of g that is <= cap: the q heads one work item handles
// (0 when cap < 1).
int32_t heads_per_item(int32_t g, int32_t cap) {
  for (int32_t h = cap < g ? cap : g; h >= 1; --h)
    if (g % h == 0) return h;
  return 0;
}

// Matrix-core items: the q heads per item h, the largest divisor of g whose Q
// x h columns (Q query tokens per sequence) fit one or two 16-column tiles
// with an instantiated width; 0 when there is none.  Two tiles share every
// key and value load.
int32_t mfma_heads_per_item(int32_t g, int32_t num_queries) {
  for (int32_t h = g < 32 ? g : 32; h >= 1; --h)
    if (g % h == 0 && num_queries * h <= 32 && pa::mfma_supports_heads(num_queries * h))
      return h;
  return 0;
}

// The vector-ALU kernel's items: up to 8 rows (Q x h).
int32_t valu_heads_per_item(int32_t g, int32_t num_queries) {
  return heads_per_item(g, 8 / num_queries);
}

// Queries in the cache dtype or fp32; with E4M3 caches any of f32, f16, bf16.
bool valid_q_dtype(int32_t q_dtype, int32_t kv_dtype) {
  if (q_dtype != PA_DTYPE_F32 && q_dtype != PA_DTYPE_F16 && q_dtype != PA_DTYPE_BF16)
    return false;
  return q_dtype == kv_dtype || q_dtype == PA_DTYPE_F32 || kv_dtype == PA_DTYPE_FP8_E4M3;
}

// Outputs in fp32 or in the 16-bit type of the attention (the cache's, or the
// queries' for E4M3 caches).
bool valid_out_dtype(int32_t out_dtype, int32_t q_dtype, int32_t kv_dtype) {
  if (out_dtype == PA_DTYPE_F32) return true;
  return out_dtype == (kv_dtype == PA_DTYPE_FP8_E4M3 ? q_dtype : kv_dtype);
}

// The matrix-core kernel multiplies 16-bit operands: 16-bit caches queried in
// their own dtype, or E4M3 caches (widened exactly to bfloat16) with bfloat16
// queries.
bool mfma_eligible(int32_t kv_dtype, int32_t q_dtype) {
  if (kv_dtype == PA_DTYPE_FP8_E4M3) return q_dtype == PA_DTYPE_BF16;
  return kv_dtype != PA_DTYPE_F32 && q_dtype == kv_dtype;
}

// Kernel family.  The matrix-core kernel takes every item whose dtypes it
// handles, single-row items included: the decode is bound by the K/V stream,
// and the matrix-core kernel's loads (buffer loads of 16-byte key pieces and
// 8-byte value quads off a scalar tile base) stream faster than the
// vector-ALU kernel's even when 15 of the tile's 16 columns are idle.
// Measured, MHA f16 batches (one q head per kv head): uniform lengths 211.5
// -> 192.1 us, skewed batch 51.4 -> 46.4 us.  fp32 caches, and queries in
// another dtype than a 16-bit cache, run on the vector ALUs.  Returns 0
// (neither) when no kernel can hold the Q x h rows.
int32_t pick_kernel(uint32_t flags, int32_t kv_dtype, int32_t q_dtype, int32_t group,
                    int32_t num_queries) {
  const bool mfma_ok =
      mfma_eligible(kv_dtype, q_dtype) && mfma_heads_per_item(group, num_queries) > 0;
  const bool valu_ok = valu_heads_per_item(group, num_queries) > 0;
  const uint32_t kernel = flags & PA_DECODE_KERNEL_MASK;
  if (kernel == PA_DECODE_FORCE_MFMA) return mfma_ok ? PA_DECODE_FORCE_MFMA : 0;
  if (kernel == PA_DECODE_FORCE_VALU) return valu_ok ? PA_DECODE_FORCE_VALU : 0;
  if (mfma_ok) return PA_DECODE_FORCE_MFMA;
  return valu_ok ? PA_DECODE_FORCE_VALU : 0;
}

// Flag bits this library knows, with a valid kernel choice.
bool valid_flags(uint32_t flags) {
  if (flags & ~(PA_DECODE_KERNEL_MASK | PA_DECODE_WAVES_MASK | PA_DECODE_GRID_MASK |
                PA_DECODE_ORDERED))
    return false;
  return (flags & PA_DECODE_KERNEL_MASK) != PA_DECODE_KERNEL_MASK;
}

bool forces_mfma(uint32_t flags) {
  return (flags & PA_DECODE_KERNEL_MASK) == PA_DECODE_FORCE_MFMA;
}

struct DecodeShape {
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  int32_t kv_dtype;
  uint32_t flags;
};

int check_shape(const DecodeShape& s) {
  if (s.num_seqs < 0 || s.num_q_heads <= 0 || s.num_kv_heads <= 0 || s.max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (s.num_q_heads % s.num_kv_heads != 0) return PA_ERR_SHAPE;
  if (!elem_bytes(s.kv_dtype)) return PA_ERR_DTYPE;
  if (s.head_dim != 64 && s.head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!valid_block_size(s.block_size)) return PA_ERR_UNSUPPORTED;
  if ((int64_t)s.max_blocks_per_seq * s.block_size > (int64_t)1 << 30) return PA_ERR_SHAPE;
  if (!valid_flags(s.flags)) return PA_ERR_UNSUPPORTED;
  if (forces_mfma(s.flags) && s.kv_dtype == PA_DTYPE_F32) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Partition policy for partition_size == 0.
//  - Mixed lengths: about a quarter of the longest context the block table can
//    hold, as a power of two in [1024, 8192] tokens, so the longest sequence
//    spreads over four or more items (16 waves) while items stay long enough
//    to amortise their start-up (context length, block-id window and first
//    chunk are dependent loads before a wave streams) and the merge stays near
//    1% of the KV bytes.
//  - Small batches: halved (down to 512) until the launch has at least one
//    (sequence, kv head, partition) item per compute unit of the device (256).
// Measured (decode kernel, best power of two in parentheses): GQA lognormal
// batch 2048 (2048), MHA batch of <= 2048 tokens 1024 (1024), 64 x 4k-32k
// contexts 8192 (8192), 4 x 32k 4096 (4096), 1 x 32k 1024 (1024; 4096 was
// 1.6x slower), 1 x 4k 512 (512), 16 x 16k 4096 (8192, 1.6% faster).  One
// pass when the longest context fits a partition.
constexpr int64_t kItemsTarget = 256;

int32_t pick_partition(const DecodeShape& s) {
  const int64_t max_ctx = (int64_t)s.max_blocks_per_seq * s.block_size;
  int64_t p = 1024;
  while (p < 8192 && p * 4 < max_ctx) p *= 2;
  const int64_t seq_heads = (int64_t)s.num_seqs * s.num_kv_heads;
  while (p > 512 && seq_heads * ((max_ctx + p - 1) / p) < kItemsTarget) p /= 2;
  if (p % s.block_size) p = ((p + s.block_size - 1) / s.block_size) * s.block_size;
  if (max_ctx <= p) return (int32_t)max_ctx;  // one pass
  return (int32_t)p;
}

int64_t n_partitions(const DecodeShape& s, int32_t p) {
  const int64_t max_ctx = (int64_t)s.max_blocks_per_seq * s.block_size;
  return (max_ctx + p - 1) / p;
}

// Waves per work item.  An explicit PA_DECODE_WAVES_* choice wins; otherwise
// 4 for partitions of 1024 tokens or more, 2 from 256 tokens, else 1:
// splitting shortens the longest items, while a wave with few chunks spends
// too much of its time starting up and merging.  Measured (decode kernel,
// us): 512-token partitions, 4 -> 2 waves: skewed batch 44.5 -> 43.4 (sorted
// grid) and 42.0 -> 40.0 (work list), GQA lognormal batch 306.9 -> 301.1
// (sorted), MHA uniform batch 189.1 -> 188.7 (work list); 256-token
// partitions, MHA batch, 1 -> 2 waves: 197.5 -> 191.2; at 1024 tokens and
// more (GQA, long contexts) 4 waves stay best.
int32_t pick_waves(const DecodeShape& s, int32_t p) {
  switch (s.flags & PA_DECODE_WAVES_MASK) {
    case PA_DECODE_WAVES_1: return 1;
    case PA_DECODE_WAVES_2: return 2;
    case PA_DECODE_WAVES_4: return 4;
    default: break;
  }
  if (p >= 1024) return 4;
  return p >= 256 ? 2 : 1;
}

// Largest work list a workgroup builds in LDS (ints); beyond it, one
// workgroup per possible item.
constexpr int kMaxListInts = 4096;

// Largest order list (num_seqs * max_partitions entries) of a sorted grid.
constexpr int64_t kMaxOrder = 65536;

enum GridMode { kGridNatural = 0, kGridSorted = 1, kGridList = 2 };

// A sorted grid with partitions of at least this many tokens runs persistent:
// as many workgroups as fit on the device, each taking its next item from a
// counter when it finishes one.  Measured (decode kernel, sorted grid ->
// persistent): 4 x 2048-token partitions (GQA lognormal batch) 273 -> 266 us,
// 9 x 4096 (long contexts) 758 -> 747 us; but 512-token partitions lose (MHA
// batch 206 -> 206, skewed batch 48.7 -> 53.5 us): the counter's round trip
// is paid once per item, and short items are many.
constexpr int32_t kPersistentOrderMin = 1024;

// Below that, a sorted grid is still persistent, but deals the order in fixed
// snake rounds (no counter): one workgroup per possible item launched, on a
// batch of uneven lengths, thousands of empty workgroups that each read their
// order entry before exiting.  Measured (decode kernel incl. ordering, us,
// one workgroup per possible item -> static deal, two runs each): skewed
// batch at 512-token partitions 47.3/47.6 -> 44.8/44.5, GQA lognormal batch
// forced to 512 321.2/321.1 -> 308.0/307.1; but uniform MHA batch forced to
// 512 185.0/186.8 -> 190.6/192.1 and to 256 190.4/192.8 -> 193.8/194.2 (items
// of one size run at uneven speeds, which dynamic dispatch absorbed).

// Grid choice for a launch of np partitions.  One workgroup per possible item
// launches num_seqs * heads * max_partitions workgroups; on a batch of mixed
// lengths most of them hold no tokens.  In grid order the empty and short
// items are mixed with full-size ones, so the device fills slowly at the
// start (empty workgroups hold the dispatcher) and drains slowly at the end
// (a full-size item dispatched late).  The sorted grid runs the items longest
// first and the empty ones last, for one small ordering kernel and one more
// dependent load per workgroup.  A persistent grid over the work list
// launches no empty workgroups, but deals the items statically (workgroups
// run at uneven speeds, which dynamic dispatch absorbs) and every workgroup
// spends a few microseconds building the list.  Measured (decode kernel,
// grid order -> sorted -> list): skewed batch, 8 partitions 68.8 -> 48.0 ->
// 50.6 us; GQA lognormal batch, 4 partitions 291 -> 273 -> 302 us; long
// contexts, 9 partitions 768 -> 759 -> 764 us; MHA uniform batch, 4
// partitions 206.5 -> 207.6 -> 216.9 us; equal lengths 290 -> 295 -> 303 us.
// So the sorted grid wherever its order fits (for partitions of 1024+
// tokens since the measurements below).  One pass never has empty items.
//
// Below 1024-token partitions, small batches walk the work list each
// workgroup builds in LDS (its cost grows with the batch), larger ones the
// sorted grid's static deal.  Measured (decode kernel incl. ordering, us,
// sorted -> work list, each at its best waves): skewed batch of 32 at 512
// tokens 43.4 -> 40.0, MHA batch of 64 at 512 190.9 -> 188.7 and at 256
// 193.5 -> 191.1; GQA batch of 256 at 512 301.1 -> 309.9.
constexpr int32_t kListMaxSeqs = 64;
//
// A decode step's launches (pa_decode_step, pa_decode_order and the decode
// with PA_DECODE_ORDERED) order the items in the launch that writes the step's
// tokens, which the step pays for anyway, so there the sorted grid is taken
// for small batches too: the decode kernel then skips the list every
// workgroup builds.  Measured (skewed batch of 32 at 512 tokens, rocprofv3):
// decode kernel 34.9-35.1 -> 33.2-34.2 us, the write + order launch as long
// as the write alone.
int grid_mode(const DecodeShape& s, int32_t p, bool step = false) {
  const int64_t np = n_partitions(s, p);
  if (np <= 1) return kGridNatural;
  const bool list_fits = pa::work_list_lds_ints(s.num_seqs, (int)np) <= kMaxListInts;
  const bool order_fits = (int64_t)s.num_seqs * np <= kMaxOrder;
  switch (s.flags & PA_DECODE_GRID_MASK) {
    case PA_DECODE_NO_WORK_LIST: return kGridNatural;
    case PA_DECODE_SORTED_GRID: return order_fits ? kGridSorted : kGridNatural;
    case PA_DECODE_WORK_LIST: return list_fits ? kGridList : kGridNatural;
    default: break;
  }
  if (order_fits && (p >= kPersistentOrderMin || step)) return kGridSorted;
  if (list_fits && s.num_seqs <= kListMaxSeqs) return kGridList;
  if (order_fits) return kGridSorted;
  return list_fits ? kGridList : kGridNatural;
}

// A step's launch: PA_DECODE_ORDERED in the flags (the plan queries take it
// to mean the step's grid).
bool step_flags(const DecodeShape& s) { return (s.flags & PA_DECODE_ORDERED) != 0; }

int32_t work_list_ints(const DecodeShape& s, int32_t p, bool step = false) {
  if (grid_mode(s, p, step) != kGridList) return 0;
  const int64_t np = n_partitions(s, p);
  const int64_t ints = pa::work_list_lds_ints(s.num_seqs, (int)np);
  return (int32_t)((ints + 3) & ~3);  // keep the merge area 16-byte aligned
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace of a partitioned decode: (m, l) and the partial output vector per
// (sequence, q head, partition), then for a sorted grid the item order.
size_t order_offset(const DecodeShape& s, int64_t np) {
  const size_t rows = (size_t)s.num_seqs * s.num_q_heads * (size_t)np;
  return round_up(rows * 2 * sizeof(float)) + round_up(rows * s.head_dim * sizeof(float));
}

size_t workspace_bytes_for(const DecodeShape& s, int32_t p) {
  const int64_t np = n_partitions(s, p);
  if (np <= 1) return 0;
  size_t bytes = order_offset(s, np);
  // the order (and its counter) wherever the launch may sort: a step sorts
  // where a plain decode would walk the work list, with the same workspace
  if (grid_mode(s, p) == kGridSorted || grid_mode(s, p, true) == kGridSorted)
    bytes += round_up((size_t)s.num_seqs * (size_t)np * sizeof(int32_t)) + kAlign;  // + counter
  return bytes;
}

// The library's own partition p (partition_size = 0) is refined on the device
// (DecodeArgs::part_dev, picked by the ordering kernel from the actual lengths
// among p / 2, p and 2p) where the launch is partitioned on the sorted grid's
// counter deal at p and at p / 2: p >= 2048 tokens.  The workspace is then
// sized for p / 2.  Multi-query decodes keep p.
bool device_partition(const DecodeShape& s, int32_t p) {
  const int64_t max_ctx = (int64_t)s.max_blocks_per_seq * s.block_size;
  return p >= 2 * kPersistentOrderMin && max_ctx > p && (p / 2) % s.block_size == 0 &&
         grid_mode(s, p) == kGridSorted && grid_mode(s, p / 2) == kGridSorted;
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return kAbiVersion; }

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "a size is out of range, inconsistent or misaligned";
    case PA_ERR_DTYPE: return "unknown dtype or unsupported dtype combination";
    case PA_ERR_UNSUPPORTED:
      return "head_dim, block_size, group size or kernel choice not supported";
    case PA_ERR_WORKSPACE: return "workspace missing or smaller than pa_decode_workspace_size()";
    case PA_ERR_HIP: return "a HIP kernel launch failed";
    case PA_ERR_CAPACITY: return "not enough free KV blocks (nothing was changed)";
    case PA_ERR_SEQUENCE: return "unknown, duplicate or swapped-out sequence id";
    case PA_ERR_SCRATCH:
      return "the decode needs more than the library's static scratch (PA_SCRATCH_BYTES)";
    default: return "unknown pa_status";
  }
}

}  // extern "C"

namespace {

// Validation and arguments of a 16-bit / fp32 cache write (pa_cache_write).
int write_args(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
               void* v_cache, int64_t num_tokens, int64_t k_token_stride, int64_t v_token_stride,
               int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size,
               int32_t dtype, pa::CacheWriteArgs* a) {
  const int eb = elem_bytes(dtype);
  if (!eb || dtype == PA_DTYPE_FP8_E4M3) return PA_ERR_DTYPE;  // E4M3: pa_cache_write_fp8
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_ERR_UNSUPPORTED;
  if (!valid_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (k_token_stride < row || v_token_stride < row) return PA_ERR_SHAPE;
  if ((k_token_stride * eb) % 16 || (v_token_stride * eb) % 16) return PA_ERR_SHAPE;
  if (num_tokens > 0) {
    if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
      return PA_ERR_SHAPE;
    const int64_t threads = num_tokens * num_kv_heads * ((int64_t)head_dim * eb / 16);
    if ((threads + 255) / 256 > 0x7fffffffLL) return PA_ERR_SHAPE;
  }
  a->k = k;
  a->v = v;
  a->slots = slot_mapping;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->num_tokens = num_tokens;
  a->num_blocks = num_blocks;
  a->k_stride = k_token_stride;
  a->v_stride = v_token_stride;
  a->num_kv_heads = num_kv_heads;
  a->head_dim = head_dim;
  a->block_size = block_size;
  a->elem_bytes = eb;
  a->k_scale = 1.0f;
  a->v_scale = 1.0f;
  a->src_dtype = dtype;
  return PA_OK;
}

// Validation and arguments of a quantizing write into E4M3 caches
// (pa_cache_write_fp8): source rows of src_dtype, per-tensor scales.
int write_args_fp8(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                   void* v_cache, int64_t num_tokens, int64_t k_token_stride,
                   int64_t v_token_stride, int32_t num_kv_heads, int32_t head_dim,
                   int64_t num_blocks, int32_t block_size, int32_t src_dtype, float k_scale,
                   float v_scale, pa::CacheWriteArgs* a) {
  if (src_dtype != PA_DTYPE_F32 && src_dtype != PA_DTYPE_F16 && src_dtype != PA_DTYPE_BF16)
    return PA_ERR_DTYPE;
  const int eb = elem_bytes(src_dtype);
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || k_scale > 3.0e38f || v_scale > 3.0e38f)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_ERR_UNSUPPORTED;
  if (!valid_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (k_token_stride < row || v_token_stride < row) return PA_ERR_SHAPE;
  if ((k_token_stride * eb) % 16 || (v_token_stride * eb) % 16) return PA_ERR_SHAPE;
  if (num_tokens > 0) {
    if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
      return PA_ERR_SHAPE;
    const int64_t threads = num_tokens * num_kv_heads * ((int64_t)head_dim / 16);
    if ((threads + 255) / 256 > 0x7fffffffLL) return PA_ERR_SHAPE;
  }
  a->k = k;
  a->v = v;
  a->slots = slot_mapping;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->num_tokens = num_tokens;
  a->num_blocks = num_blocks;
  a->k_stride = k_token_stride;
  a->v_stride = v_token_stride;
  a->num_kv_heads = num_kv_heads;
  a->head_dim = head_dim;
  a->block_size = block_size;
  a->elem_bytes = 1;
  a->k_scale = k_scale;
  a->v_scale = v_scale;
  a->src_dtype = src_dtype;
  return PA_OK;
}

// A cache write on its own launch: quantizing into E4M3 caches, else a copy.
hipError_t launch_write(const pa::CacheWriteArgs& w, hipStream_t s) {
  return w.elem_bytes == 1 ? pa::launch_cache_write_fp8(w, w.src_dtype, s)
                           : pa::launch_cache_write(w, s);
}

}  // namespace

extern "C" {

int pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                   void* v_cache, int64_t num_tokens, int64_t k_token_stride,
                   int64_t v_token_stride, int32_t num_kv_heads, int32_t head_dim,
                   int64_t num_blocks, int32_t block_size, int32_t dtype, void* stream) {
  pa::CacheWriteArgs a;
  const int st = write_args(k, v, slot_mapping, k_cache, v_cache, num_tokens, k_token_stride,
                            v_token_stride, num_kv_heads, head_dim, num_blocks, block_size, dtype,
                            &a);
  if (st != PA_OK || num_tokens == 0) return st;
  return pa::launch_cache_write(a, (hipStream_t)stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_cache_write_fp8(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                       void* v_cache, int64_t num_tokens, int64_t k_token_stride,
                       int64_t v_token_stride, int32_t num_kv_heads, int32_t head_dim,
                       int64_t num_blocks, int32_t block_size, int32_t src_dtype, float k_scale,
                       float v_scale, void* stream) {
  pa::CacheWriteArgs a;
  const int st = write_args_fp8(k, v, slot_mapping, k_cache, v_cache, num_tokens, k_token_stride,
                                v_token_stride, num_kv_heads, head_dim, num_blocks, block_size,
                                src_dtype, k_scale, v_scale, &a);
  if (st != PA_OK || num_tokens == 0) return st;
  return pa::launch_cache_write_fp8(a, src_dtype, (hipStream_t)stream) == hipSuccess ? PA_OK
                                                                                      : PA_ERR_HIP;
}

int pa_advance_step(int32_t num_seqs, int32_t num_queries, int32_t block_size,
                    int64_t* input_tokens, const int64_t* sampled_token_ids,
                    int64_t* input_positions, int32_t* seq_lens, int64_t* slot_mapping,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, void* stream) {
  if (num_seqs < 0 || num_queries < 0 || num_queries > num_seqs || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (block_size <= 0) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!input_tokens || !input_positions || !seq_lens || !slot_mapping || !block_tables ||
      (num_queries > 0 && !sampled_token_ids))
    return PA_ERR_NULL;
  pa::AdvanceArgs a;
  a.input_tokens = input_tokens;
  a.sampled_token_ids = sampled_token_ids;
  a.input_positions = input_positions;
  a.seq_lens = seq_lens;
  a.slot_mapping = slot_mapping;
  a.block_tables = block_tables;
  a.num_seqs = num_seqs;
  a.num_queries = num_queries;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  return pa::launch_advance_step(a, (hipStream_t)stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_check_tables(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks,
                    uint32_t* status, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size < 1 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if ((int64_t)num_seqs * max_blocks_per_seq > ((int64_t)1 << 38)) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !context_lens || !status) return PA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(status) & 3u) return PA_ERR_SHAPE;
  return pa::launch_check_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                 block_size, num_blocks, status,
                                 (hipStream_t)stream) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int pa_check_slots(const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                   int32_t block_size, uint32_t* status, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || block_size < 1) return PA_ERR_SHAPE;
  if (num_tokens > ((int64_t)1 << 38)) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping || !status) return PA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(status) & 3u) return PA_ERR_SHAPE;
  return pa::launch_check_slots(slot_mapping, num_tokens, num_blocks * (int64_t)block_size,
                                status, (hipStream_t)stream) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int32_t kv_dtype, uint32_t flags) {
  DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                kv_dtype, flags};
  const int st = check_shape(s);
  if (st != PA_OK) return st;
  return pick_partition(s);
}

int32_t pa_decode_mq_kernel(int32_t num_queries, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t q_dtype, int32_t kv_dtype, uint32_t flags) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return PA_ERR_SHAPE;
  if (num_queries < 1 || num_queries > 16) return PA_ERR_SHAPE;
  if (!elem_bytes(q_dtype) || !elem_bytes(kv_dtype)) return PA_ERR_DTYPE;
  if (!valid_q_dtype(q_dtype, kv_dtype)) return PA_ERR_DTYPE;
  if (!valid_flags(flags)) return PA_ERR_UNSUPPORTED;
  if (forces_mfma(flags) && !mfma_eligible(kv_dtype, q_dtype)) return PA_ERR_UNSUPPORTED;
  const int32_t k =
      pick_kernel(flags, kv_dtype, q_dtype, num_q_heads / num_kv_heads, num_queries);
  return k ? k : PA_ERR_UNSUPPORTED;
}

int32_t pa_decode_kernel(int32_t num_q_heads, int32_t num_kv_heads, int32_t q_dtype,
                         int32_t kv_dtype, uint32_t flags) {
  return pa_decode_mq_kernel(1, num_q_heads, num_kv_heads, q_dtype, kv_dtype, flags);
}

namespace {

// Shared validation of the plan queries; the partition size pa_decode uses in *p.
int32_t plan_args(const DecodeShape& s, int32_t partition_size, int32_t q_dtype, int32_t* p) {
  const int st = check_shape(s);
  if (st != PA_OK) return st;
  if (!valid_q_dtype(q_dtype, s.kv_dtype)) return PA_ERR_DTYPE;
  if (forces_mfma(s.flags) && !mfma_eligible(s.kv_dtype, q_dtype)) return PA_ERR_UNSUPPORTED;
  if (partition_size < 0 || (partition_size > 0 && partition_size % s.block_size))
    return PA_ERR_SHAPE;
  const int64_t max_ctx = (int64_t)s.max_blocks_per_seq * s.block_size;
  *p = partition_size ? partition_size : pick_partition(s);
  if (*p > max_ctx) *p = (int32_t)max_ctx;
  return PA_OK;
}

}  // namespace

int32_t pa_decode_waves(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                        int32_t partition_size, int32_t q_dtype, int32_t kv_dtype,
                        uint32_t flags) {
  DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                kv_dtype, flags};
  int32_t p = 0;
  const int32_t st = plan_args(s, partition_size, q_dtype, &p);
  return st != PA_OK ? st : pick_waves(s, p);
}

int32_t pa_decode_work_list(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                            int32_t partition_size, int32_t q_dtype, int32_t kv_dtype,
                            uint32_t flags) {
  DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                kv_dtype, flags};
  int32_t p = 0;
  const int32_t st = plan_args(s, partition_size, q_dtype, &p);
  return st != PA_OK ? st : (work_list_ints(s, p, step_flags(s)) > 0 ? 1 : 0);
}

int32_t pa_decode_grid(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                       int32_t partition_size, int32_t q_dtype, int32_t kv_dtype, uint32_t flags) {
  DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                kv_dtype, flags};
  int32_t p = 0;
  const int32_t st = plan_args(s, partition_size, q_dtype, &p);
  if (st != PA_OK) return st;
  switch (grid_mode(s, p, step_flags(s))) {
    case kGridSorted: return PA_DECODE_SORTED_GRID;
    case kGridList: return PA_DECODE_WORK_LIST;
    default: return PA_DECODE_NO_WORK_LIST;
  }
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t partition_size, int32_t kv_dtype, uint32_t flags) {
  DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                kv_dtype, flags};
  if (check_shape(s) != PA_OK) return 0;
  if (partition_size < 0 || (partition_size > 0 && partition_size % block_size)) return 0;
  if (partition_size) return workspace_bytes_for(s, partition_size);
  const int32_t p = pick_partition(s);
  return workspace_bytes_for(s, device_partition(s, p) ? p / 2 : p);
}

int32_t pa_decode_partition_used(const void* workspace, size_t workspace_bytes,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int32_t kv_dtype, uint32_t flags,
                                 void* stream) {
  DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                kv_dtype, flags};
  const int st = check_shape(s);
  if (st != PA_OK) return st;
  const int32_t p = pick_partition(s);
  if (!device_partition(s, p)) return p;
  const int64_t np = n_partitions(s, p / 2);
  // the ordering kernel's words sit a 128-byte line after the ticket counter
  const size_t off = order_offset(s, np) + round_up((size_t)num_seqs * (size_t)np * 4) + 128;
  if (!workspace || workspace_bytes < off + 4 || workspace_bytes < workspace_bytes_for(s, p / 2))
    return PA_ERR_WORKSPACE;
  int32_t used = 0;
  if (hipMemcpyAsync(&used, reinterpret_cast<const char*>(workspace) + off, 4,
                     hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess ||
      hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
    return PA_ERR_HIP;
  return (used == p / 2 || used == p || used == 2 * p) ? used : p;
}

}  // extern "C"

// ---- pa_decode_noalloc: the partition workspace in a static device array ----
namespace {

// The library's own partition workspace for pa_decode_noalloc: a file-scope
// device array, one copy per GPU for the life of the process.  Host code never
// passes `scratch` itself to a kernel (on the host it is only a stand-in for
// the symbol): its device address is looked up once per device and kept.
constexpr size_t kScratchBytes = PA_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
std::atomic<void*> scratch_ptr[kMaxDevices];

// The device address of the current device's scratch (looked up on the first
// call on that device, with that device current), or NULL on failure.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> g(scratch_mu);
  p = scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
  scratch_ptr[dev].store(addr, std::memory_order_release);
  return addr;
}

}  // namespace

namespace pa {
namespace {
int cu_count();  // compute units of the current device (below)
}  // namespace
}  // namespace pa

namespace {

// kOrder: only the launch before the decode kernel (a step's write and/or the
// item ordering), for pa_decode_order
enum Phase { kPartitions = 1, kMerge = 2, kBoth = 3, kOrder = 4 };

int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, float scale,
                int32_t block_size, int32_t partition_size, int32_t num_seqs, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                int32_t max_blocks_per_seq, int32_t q_dtype, int32_t kv_dtype, int32_t out_dtype,
                void* workspace, size_t workspace_bytes, uint32_t flags, void* stream, int phase,
                float k_scale = 1.0f, float v_scale = 1.0f, int32_t num_queries = 1,
                const pa::CacheWriteArgs* pre_write = nullptr, bool use_scratch = false) {
  DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                kv_dtype, flags};
  int st = check_shape(s);
  if (st != PA_OK) return st;
  if (num_blocks <= 0) return PA_ERR_SHAPE;
  if (!valid_q_dtype(q_dtype, kv_dtype)) return PA_ERR_DTYPE;
  if (!valid_out_dtype(out_dtype, q_dtype, kv_dtype)) return PA_ERR_DTYPE;
  if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || k_scale > 3.0e38f || v_scale > 3.0e38f)
    return PA_ERR_SHAPE;
  if (partition_size < 0 || (partition_size > 0 && partition_size % block_size))
    return PA_ERR_SHAPE;
  if (forces_mfma(flags) && !mfma_eligible(kv_dtype, q_dtype)) return PA_ERR_UNSUPPORTED;
  if (num_queries < 1 || num_queries > 16) return PA_ERR_SHAPE;
  const bool preordered = (flags & PA_DECODE_ORDERED) != 0 && phase != kOrder;
  if (preordered && (num_queries > 1 || pre_write || use_scratch)) return PA_ERR_UNSUPPORTED;
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t kernel = pick_kernel(flags, kv_dtype, q_dtype, group, num_queries);
  if (!kernel) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) {  // nothing to attend; a step's cache write still runs
    if (pre_write && pre_write->num_tokens > 0 && (phase & (kPartitions | kOrder)))
      return launch_write(*pre_write, (hipStream_t)stream) == hipSuccess ? PA_OK
                                                                                  : PA_ERR_HIP;
    return PA_OK;
  }
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_SHAPE;

  // The workspace holds a (m, l) pair and a partial vector per query row, and
  // the plan queries take num_seqs * num_queries for a multi-query decode: the
  // partition is picked on that shape too, so that both agree.
  DecodeShape rows_shape = s;
  if ((int64_t)num_seqs * num_queries > 0x7fffffffLL) return PA_ERR_SHAPE;
  rows_shape.num_seqs = num_seqs * num_queries;
  const int64_t max_ctx = (int64_t)max_blocks_per_seq * block_size;
  int32_t p = partition_size ? partition_size : pick_partition(rows_shape);
  if (p > max_ctx) p = (int32_t)max_ctx;
  // the smallest partition the launch may use: p, or p / 2 where the device picks
  const bool on_device = partition_size == 0 && num_queries == 1 &&
                         device_partition(rows_shape, p);
  const int32_t p_min = on_device ? p / 2 : p;
  const int64_t np = n_partitions(s, p_min);
  const size_t need = workspace_bytes_for(rows_shape, p_min);
  if (use_scratch && need > 0) {  // pa_decode_noalloc: the library's static array
    if (need > kScratchBytes) return PA_ERR_SCRATCH;
    if (!(workspace = device_scratch())) return PA_ERR_HIP;
    workspace_bytes = kScratchBytes;
  }
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return PA_ERR_WORKSPACE;
  if (np > 65535 || (int64_t)num_seqs * num_queries * num_q_heads > 0x7fffffffLL)
    return PA_ERR_SHAPE;

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t rows = (size_t)num_seqs * num_queries * num_q_heads * (size_t)np;
  char* ws = reinterpret_cast<char*>(workspace);
  a.ws_ml = need ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_acc = need ? reinterpret_cast<float*>(ws + round_up(rows * 2 * sizeof(float))) : nullptr;
  a.scale_log2 = scale * k_scale * 1.4426950408889634f;
  a.v_scale = v_scale;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  const bool mfma = kernel == PA_DECODE_FORCE_MFMA;
  a.heads_per_item =
      mfma ? mfma_heads_per_item(group, num_queries) : valu_heads_per_item(group, num_queries);
  a.num_queries = num_queries;
  a.block_size = block_size;
  a.log2_block_size = log2_exact(block_size);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.partition_size = p;
  a.max_partitions = (int32_t)np;
  a.q_dtype = q_dtype;
  a.out_dtype = out_dtype;
  a.waves = pick_waves(s, p);
  // one grid decision for the workspace and the launch (both on the query rows' shape)
  // a step's launches (its write, its ordering, the decode after them) sort
  const bool step = pre_write || phase == kOrder || preordered;
  const int mode = grid_mode(rows_shape, p_min, step);
  a.list_ints = mode == kGridList ? work_list_ints(rows_shape, p_min, step) : 0;
  a.order = mode == kGridSorted
                ? reinterpret_cast<const int32_t*>(ws + order_offset(rows_shape, np))
                : nullptr;
  a.order_ctr = a.order && p >= kPersistentOrderMin
                    ? reinterpret_cast<int32_t*>(
                          ws + order_offset(rows_shape, np) +
                          round_up((size_t)rows_shape.num_seqs * (size_t)np * sizeof(int32_t)))
                    : nullptr;
  a.order_static = a.order && !a.order_ctr ? 1 : 0;  // shorter partitions: static deal
  // the ordering kernel's two words: in the counter's 256-byte slot, on the
  // next 128-byte line (the ticket atomics keep the counter's line busy).
  // Only where it picks the partition: the entry count alone, read per item,
  // measured 0.4% slower on the MHA batch at 1024-token partitions.
  a.part_dev = on_device ? a.order_ctr + 32 : nullptr;
  a.part_pick = on_device ? 1 : 0;
  a.num_cus = pa::cu_count();

  hipStream_t hs = (hipStream_t)stream;
  if (phase == kOrder) {  // the write and the ordering, no decode
    if (a.order) {
      if (pa::launch_decode_order(a, const_cast<int32_t*>(a.order), pre_write, hs) != hipSuccess)
        return PA_ERR_HIP;
    } else if (pre_write && pre_write->num_tokens > 0 &&
               launch_write(*pre_write, hs) != hipSuccess) {
      return PA_ERR_HIP;
    }
    return PA_OK;
  }
  if (phase & kPartitions) {
    // a step's cache write goes first: in the launch that orders the items, or on its own
    if (a.order && !preordered) {
      if (pa::launch_decode_order(a, const_cast<int32_t*>(a.order), pre_write, hs) != hipSuccess)
        return PA_ERR_HIP;
    } else if (!a.order && pre_write && pre_write->num_tokens > 0 &&
               launch_write(*pre_write, hs) != hipSuccess) {
      return PA_ERR_HIP;
    }
    const hipError_t e = mfma ? pa::launch_decode_mfma(a, kv_dtype, head_dim, hs)
                              : pa::launch_decode_valu(a, kv_dtype, head_dim, hs);
    if (e != hipSuccess) return PA_ERR_HIP;
  }
  if ((phase & kMerge) && np > 1 && pa::launch_decode_reduce(a, head_dim, hs) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

}  // namespace

extern "C" {

#define PA_DECODE_PARAMS                                                                       \
  void *out, const void *q, const void *k_cache, const void *v_cache,                          \
      const int32_t *block_tables, const int32_t *context_lens, float scale, int32_t block_size, \
      int32_t partition_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,     \
      int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t q_dtype,       \
      int32_t kv_dtype, int32_t out_dtype, void *workspace, size_t workspace_bytes,            \
      uint32_t flags, void *stream
#define PA_DECODE_ARGS                                                                       \
  out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, partition_size,   \
      num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, q_dtype, \
      kv_dtype, out_dtype, workspace, workspace_bytes, flags, stream

// E4M3 caches go through pa_decode_fp8 (they need their scales)
int pa_decode(PA_DECODE_PARAMS) {
  if (kv_dtype == PA_DTYPE_FP8_E4M3) return PA_ERR_DTYPE;
  return decode_impl(PA_DECODE_ARGS, kBoth);
}
int pa_decode_partitions(PA_DECODE_PARAMS) {
  if (kv_dtype == PA_DTYPE_FP8_E4M3) return PA_ERR_DTYPE;
  return decode_impl(PA_DECODE_ARGS, kPartitions);
}
int pa_decode_merge(PA_DECODE_PARAMS) { return decode_impl(PA_DECODE_ARGS, kMerge); }

// pa_decode with the static scratch as its workspace; every argument is
// validated (and the scratch's limit checked) before the scratch is looked up.
int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t partition_size, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int64_t num_blocks, int32_t max_blocks_per_seq, int32_t q_dtype,
                      int32_t kv_dtype, int32_t out_dtype, uint32_t flags, void* stream) {
  if (kv_dtype == PA_DTYPE_FP8_E4M3) return PA_ERR_DTYPE;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                     partition_size, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                     max_blocks_per_seq, q_dtype, kv_dtype, out_dtype, nullptr, 0, flags, stream,
                     kBoth, 1.0f, 1.0f, 1, nullptr, true);
}

#define PA_STEP_PARAMS                                                                         \
  const void *k, const void *v, const int64_t *slot_mapping, int64_t num_tokens,              \
      int64_t k_token_stride, int64_t v_token_stride, void *out, const void *q, void *k_cache, \
      void *v_cache, const int32_t *block_tables, const int32_t *context_lens, float scale,    \
      int32_t block_size, int32_t partition_size, int32_t num_seqs, int32_t num_q_heads,       \
      int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,  \
      int32_t q_dtype, int32_t kv_dtype, int32_t out_dtype, void *workspace,                   \
      size_t workspace_bytes, uint32_t flags, void *stream

// A decode step: the step's cache write, then the decode; nothing is launched
// unless both validate.  kOrder (pa_decode_order): the write and the item
// ordering only; E4M3 caches there only without a write.
static int step_impl(PA_STEP_PARAMS, int phase) {
  if (phase == kOrder && kv_dtype == PA_DTYPE_FP8_E4M3 && num_tokens == 0)
    return decode_impl(PA_DECODE_ARGS, phase);
  if (kv_dtype == PA_DTYPE_FP8_E4M3) return PA_ERR_DTYPE;
  if (phase != kOrder && (flags & PA_DECODE_ORDERED)) return PA_ERR_UNSUPPORTED;
  pa::CacheWriteArgs w;
  const int st = write_args(k, v, slot_mapping, k_cache, v_cache, num_tokens, k_token_stride,
                            v_token_stride, num_kv_heads, head_dim, num_blocks, block_size,
                            kv_dtype, &w);
  if (st != PA_OK) return st;
  return decode_impl(PA_DECODE_ARGS, phase, 1.0f, 1.0f, 1, &w);
}

int pa_decode_step(PA_STEP_PARAMS) {
  return step_impl(k, v, slot_mapping, num_tokens, k_token_stride, v_token_stride, PA_DECODE_ARGS,
                   kBoth);
}
int pa_decode_step_partitions(PA_STEP_PARAMS) {
  return step_impl(k, v, slot_mapping, num_tokens, k_token_stride, v_token_stride, PA_DECODE_ARGS,
                   kPartitions);
}
int pa_decode_order(PA_STEP_PARAMS) {
  return step_impl(k, v, slot_mapping, num_tokens, k_token_stride, v_token_stride, PA_DECODE_ARGS,
                   kOrder);
}

int pa_decode_order_fp8(const void* k, const void* v, const int64_t* slot_mapping,
                        int64_t num_tokens, int64_t k_token_stride, int64_t v_token_stride,
                        int32_t src_dtype, float k_scale, float v_scale, void* out,
                        const void* q, void* k_cache, void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens, float scale,
                        int32_t block_size, int32_t partition_size, int32_t num_seqs,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int64_t num_blocks, int32_t max_blocks_per_seq, int32_t q_dtype,
                        int32_t out_dtype, void* workspace, size_t workspace_bytes,
                        uint32_t flags, void* stream) {
  pa::CacheWriteArgs w;
  const int st = write_args_fp8(k, v, slot_mapping, k_cache, v_cache, num_tokens, k_token_stride,
                                v_token_stride, num_kv_heads, head_dim, num_blocks, block_size,
                                src_dtype, k_scale, v_scale, &w);
  if (st != PA_OK) return st;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                     partition_size, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                     max_blocks_per_seq, q_dtype, PA_DTYPE_FP8_E4M3, out_dtype, workspace,
                     workspace_bytes, flags, stream, kOrder, k_scale, v_scale, 1, &w);
}

#define PA_DECODE_FP8_PARAMS                                                                   \
  void *out, const void *q, const void *k_cache, const void *v_cache,                          \
      const int32_t *block_tables, const int32_t *context_lens, float scale, float k_scale,    \
      float v_scale, int32_t block_size, int32_t partition_size, int32_t num_seqs,             \
      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,         \
      int32_t max_blocks_per_seq, int32_t q_dtype, int32_t out_dtype, void *workspace,         \
      size_t workspace_bytes, uint32_t flags, void *stream

#define PA_DECODE_MQ_PARAMS                                                                    \
  void *out, const void *q, const void *k_cache, const void *v_cache,                          \
      const int32_t *block_tables, const int32_t *context_lens, float scale, float k_scale,    \
      float v_scale, int32_t block_size, int32_t partition_size, int32_t num_seqs,             \
      int32_t num_queries, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,        \
      int64_t num_blocks, int32_t max_blocks_per_seq, int32_t q_dtype, int32_t kv_dtype,       \
      int32_t out_dtype, void *workspace, size_t workspace_bytes, uint32_t flags, void *stream
#define PA_DECODE_MQ_ARGS(phase)                                                               \
  out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, partition_size,     \
      num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, q_dtype,   \
      kv_dtype, out_dtype, workspace, workspace_bytes, flags, stream, phase, k_scale, v_scale,  \
      num_queries

int pa_decode_mq(PA_DECODE_MQ_PARAMS) { return decode_impl(PA_DECODE_MQ_ARGS(kBoth)); }
int pa_decode_mq_partitions(PA_DECODE_MQ_PARAMS) {
  return decode_impl(PA_DECODE_MQ_ARGS(kPartitions));
}
int pa_decode_mq_merge(PA_DECODE_MQ_PARAMS) { return decode_impl(PA_DECODE_MQ_ARGS(kMerge)); }

int pa_decode_fp8(PA_DECODE_FP8_PARAMS) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                     partition_size, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                     max_blocks_per_seq, q_dtype, PA_DTYPE_FP8_E4M3, out_dtype, workspace,
                     workspace_bytes, flags, stream, kBoth, k_scale, v_scale);
}
int pa_decode_fp8_partitions(PA_DECODE_FP8_PARAMS) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                     partition_size, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                     max_blocks_per_seq, q_dtype, PA_DTYPE_FP8_E4M3, out_dtype, workspace,
                     workspace_bytes, flags, stream, kPartitions, k_scale, v_scale);
}

}  // extern "C"


namespace pa {

namespace {

int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) {
    const int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      c <= 0)
    c = 1;
  if (dev >= 0 && dev < 64) cached[dev].store(c, std::memory_order_relaxed);
  return c;
}

// Resident workgroups per CU of a kernel, cached per (kernel, block, LDS).
int resident_per_cu(const void* fn, int block, size_t lds) {
  struct Entry {
    const void* fn;
    int block;
    size_t lds;
    int occ;
  };
  static std::mutex mu;
  static Entry cache[64];
  static int next = 0;
  {
    std::lock_guard<std::mutex> g(mu);
    for (const Entry& e : cache)
      if (e.fn == fn && e.block == block && e.lds == lds) return e.occ;
  }
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, block, lds) != hipSuccess ||
      occ <= 0)
    occ = 1;
  std::lock_guard<std::mutex> g(mu);
  cache[next] = Entry{fn, block, lds, occ};
  next = (next + 1) % 64;
  return occ;
}

}  // namespace

hipError_t launch_decode_grid(const void* kernel, const DecodeArgs& a, int64_t items_x,
                              size_t lds, hipStream_t s) {
  const dim3 block(64 * a.waves);
  dim3 grid;
  if (a.list_ints > 0 || a.order_ctr || a.order_static) {
    const int64_t fit = (int64_t)cu_count() * resident_per_cu(kernel, (int)block.x, lds);
    // at most one workgroup per item at partition_size: where the ordering
    // kernel picks the partition, max_partitions counts the half, and the
    // surplus workgroups (with a batch of fewer items than the device holds
    // workgroups) cost 2% on uniform batches; the counter deals any extra items
    const int64_t max_ctx = (int64_t)a.max_blocks_per_seq * a.block_size;
    const int64_t np = a.part_pick ? (max_ctx + a.partition_size - 1) / a.partition_size
                                   : a.max_partitions;
    const int64_t upper = items_x * np;
    const int64_t g = fit < upper ? fit : upper;
    grid = dim3((unsigned)(g < 0x7fffffff ? g : 0x7fffffff));
  } else {
    grid = dim3((unsigned)items_x, (unsigned)a.max_partitions);
  }
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  return hipLaunchKernel(kernel, grid, block, args, lds, s);
}

}  // namespace pa
