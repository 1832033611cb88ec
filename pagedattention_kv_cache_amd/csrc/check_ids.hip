// check_ids.hip -- opt-in checks of the ids the hot path takes on trust.
//
// Block-table entries inside a context and the slots of a cache write are
// preconditions: the decode kernels clamp an entry outside the pool into it
// (and a context length beyond what the table can address down to it), the
// cache write drops a slot past the pool, so memory stays in bounds, but a
// broken table or slot mapping gives a wrong answer with no signal.  These
// kernels evaluate exactly the conditions under which the hot kernels clamp or
// drop, and OR a bit per kind into a caller-owned device status word.  They
// run on their own, before the decode or write they vouch for, so the hot
// kernels carry no extra code or registers.
#include "pa.h"
#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {
namespace {

// OR of the wave's bits; one lane writes them with a vector atomic.
__device__ __forceinline__ void report(uint32_t* status, uint32_t bits) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) bits |= (uint32_t)__shfl_xor((int)bits, o);
  if ((threadIdx.x & 63) == 0 && bits) atomicOr(status, bits);
}

// One thread per block-table entry (sequence b, logical block j).
__global__ __launch_bounds__(256) void check_tables_kernel(const int32_t* block_tables,
                                                           const int32_t* context_lens,
                                                           int32_t num_seqs,
                                                           int32_t max_blocks_per_seq,
                                                           int32_t block_size, int64_t num_blocks,
                                                           uint32_t* status) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t bits = 0;
  if (i < (int64_t)num_seqs * max_blocks_per_seq) {
    const int b = (int)(i / max_blocks_per_seq);
    const int j = (int)(i - (int64_t)b * max_blocks_per_seq);
    const int L = context_lens[b];
    if (j == 0 && (L < 0 || (int64_t)L > (int64_t)max_blocks_per_seq * block_size))
      bits |= PA_CHECK_CONTEXT_LEN;
    // the blocks the kernels read: those of the (clamped) context
    const int Lc = clamp_len(L, max_blocks_per_seq, block_size);
    if (Lc > 0 && j < (Lc + block_size - 1) / block_size) {
      const int32_t e = block_tables[i];
      if (e < 0 || (int64_t)e >= num_blocks) bits |= PA_CHECK_BLOCK_ID;
    }
  }
  report(status, bits);
}

// One thread per token of a cache write.
__global__ __launch_bounds__(256) void check_slots_kernel(const int64_t* slots,
                                                          int64_t num_tokens, int64_t capacity,
                                                          uint32_t* status) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t bits = 0;
  if (i < num_tokens && slots[i] >= capacity) bits = PA_CHECK_SLOT;
  report(status, bits);
}

}  // namespace

hipError_t launch_check_tables(const int32_t* block_tables, const int32_t* context_lens,
                               int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                               int64_t num_blocks, uint32_t* status, hipStream_t s) {
  const int64_t n = (int64_t)num_seqs * max_blocks_per_seq;
  hipLaunchKernelGGL(check_tables_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size,
                     num_blocks, status);
  return hipGetLastError();
}

hipError_t launch_check_slots(const int64_t* slots, int64_t num_tokens, int64_t capacity,
                              uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(check_slots_kernel, dim3((unsigned)((num_tokens + 255) / 256)), dim3(256), 0,
                     s, slots, num_tokens, capacity, status);
  return hipGetLastError();
}

}  // namespace pa
