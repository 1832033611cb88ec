// advance_step.hip -- advance the per-sequence decode state by one step on the
// device, so several decode steps can run back to back (or be captured once
// in a HIP graph and replayed) without the host recomputing slots.
//
// The "[core] Multi Step Scheduling" pull request (vllm-project/vllm #7000),
// review thread on ops.advance_step: between steps the GPU updates the next
// input tokens, positions, sequence lengths and slot mapping in place from
// the sampled ids, the block tables and the block size.  Restated here: for a
// live sequence i, the sampled id becomes its next input token, its position
// moves one forward, its length becomes position + 1 and its slot is the
// position's offset inside the physical block the table names.
#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void advance_step_kernel(AdvanceArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.num_seqs) return;
  if (i >= a.num_queries) {  // padding row: nothing to write next step
    a.slot_mapping[i] = -1;
    return;
  }
  a.input_tokens[i] = a.sampled_token_ids[i];
  const int64_t pos = a.input_positions[i] + 1;
  a.input_positions[i] = pos;
  a.seq_lens[i] = (int32_t)(pos + 1);
  const int64_t lblk = pos / a.block_size;
  int64_t slot = -1;  // no block allocated for the position: the write skips it
  if (lblk < a.max_blocks_per_seq) {
    const int32_t phys = a.block_tables[(int64_t)i * a.max_blocks_per_seq + lblk];
    if (phys >= 0) slot = (int64_t)phys * a.block_size + pos % a.block_size;
  }
  a.slot_mapping[i] = slot;
}

}  // namespace

hipError_t launch_advance_step(const AdvanceArgs& a, hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  const int threads = 256;
  hipLaunchKernelGGL(advance_step_kernel, dim3((a.num_seqs + threads - 1) / threads),
                     dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
