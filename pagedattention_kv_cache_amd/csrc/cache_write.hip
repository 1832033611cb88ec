// cache_write.hip -- the paged KV-cache slot write (reshape-and-cache).
//
// Every new token's key and value rows go to the slot the caller assigned
// ("[core] Multi Step Scheduling" pull request, advance_step review thread:
// slot_mapping next to block_tables and block_size).  A bit copy, no
// arithmetic on values.
//
// Thread mapping: one thread moves one 16-byte chunk of one (token, kv head)
// row.  Both caches keep the tokens of a block in quads of four consecutive
// offsets.  Keys: [block][head][quad][chunk][4][16 bytes], so chunk c of the
// token at offset o lands at ((o/4 * chunks + c) * 4 + o%4) * 16 bytes into
// the (block, head) tile.  Values: [block][head][quad][dim][4], so the
// chunk's elements go to consecutive dims of row o%4, four elements apart.
// A single token therefore fills 32 of every 128 bytes it touches, not a
// single 16- or 2-byte slot of each line.
#include "cache_write.hpp"
#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {
namespace {

template <int EB>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a, int chunks_per_row) {
  cache_write_chunk<EB>(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x, chunks_per_row);
}

// Quantizing write into E4M3 caches ("vLLM Project Update" talk, quantization
// update: an 8-bit floating-point KV cache; the talk fixes no format, the one
// taken is OCP E4M3 with a scale per cache tensor): one thread per 16-element
// key chunk of a (token, kv head) row, cache_write_fp8_chunk.
template <Elem SRC>
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(CacheWriteArgs a,
                                                              int chunks_per_row) {
  cache_write_fp8_chunk<SRC>(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x, chunks_per_row);
}

}  // namespace

hipError_t launch_cache_write_fp8(const CacheWriteArgs& a, int src_dtype, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int chunks = a.head_dim / 16;
  const int64_t total = a.num_tokens * a.num_kv_heads * chunks;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(threads);
  switch (src_dtype) {
    case 0:
      hipLaunchKernelGGL(cache_write_fp8_kernel<Elem::F32>, grid, block, 0, stream, a, chunks);
      break;
    case 1:
      hipLaunchKernelGGL(cache_write_fp8_kernel<Elem::F16>, grid, block, 0, stream, a, chunks);
      break;
    case 2:
      hipLaunchKernelGGL(cache_write_fp8_kernel<Elem::BF16>, grid, block, 0, stream, a, chunks);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int chunks = a.head_dim * a.elem_bytes / 16;
  const int64_t total = a.num_tokens * a.num_kv_heads * chunks;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.elem_bytes == 4) {
    hipLaunchKernelGGL(cache_write_kernel<4>, dim3((unsigned)blocks), dim3(threads), 0, stream, a,
                       chunks);
  } else {
    hipLaunchKernelGGL(cache_write_kernel<2>, dim3((unsigned)blocks), dim3(threads), 0, stream, a,
                       chunks);
  }
  return hipGetLastError();
}

}  // namespace pa
