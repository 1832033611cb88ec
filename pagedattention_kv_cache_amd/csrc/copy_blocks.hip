// copy_blocks.hip -- whole-block copies of the paged caches (include/pa_blocks.h).
//
// pa_copy_blocks is the device side of copy-on-write: a sequence about to
// write into a block it shares gets a private copy first (KV cache managed
// like virtual memory with shared pages, "vLLM Project Update" talk,
// PagedAttention recap).  pa_swap_blocks moves blocks between a device cache
// and a host swap pool (the v2 block manager's swap space in the
// "[core] Multi Step Scheduling" pull request).
//
// A physical block is one contiguous run of bytes in each cache (the block
// index is the outermost dimension of both layouts), so a block copy is a
// plain 16-byte-vector copy: HBM-bound, 2 x block_bytes read and written per
// pair and cache.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_blocks.h"

namespace {

__global__ __launch_bounds__(256) void copy_blocks_kernel(char* k_cache, char* v_cache,
                                                          const int32_t* pairs, int32_t num_pairs,
                                                          int64_t num_blocks, int64_t block_bytes) {
  char* base = blockIdx.z ? v_cache : k_cache;
  const int64_t chunks = block_bytes / 16;
  for (int32_t p = blockIdx.y; p < num_pairs; p += gridDim.y) {
    const int32_t src = pairs[2 * p];
    const int32_t dst = pairs[2 * p + 1];
    // out-of-range pairs break the caller's contract; skipped, not followed
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
    const uint4* s = reinterpret_cast<const uint4*>(base + (int64_t)src * block_bytes);
    uint4* d = reinterpret_cast<uint4*>(base + (int64_t)dst * block_bytes);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks;
         i += (int64_t)gridDim.x * blockDim.x)
      d[i] = s[i];
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                   int64_t num_blocks, int64_t block_bytes, void* stream) {
  if (num_pairs < 0 || num_blocks < 1 || block_bytes <= 0 || block_bytes % 16) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_SHAPE;
  const int64_t chunks = block_bytes / 16;
  const int64_t per_block = (chunks + 255) / 256;
  const dim3 grid((unsigned)(per_block < 64 ? per_block : 64),
                  (unsigned)(num_pairs < 65535 ? num_pairs : 65535), 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache), pairs, num_pairs,
                     num_blocks, block_bytes);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_swap_blocks(void* dst_pool, const void* src_pool, const int32_t* pairs, int32_t num_pairs,
                   int64_t block_bytes, void* stream) {
  if (num_pairs < 0 || block_bytes <= 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!dst_pool || !src_pool || !pairs) return PA_ERR_NULL;
  for (int32_t p = 0; p < num_pairs; ++p)
    if (pairs[2 * p] < 0 || pairs[2 * p + 1] < 0) return PA_ERR_SHAPE;
  const char* src = static_cast<const char*>(src_pool);
  char* dst = static_cast<char*>(dst_pool);
  for (int32_t p = 0; p < num_pairs;) {
    // a run of pairs whose sources and destinations both go up by one
    int32_t q = p + 1;
    while (q < num_pairs && pairs[2 * q] == pairs[2 * (q - 1)] + 1 &&
           pairs[2 * q + 1] == pairs[2 * (q - 1) + 1] + 1)
      ++q;
    const hipError_t e =
        hipMemcpyAsync(dst + (int64_t)pairs[2 * p + 1] * block_bytes,
                       src + (int64_t)pairs[2 * p] * block_bytes, (size_t)(q - p) * block_bytes,
                       hipMemcpyDefault, (hipStream_t)stream);
    if (e != hipSuccess) return PA_ERR_HIP;
    p = q;
  }
  return PA_OK;
}

}  // extern "C"
