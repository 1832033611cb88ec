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
// taken is OCP E4M3 with a scale per cache tensor).  One thread per 16-byte
// key chunk = 16 elements of one (token, kv head) row: each element x becomes
// e4m3(x / scale), the quotient an IEEE fp32 division (correctly rounded), the
// conversion fp8_e4m3_encode.  Key chunk c of the token at offset o lands at
// ((o/4 * chunks + c) * 4 + o%4) * 16 bytes into the (block, head) tile; the
// chunk's 16 value elements go to consecutive dims of row o%4, 4 bytes apart.
template <Elem SRC>
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(CacheWriteArgs a,
                                                              int chunks_per_row) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)a.num_kv_heads * chunks_per_row;
  const int64_t total = a.num_tokens * per_token;
  if (gid >= total) return;
  const int64_t t = gid / per_token;
  const int rem = (int)(gid - t * per_token);
  const int h = rem / chunks_per_row;
  const int c = rem - h * chunks_per_row;
  constexpr int SB = ElemTraits<SRC>::bytes;
  constexpr int SPL = 16 / SB;  // source elements per 16-byte load
  const int64_t D = a.head_dim;
  const int e0 = c * 16;
  // the source rows and the slot go out together (one round trip, not two)
  const char* ksrc = reinterpret_cast<const char*>(a.k) + ((t * a.k_stride) + h * D + e0) * SB;
  const char* vsrc = reinterpret_cast<const char*>(a.v) + ((t * a.v_stride) + h * D + e0) * SB;
  uint4 kraw[16 / SPL], vraw[16 / SPL];
#pragma unroll
  for (int i = 0; i < 16 / SPL; ++i) {
    kraw[i] = ld16(ksrc + 16 * i);
    vraw[i] = ld16(vsrc + 16 * i);
  }
  const int64_t slot = a.slots[t];
#pragma unroll
  for (int i = 0; i < 16 / SPL; ++i) loaded_here(kraw[i], vraw[i], slot);
  if (slot < 0 || slot >= a.num_blocks * a.block_size) return;
  const int64_t blk = slot / a.block_size;
  const int off = (int)(slot - blk * a.block_size);

  float kx[16], vx[16];
#pragma unroll
  for (int i = 0; i < 16 / SPL; ++i) {
    widen16<SRC>(kraw[i], kx + SPL * i);
    widen16<SRC>(vraw[i], vx + SPL * i);
  }
  uint32_t kw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) kw[i / 4] |= fp8_e4m3_encode(kx[i] / a.k_scale) << (8 * (i % 4));

  const int64_t quad = (blk * a.num_kv_heads + h) * (a.block_size / 4) + off / 4;
  const int row = off % 4;
  char* kdst = reinterpret_cast<char*>(a.k_cache) + ((quad * chunks_per_row + c) * 4 + row) * 16;
  *reinterpret_cast<uint4*>(kdst) = uint4{kw[0], kw[1], kw[2], kw[3]};

  unsigned char* vrow = reinterpret_cast<unsigned char*>(a.v_cache) + (quad * D + e0) * 4 + row;
#pragma unroll
  for (int i = 0; i < 16; ++i) vrow[4 * i] = (unsigned char)fp8_e4m3_encode(vx[i] / a.v_scale);
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
