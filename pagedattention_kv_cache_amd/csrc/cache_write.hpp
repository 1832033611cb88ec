// cache_write.hpp -- the per-thread body of the paged KV-cache slot write,
// shared by the write kernel and the fused write + item-ordering launch.
//
// Every new token's key and value rows go to the slot the caller assigned
// ("[core] Multi Step Scheduling" pull request, advance_step review thread:
// slot_mapping next to block_tables and block_size).  A bit copy, no
// arithmetic on values.  Thread gid moves one 16-byte chunk of one (token, kv
// head) row; tokens of a block are kept in quads of four consecutive offsets.
#pragma once

#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {

template <int EB>
__device__ __forceinline__ void cache_write_chunk(const CacheWriteArgs& a, int64_t gid,
                                                  int chunks_per_row) {
  const int64_t per_token = (int64_t)a.num_kv_heads * chunks_per_row;
  const int64_t total = a.num_tokens * per_token;
  if (gid >= total) return;
  const int64_t t = gid / per_token;
  const int rem = (int)(gid - t * per_token);
  const int h = rem / chunks_per_row;
  const int c = rem - h * chunks_per_row;
  constexpr int EPC = 16 / EB;  // elements per chunk
  const int64_t D = a.head_dim;
  const int e0 = c * EPC;
  // the source rows and the slot go out together (the rows do not depend on
  // the slot): one round trip before the stores instead of two
  const char* ksrc = reinterpret_cast<const char*>(a.k) + ((t * a.k_stride) + h * D + e0) * EB;
  const char* vsrc = reinterpret_cast<const char*>(a.v) + ((t * a.v_stride) + h * D + e0) * EB;
  const uint4 kraw = ld16(ksrc);
  const uint4 vraw = ld16(vsrc);
  const int64_t slot = a.slots[t];
  loaded_here(kraw, vraw, slot);
  // negative = padding; a slot past the pool breaks the caller's contract and
  // is dropped rather than written out of bounds
  if (slot < 0 || slot >= a.num_blocks * a.block_size) return;
  const int64_t blk = slot / a.block_size;
  const int off = (int)(slot - blk * a.block_size);

  const int64_t quad = (blk * a.num_kv_heads + h) * (a.block_size / 4) + off / 4;
  const int row = off % 4;
  char* kdst = reinterpret_cast<char*>(a.k_cache) + ((quad * chunks_per_row + c) * 4 + row) * 16;
  *reinterpret_cast<uint4*>(kdst) = kraw;

  char* vrow = reinterpret_cast<char*>(a.v_cache) + ((quad * D + e0) * 4 + row) * EB;
  const int64_t vstep = 4 * EB;  // next dim of the same row
  if constexpr (EB == 4) {
    const uint32_t w[4] = {vraw.x, vraw.y, vraw.z, vraw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(vrow + i * vstep) = w[i];
  } else {
    const uint32_t w[4] = {vraw.x, vraw.y, vraw.z, vraw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint16_t*>(vrow + (2 * i) * vstep) = (uint16_t)(w[i] & 0xffffu);
      *reinterpret_cast<uint16_t*>(vrow + (2 * i + 1) * vstep) = (uint16_t)(w[i] >> 16);
    }
  }
}

// The quantizing write into E4M3 caches, one thread per 16-element key chunk
// of one (token, kv head) row: each element x becomes e4m3(x / scale) (an IEEE
// fp32 division, correctly rounded, then fp8_e4m3_encode); key chunk c of the
// token at offset o lands at ((o/4 * chunks + c) * 4 + o%4) * 16 bytes into the
// (block, head) tile, the chunk's 16 value elements at consecutive dims of row
// o%4, 4 bytes apart.  Shared by the E4M3 write kernel and the E4M3 write +
// order launch.
template <Elem SRC>
__device__ __forceinline__ void cache_write_fp8_chunk(const CacheWriteArgs& a, int64_t gid,
                                                      int chunks_per_row) {
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

}  // namespace pa
