// pa_device.hpp -- gfx950 device helpers shared by the paged-attention kernels.
//
// Element types are carried as raw bits (uint8_t for E4M3, uint16_t for
// f16/bf16, float for f32) and widened to fp32 with exact conversions; all
// accumulation is fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// FP8: OCP 8-bit float E4M3 (bias 7, 3 significand bits, largest finite 448,
// no infinities), a cache storage type only.
enum class Elem : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };

template <Elem E> struct ElemTraits;
template <> struct ElemTraits<Elem::F32> { static constexpr int bytes = 4; };
template <> struct ElemTraits<Elem::F16> { static constexpr int bytes = 2; };
template <> struct ElemTraits<Elem::BF16> { static constexpr int bytes = 2; };
template <> struct ElemTraits<Elem::FP8> { static constexpr int bytes = 1; };

// ---- E4M3 ----------------------------------------------------------------
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float fp8_f32x2_t;

// The four E4M3 values packed in a dword, widened exactly to fp32 by the
// hardware conversion (gfx950 converts the OCP E4M3 format).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out) {
  const fp8_f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const fp8_f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// fp32 -> E4M3, nearest value with ties to the even significand, magnitudes
// beyond 448 (infinities too) saturating to +-448, NaN to the NaN pattern of
// its sign.  Integer/exact-float steps only, so the result does not depend on
// any conversion mode: below 2^-6 the values are the multiples of 2^-9 (code
// = the multiple, 8 being the smallest normal); above, a*2^(3-e) in [8, 16]
// is rounded and a carry into 16 moves to the next exponent.
__device__ __forceinline__ uint32_t fp8_e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = __builtin_fabsf(y);
  if (!(a == a)) return sign | 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
  const float m = __builtin_rintf(a * __uint_as_float((uint32_t)(127 + 3 - e) << 23));
  return sign | ((((uint32_t)(e + 7)) << 3) + ((uint32_t)m - 8u));
}

// ---- exact widening of the two 16-bit elements packed in one dword --------
template <Elem E> __device__ __forceinline__ float lo_to_f32(uint32_t w);
template <Elem E> __device__ __forceinline__ float hi_to_f32(uint32_t w);

template <> __device__ __forceinline__ float lo_to_f32<Elem::BF16>(uint32_t w) {
  return __uint_as_float(w << 16);
}
template <> __device__ __forceinline__ float hi_to_f32<Elem::BF16>(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
template <> __device__ __forceinline__ float lo_to_f32<Elem::F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <> __device__ __forceinline__ float hi_to_f32<Elem::F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Widen the 16 bytes held in `raw` into fp32: 4 values for f32, 8 for 16-bit.
template <Elem E>
__device__ __forceinline__ void widen16(const uint4& raw, float* out) {
  if constexpr (E == Elem::F32) {
    out[0] = __uint_as_float(raw.x);
    out[1] = __uint_as_float(raw.y);
    out[2] = __uint_as_float(raw.z);
    out[3] = __uint_as_float(raw.w);
  } else {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = lo_to_f32<E>(w[i]);
      out[2 * i + 1] = hi_to_f32<E>(w[i]);
    }
  }
}

// Widen the 8 E4M3 bytes held in `raw` into fp32.
__device__ __forceinline__ void widen8_fp8(const uint2& raw, float* out) {
  fp8x4_to_f32(raw.x, out);
  fp8x4_to_f32(raw.y, out + 4);
}

// One element of type E (at element index i of p) as fp32.
__device__ __forceinline__ float load_elem_f32(const void* p, int64_t i, int dtype) {
  if (dtype == 0) return reinterpret_cast<const float*>(p)[i];
  const uint16_t b = reinterpret_cast<const uint16_t*>(p)[i];
  if (dtype == 1) return (float)__builtin_bit_cast(_Float16, b);
  return __uint_as_float(((uint32_t)b) << 16);
}

// Store fp32 as dtype (round to nearest even for the 16-bit types).
__device__ __forceinline__ void store_elem(void* p, int64_t i, float x, int dtype) {
  if (dtype == 0) {
    reinterpret_cast<float*>(p)[i] = x;
  } else if (dtype == 1) {
    reinterpret_cast<_Float16*>(p)[i] = (_Float16)x;
  } else {
    reinterpret_cast<__bf16*>(p)[i] = (__bf16)x;
  }
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Holds loaded values to this point: an empty asm that reads them, so the
// loads are issued (and waited for) before it and cannot be sunk past a
// branch that follows, e.g. into the block that alone uses them.
__device__ __forceinline__ void loaded_here(const uint4& a, const uint4& b, int64_t c) {
  asm volatile("" ::"v"(a.x), "v"(a.y), "v"(a.z), "v"(a.w), "v"(b.x), "v"(b.y), "v"(b.z),
               "v"(b.w), "v"(c));
}

// 16-byte load with the non-temporal hint: cache data that is streamed once
// (keys and values) without displacing reused lines.
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw buffer resource over [base, base + range) bytes: 32-bit lane offsets,
// no swizzle, dword data format (the gfx9 raw-buffer word 3).  Loads past the
// range return zero without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int range) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, range, 0x00020000);
}

__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// ---- cross-lane reductions -----------------------------------------------
// DPP row (16-lane) butterflies: after the four steps every lane of a row
// holds the row's total.  Control codes are the GFX9 DPP encodings:
// quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over groups of N consecutive lanes (N = 1, 2, 4, 8, 16, 32, 64); every
// lane of a group gets the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);
  if constexpr (N >= 4) x += dpp<0x4E>(x);
  if constexpr (N >= 8) x += dpp<0x141>(x);
  if constexpr (N >= 16) x += dpp<0x140>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Max / sum across the 64/N groups of a wave for values that are already
// uniform within each group of N lanes.
template <int N>
__device__ __forceinline__ float across_groups_max(float x) {
  if constexpr (N <= 16) {
    if constexpr (N <= 8) x = fmaxf(x, __shfl_xor(x, 8));
    if constexpr (N <= 4) x = fmaxf(x, __shfl_xor(x, 4));
    if constexpr (N <= 2) x = fmaxf(x, __shfl_xor(x, 2));
    if constexpr (N <= 1) x = fmaxf(x, __shfl_xor(x, 1));
    x = fmaxf(x, __shfl_xor(x, 16));
  }
  if constexpr (N <= 32) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

template <int N>
__device__ __forceinline__ float across_groups_sum(float x) {
  if constexpr (N <= 16) {
    if constexpr (N <= 8) x += __shfl_xor(x, 8);
    if constexpr (N <= 4) x += __shfl_xor(x, 4);
    if constexpr (N <= 2) x += __shfl_xor(x, 2);
    if constexpr (N <= 1) x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 16);
  }
  if constexpr (N <= 32) x += __shfl_xor(x, 32);
  return x;
}

// Context length as the kernels use it: clamped to what the block table can
// address, so a length beyond the contract never walks past the table.
__device__ __forceinline__ int clamp_len(int L, int max_blocks_per_seq, int block_size) {
  const int cap = max_blocks_per_seq * block_size;
  return L < cap ? L : cap;
}

// A block-table entry clamped into the pool: entries inside a sequence's
// context must already be valid; the clamp only keeps a broken table from
// turning into an out-of-bounds access.
__device__ __forceinline__ int64_t clamp_block(int32_t phys, int64_t num_blocks) {
  int64_t p = phys < 0 ? 0 : (int64_t)phys;
  return p < num_blocks ? p : num_blocks - 1;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Orders one wave's LDS stores before its later LDS loads (and the reverse).
// A wave's LDS operations complete in issue order, so only the compiler has
// to be kept from moving them across this point; no other wave is waited for.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pa
