// decode_mfma.hip -- paged decode attention for a GQA head group on the matrix
// cores (v_mfma_f32_16x16x32_{bf16,f16}), for 16-bit KV caches.
//
// A grouped-query head group is a real dense tile: the g query heads that
// share a kv head multiply the same keys and values, so per 32-token chunk
//   S[token][head]   = K[token][:] . Q[head][:]        (2 tiles of 16 tokens)
//   O^T[dim][head]  += V^T[dim][token] . P^T[token][head]
// are small GEMMs with N = g (up to 16) columns.  Keys and values are still
// read from HBM once per kv head; the matrix cores take the multiply-adds off
// the vector ALUs, which then only run the online softmax ("vLLM Project
// Update" talk: PagedAttention over KV blocks; second kernel: sequences split
// into partitions merged "similar to flash decoding").
//
// Lane layout (one wave = one (sequence, kv head, partition) work item):
//   lane = 16*j + n, n in [0,16), j in [0,4).
//   QK^T: A = keys, row n = token tau(n) of the tile, k-slots = 8 dims at
//         32c + 8j; B = queries, column n = head n, same k-slots.
//         Result: lane (n, j) holds head n's scores of 4 tokens.  Tile A
//         rows are tokens 8*(i/4) + i%4, tile B rows the same + 4, so lane
//         (n, j) ends up with head n's scores for tokens 8j .. 8j+7.
//   P.V:  A = values from the [dim][block_size] value layout, row n = dim
//         16c + n, k-slots = tokens 8j .. 8j+7 (one contiguous 16-byte run);
//         B = probabilities, column n = head n, k-slots = the same tokens --
//         exactly the registers the QK^T result left in the lane, so no
//         shuffle is needed.  Result: lane (n, j) holds O^T[16c + 4j + r][n].
//   Every per-head quantity (running max, sum, rescale factor) therefore
//   lives in the lanes of column n.
//
// Precision: probabilities go to the matrix cores as hi + lo 16-bit parts
// (p = hi + lo with |lo| <= 2^-9 |p| for bf16), so P.V keeps ~16 significant
// bits; all accumulation is fp32.  p = 1 and p = 0 stay exact.
//
// Memory: the block ids of the current 64-block window are held one per lane
// and fetched with a lane shuffle; the keys and values of chunk i+1 are
// loaded while chunk i is computed (two register buffers).
#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

template <Elem E> struct Mma;
template <> struct Mma<Elem::BF16> {
  using vec8 = bf16x8_t;
  using scalar = __bf16;
  static __device__ __forceinline__ f32x4_t mma(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<Elem::F16> {
  using vec8 = f16x8_t;
  using scalar = _Float16;
  static __device__ __forceinline__ f32x4_t mma(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kChunk = 32;  // tokens per iteration

template <Elem KV, int D>
struct Buffers {
  using vec8 = typename Mma<KV>::vec8;
  vec8 k[2][D / 32];  // [tile][dim chunk]
  vec8 v[D / 16];     // [dim chunk]
};

template <Elem KV, int D, int G>
__global__ __launch_bounds__(64) void decode_mfma_kernel(DecodeArgs a) {
  using M = Mma<KV>;
  using vec8 = typename M::vec8;
  using scalar = typename M::scalar;
  constexpr int KC = D / 32;  // QK^T k-chunks
  constexpr int VC = D / 16;  // P.V row chunks
  constexpr int RB = D * 2;   // bytes per key row

  const int part = blockIdx.x;
  const int b = blockIdx.z;
  const int chunks = a.group / G;
  const int h = blockIdx.y / chunks;
  const int hq0 = h * a.group + (blockIdx.y % chunks) * G;
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int j = lane >> 4;

  const int L = clamp_len(a.context_lens[b], a.max_blocks_per_seq, a.block_size);
  const int P = a.partition_size;
  if (L <= 0) {
    if (part == 0) {
      for (int g = 0; g < G; ++g)
        for (int e = lane; e < D; e += 64)
          store_elem(a.out, ((int64_t)b * a.num_q_heads + hq0 + g) * D + e, 0.0f, a.out_dtype);
    }
    return;
  }
  const int n_parts = (L + P - 1) / P;
  if (part >= n_parts) return;
  const int t_begin = part * P;
  const int t_end = min(t_begin + P, L);
  const int lbs = a.log2_block_size;
  const int bs = a.block_size;
  const int last_blk = (L - 1) >> lbs;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  const int64_t head_tile = (int64_t)bs * D * 2;  // bytes of one (block, head) tile
  const char* kc = reinterpret_cast<const char*>(a.k_cache) + (int64_t)h * head_tile;
  const char* vc = reinterpret_cast<const char*>(a.v_cache) + (int64_t)h * head_tile;
  const int64_t block_stride = (int64_t)a.num_kv_heads * head_tile;

  // queries: column n = head hq0 + n (zero beyond the group)
  vec8 qv[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (n < G) {
      const char* qp = reinterpret_cast<const char*>(a.q) +
                       (((int64_t)b * a.num_q_heads + hq0 + n) * D + 32 * c + 8 * j) * 2;
      qv[c] = *reinterpret_cast<const vec8*>(qp);
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) qv[c][r] = (scalar)0.0f;
    }
  }

  // block-id window: lane i holds the physical block of logical block wb + i
  int wb = t_begin >> lbs;
  int bt_lane = (int)clamp_block(bt[min(wb + lane, last_blk)], a.num_blocks);

  // token of this lane's key row in tiles A and B, and of its value run
  const int tokA = 8 * (n >> 2) + (n & 3);
  const int tokB = tokA + 4;
  const int tokV = 8 * j;

  auto issue = [&](Buffers<KV, D>& buf, int t0) {
    const int need_last = min((t0 + kChunk - 1) >> lbs, last_blk);
    if (need_last - wb >= 64) {  // slide the block-id window (uniform)
      wb = t0 >> lbs;
      bt_lane = (int)clamp_block(bt[min(wb + lane, last_blk)], a.num_blocks);
    }
    const int ta = t0 + tokA, tb = t0 + tokB, tv = t0 + tokV;
    const int pa_ = __shfl(bt_lane, min(ta >> lbs, last_blk) - wb);
    const int pb_ = __shfl(bt_lane, min(tb >> lbs, last_blk) - wb);
    const int pv_ = __shfl(bt_lane, min(tv >> lbs, last_blk) - wb);
    const char* ka = kc + (int64_t)pa_ * block_stride + (int64_t)(ta & (bs - 1)) * RB + 16 * j;
    const char* kb = kc + (int64_t)pb_ * block_stride + (int64_t)(tb & (bs - 1)) * RB + 16 * j;
    const char* vp = vc + (int64_t)pv_ * block_stride + ((int64_t)n * bs + (tv & (bs - 1))) * 2;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      buf.k[0][c] = *reinterpret_cast<const vec8*>(ka + 64 * c);
      buf.k[1][c] = *reinterpret_cast<const vec8*>(kb + 64 * c);
    }
#pragma unroll
    for (int c = 0; c < VC; ++c)
      buf.v[c] = *reinterpret_cast<const vec8*>(vp + (int64_t)c * 16 * bs * 2);
  };

  f32x4_t o[VC];
#pragma unroll
  for (int c = 0; c < VC; ++c) o[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY;  // running max of head n (log2 domain), uniform over j
  float lsum = 0.0f;    // this lane's share of head n's sum

  auto compute = [&](Buffers<KV, D>& buf, int t0) {
    f32x4_t sa = {0.0f, 0.0f, 0.0f, 0.0f}, sb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      sa = M::mma(buf.k[0][c], qv[c], sa);
      sb = M::mma(buf.k[1][c], qv[c], sb);
    }
    float s[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = sa[r] * a.scale_log2;
      s[4 + r] = sb[r] * a.scale_log2;
    }
    const bool tail = t0 + kChunk > t_end;
    if (tail) {  // uniform: mask tokens past the partition / context
      const int nv = t_end - t0 - 8 * j;  // valid tokens of this lane's run
#pragma unroll
      for (int r = 0; r < 8; ++r) s[r] = r < nv ? s[r] : -INFINITY;
#pragma unroll
      for (int c = 0; c < VC; ++c)
#pragma unroll
        for (int r = 0; r < 8; ++r)
          if (r >= nv) buf.v[c][r] = (scalar)0.0f;
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    vec8 phi, plo;
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float p = fast_exp2(s[r] - m_new);
      ps += p;
      const scalar hi = (scalar)p;
      phi[r] = hi;
      plo[r] = (scalar)(p - (float)hi);
    }
    lsum = lsum * alpha + ps;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < VC; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[c][r] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      o[c] = M::mma(buf.v[c], phi, o[c]);
      o[c] = M::mma(buf.v[c], plo, o[c]);
    }
  };

  Buffers<KV, D> b0, b1;
  int t0 = t_begin;
  issue(b0, t0);
  for (;;) {
    if (t0 + kChunk < t_end) issue(b1, t0 + kChunk);
    compute(b0, t0);
    t0 += kChunk;
    if (t0 >= t_end) break;
    if (t0 + kChunk < t_end) issue(b0, t0 + kChunk);
    compute(b1, t0);
    t0 += kChunk;
    if (t0 >= t_end) break;
  }

  // ---- finish the work item ------------------------------------------------
  float l = lsum + __shfl_xor(lsum, 16);
  l += __shfl_xor(l, 32);
  if (n < G) {
    const int64_t row_id = (int64_t)b * a.num_q_heads + hq0 + n;
    if (n_parts == 1) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int c = 0; c < VC; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store_elem(a.out, row_id * D + 16 * c + 4 * j + r, o[c][r] * inv, a.out_dtype);
    } else {
      const int64_t slot = row_id * a.max_partitions + part;
      float* dst = a.ws_acc + slot * D;
#pragma unroll
      for (int c = 0; c < VC; ++c)
        *reinterpret_cast<f32x4_t*>(dst + 16 * c + 4 * j) = o[c];
      if (j == 0) {
        a.ws_ml[slot * 2] = m;
        a.ws_ml[slot * 2 + 1] = l;
      }
    }
  }
}

template <Elem KV, int D>
hipError_t dispatch_g(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  switch (a.heads_per_item) {
#define PA_CASE(GG)                                                               \
  case GG:                                                                        \
    hipLaunchKernelGGL((decode_mfma_kernel<KV, D, GG>), grid, dim3(64), 0, s, a); \
    break;
    PA_CASE(1) PA_CASE(2) PA_CASE(4) PA_CASE(8) PA_CASE(16)
    PA_CASE(3) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(10) PA_CASE(12)
#undef PA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool mfma_supports_heads(int heads_per_item) {
  switch (heads_per_item) {
    case 1: case 2: case 3: case 4: case 5: case 6: case 7: case 8: case 10: case 12: case 16:
      return true;
    default:
      return false;
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int kv_dtype, int head_dim, hipStream_t s) {
  const int chunks = a.group / a.heads_per_item;
  dim3 grid((unsigned)a.max_partitions, (unsigned)(a.num_kv_heads * chunks), (unsigned)a.num_seqs);
  if (kv_dtype == 2) {
    if (head_dim == 128) return dispatch_g<Elem::BF16, 128>(a, grid, s);
    if (head_dim == 64) return dispatch_g<Elem::BF16, 64>(a, grid, s);
  } else if (kv_dtype == 1) {
    if (head_dim == 128) return dispatch_g<Elem::F16, 128>(a, grid, s);
    if (head_dim == 64) return dispatch_g<Elem::F16, 64>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
