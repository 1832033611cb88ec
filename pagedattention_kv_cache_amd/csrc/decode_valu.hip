// decode_valu.hip -- paged single-query decode attention on the vector ALUs.
//
// A workgroup of 1, 2 or 4 waves handles one work item: a (sequence, kv head,
// partition) with all the query heads of that kv head's group (or a chunk of
// at most 8 of them), so every key/value byte of the item is read from HBM
// once.  Wave w takes tiles w, w + W, ... with its own softmax state; the
// waves' partial results are merged through LDS by log-sum-exp at the end.  Tokens
// are walked in tiles of 16 through the block table ("vLLM Project Update"
// talk, PagedAttention recap: attention over fixed-size blocks of the KV
// cache); a partition covers partition_size tokens and long or uneven contexts
// are split into several partitions merged later by log-sum-exp (same talk,
// second PagedAttention kernel, which the talk likens to flash decoding).
//
// Per tile:
//  * scores: a key row (head_dim * elem bytes) is spread over RL = row/16
//    lanes holding one 16-byte chunk each, TPI = 64/RL tokens per load
//    instruction (with the token-quad key layout the lanes of one
//    instruction read one contiguous run); each lane forms partial dots for
//    every head of the group and a DPP butterfly within the row completes
//    them;
//  * online softmax in the exp2 domain (scale * log2 e folded into the
//    scores): the tile max is made wave-uniform, so the running max m, the
//    rescale factor and the accumulator rescale are uniform per head;
//  * the tile's probabilities go through LDS (broadcast reads) and each lane
//    accumulates p * v for head_dim/64 output dims from the value cache's
//    [quad][dim][4] layout: the four tokens of a quad of one dim are one
//    contiguous run, and consecutive lanes read consecutive dims.
// Memory: the block ids of a 64-block window sit one per lane and are read
// with readlane; each 8-token segment of a tile gets a buffer resource at its
// block, so lanes only add fixed 32-bit offsets; tile i+1 is loaded while
// tile i is computed.
// Masking is by selection (score -inf, value term skipped), never by
// multiplying by zero, so unused cache slots may hold anything (even NaN).
#include "pa_device.hpp"
#include "pa_launch.hpp"
#include "work_list.hpp"

namespace pa {
namespace {

constexpr int kTile = 16;

// Four tokens of one value dim: 4 bytes for E4M3, 8 for the 16-bit types,
// 16 for fp32.
template <int EB> struct QuadRaw;
template <> struct QuadRaw<1> { using type = uint32_t; };
template <> struct QuadRaw<2> { using type = uint2; };
template <> struct QuadRaw<4> { using type = uint4; };

// A lane's piece of a key row: one 16-byte chunk (16-bit and fp32 caches) or
// half of one (E4M3, so that a row still spans at least 8 lanes).
template <int EB> struct KeyPiece { using type = uint4; static constexpr int bytes = 16; };
template <> struct KeyPiece<1> { using type = uint2; static constexpr int bytes = 8; };

template <Elem KV, int D>
struct Tile {
  static constexpr int EB = ElemTraits<KV>::bytes;
  static constexpr int KB = KeyPiece<EB>::bytes;  // key bytes per lane and token
  static constexpr int RL = D * EB / KB;          // lanes per key row
  static constexpr int CPR = D * EB / 16;         // 16-byte key chunks per row
  static constexpr int NI = kTile / (64 / RL);    // key load instructions per tile
  static constexpr int DPL = D / 64;              // value dims per lane
  using VQ = typename QuadRaw<EB>::type;
  typename KeyPiece<EB>::type k[NI];
  VQ v[4][DPL];  // [token quad of the tile][owned dim]
};

// Byte offset of lane piece c of the key of token `row` (quad row/4, row
// row%4) from its token quad.
template <Elem KV, int D>
__device__ __forceinline__ int key_piece_off(int row, int c) {
  using T = Tile<KV, D>;
  if constexpr (T::KB == 16) return ((row >> 2) * T::CPR + c) * 64 + (row & 3) * 16;
  else return ((row >> 2) * T::CPR + (c >> 1)) * 64 + (row & 3) * 16 + (c & 1) * 8;
}

template <Elem KV>
__device__ __forceinline__ void widen_key(const uint4& raw, float* out) {
  widen16<KV>(raw, out);
}
template <Elem KV>
__device__ __forceinline__ void widen_key(const uint2& raw, float* out) {
  widen8_fp8(raw, out);
}

__device__ __forceinline__ uint4 load_key(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                          uint4*) {
  return buf_ld16(r, voff, soff);
}
__device__ __forceinline__ uint2 load_key(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                          uint2*) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

template <Elem KV>
__device__ __forceinline__ void widen_quad(const uint32_t& r, float* out) {
  fp8x4_to_f32(r, out);
}
template <Elem KV>
__device__ __forceinline__ void widen_quad(const uint2& r, float* out) {
  out[0] = lo_to_f32<KV>(r.x);
  out[1] = hi_to_f32<KV>(r.x);
  out[2] = lo_to_f32<KV>(r.y);
  out[3] = hi_to_f32<KV>(r.y);
}
template <Elem KV>
__device__ __forceinline__ void widen_quad(const uint4& r, float* out) {
  out[0] = __uint_as_float(r.x);
  out[1] = __uint_as_float(r.y);
  out[2] = __uint_as_float(r.z);
  out[3] = __uint_as_float(r.w);
}

template <int EB>
__device__ __forceinline__ typename QuadRaw<EB>::type buf_ld_quad(__amdgpu_buffer_rsrc_t r,
                                                                  int voff, int soff);
template <>
__device__ __forceinline__ uint32_t buf_ld_quad<1>(__amdgpu_buffer_rsrc_t r, int voff,
                                                   int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
template <>
__device__ __forceinline__ uint2 buf_ld_quad<2>(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
template <>
__device__ __forceinline__ uint4 buf_ld_quad<4>(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return buf_ld16(r, voff, soff);
}

template <Elem KV, int D, int G>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs args) {
  using T = Tile<KV, D>;
  constexpr int EB = T::EB;
  constexpr int EPL = T::KB / EB;  // key elements per lane piece
  constexpr int RL = T::RL;        // lanes per key row
  constexpr int CPR = T::CPR;      // 16-byte key chunks per row
  constexpr int TPI = 64 / RL;     // tokens per key load instruction
  constexpr int NI = T::NI;
  constexpr int DPL = T::DPL;
  constexpr int SEG = 8;           // tokens per load segment (one block)
  constexpr int NSEG = kTile / SEG;
  static_assert(RL >= 8 && RL <= 64 && 64 % RL == 0, "row layout");
  static_assert(TPI <= SEG, "a key load instruction stays inside one block");


  __shared__ float p_lds_all[4][G][kTile];

  // Work items (sequence, kv head, head chunk, partition).  With a work list
  // (a.list_ints > 0) the grid is persistent: every workgroup builds the list
  // of the items that hold tokens and takes every gridDim.x-th one, head
  // chunks fastest.  Without one, each workgroup runs one item: grid.x walks
  // (sequence, kv head, head chunk) fastest so that consecutive workgroups --
  // which the dispatcher deals round-robin to the XCDs -- carry the same
  // partition index of different sequences and heads, and grid.y walks the
  // partitions from the last to the first.
  extern __shared__ __align__(16) int dyn_lds[];
  const bool listed = args.list_ints > 0;
  int n_work = (int)blockIdx.x + 1, step = 1;
  if (listed) {
    n_work = build_work_list(args, dyn_lds) * args.num_kv_heads *
             (args.group / args.heads_per_item);
    step = (int)gridDim.x;
  }
  if (args.order_ctr) n_work = 0x7fffffff;  // a dynamic deal: until the order runs out
  if (args.order_static) {                   // a static deal: until the order runs out
    n_work = 0x7fffffff;
    step = (int)gridDim.x;
  }
  __shared__ int ticket_lds[2];
  // Round r takes entry r * gridDim.x + blockIdx.x, or the mirrored one on
  // odd rounds: the list runs longest first, so a workgroup that drew a long
  // entry in one round draws a short one in the next (a snake deal).
  int cursor = 0;
  const int bx = (int)blockIdx.x;
  int round = 0, it = bx;
  // with a partition picked on the device: the number of entries in the
  // order, from the item before, so that a ticket past it ends the workgroup
  // without reading the entry (a last dependent load that cost 2% where every
  // workgroup has one item)
  int order_total = 0x7fffffff;
  while (it < n_work) {
    {
    KernArgs& a = *fresh_args();
    // rows: G = Q x Gh, row g = (query g / Gh, head hq0 + g % Gh)
    const int Q = a.num_queries;
    const int Gh = a.heads_per_item;
    const int chunks = a.group / Gh;
    const int per_seq = a.num_kv_heads * chunks;
    const int W = a.waves;
    const int tid = fresh_tid();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    float* red = reinterpret_cast<float*>(dyn_lds + a.list_ints);  // wave merge area
    float (*p_lds)[kTile] = p_lds_all[wave];  // this wave's tile probabilities
    const int c = lane % RL;    // 16-byte chunk of the key row
    const int row = lane / RL;  // token within a key load instruction
    const int lbs = a.log2_block_size;
    const int bs = a.block_size;
    int P = a.partition_size;  // or the ordering kernel's pick (below)
    const int64_t head_tile = (int64_t)bs * D * EB;  // bytes of one (block, head) tile
    const int64_t block_stride = (int64_t)a.num_kv_heads * head_tile;

    // per-lane byte offsets from a segment's first token quad: key chunk c of
    // token `row` (quad row/4, row row%4); the value quad of each owned dim
    const int koff = key_piece_off<KV, D>(row, c);
    int voff[DPL];
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) voff[dd] = (dd * 64 + lane) * 4 * EB;

    int b, hc, part;
    if (listed) {
      const int item = it / per_seq;
      hc = it - item * per_seq;
      work_item(dyn_lds, a.max_partitions, item, cursor, b, part);
    } else if (a.order) {
      const int64_t lin = a.order_ctr || a.order_static
                              ? (int64_t)it
                              : (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
      const int64_t e = lin / per_seq;
      hc = (int)(lin - e * per_seq);
      if (e < 0 || e >= (int64_t)a.num_seqs * a.max_partitions || e >= order_total)
        break;  // past the order
      const int entry = a.order[e];
      if (a.part_dev) {
        // the partition the ordering kernel picked and its entry count, loaded
        // beside the entry (a load of their own first cost a round trip)
        P = partition_of(a);
        order_total = __builtin_amdgcn_readfirstlane(a.part_dev[1]);
      }
      // -1: every item is taken; an entry out of range (an order the caller
      // said was prepared and was not) ends the workgroup rather than a read
      if (entry < 0 || entry >= a.num_seqs * a.max_partitions) break;
      b = entry / a.max_partitions;
      part = entry - b * a.max_partitions;
    } else {
      b = it / per_seq;
      hc = it - b * per_seq;
      part = (int)gridDim.y - 1 - (int)blockIdx.y;
    }
    const int h = hc / chunks;
    const int hq0 = h * a.group + (hc % chunks) * Gh;
    auto row_of = [&](int g) -> int64_t {
      return ((int64_t)b * Q + g / Gh) * a.num_q_heads + hq0 + g % Gh;
    };

    // start-up loads that do not depend on the context length go out with it
    const int t_begin = part * P;
    const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
    const int L_in = a.context_lens[b];
    const int bt_first = bt[min((t_begin >> lbs) + lane, a.max_blocks_per_seq - 1)];

    // query chunk for every head of the group, widened to fp32
    float qf[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t qb = row_of(g) * D + c * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[g][e] = load_elem_f32(a.q, qb + e, a.q_dtype);
    }

    const int L = clamp_len(L_in, a.max_blocks_per_seq, a.block_size);
    if (L <= 0) {
      if (part == 0 && wave == 0) {
        for (int g = 0; g < G; ++g)
          for (int e = lane; e < D; e += 64)
            store_elem(a.out, row_of(g) * D + e, 0.0f, a.out_dtype);
      }
      goto next_item;
    }
    const int n_parts = (L + P - 1) / P;
    if (part >= n_parts) goto next_item;
    const int t_end = min(t_begin + P, L);
    const int last_blk = (L - 1) >> lbs;
    // query g / Gh sits at position L - Q + g / Gh and sees the positions up to it
    const int lim_lo = L - Q + 1;
    const char* kc = reinterpret_cast<const char*>(a.k_cache) + (int64_t)h * head_tile;
    const char* vc = reinterpret_cast<const char*>(a.v_cache) + (int64_t)h * head_tile;

    int wb = t_begin >> lbs;  // block-id window: lane i holds the block of wb + i
    int bt_lane = (int)clamp_block(bt_first, a.num_blocks);

    // Loads of one 16-token tile (two 8-token segments, each inside one block),
    // through buffer resources based at each segment.  Always issued; the
    // prefetch past the last tile reads through an empty range (zeros, no
    // memory access), so the wait counts are the same on every path.
    auto issue = [&](T& buf, int t0, bool none) {
      const int range = none ? 0 : 0x7fffffff;
      __amdgpu_buffer_rsrc_t rk[NSEG], rv[NSEG];
#pragma unroll
      for (int sgm = 0; sgm < NSEG; ++sgm) {
        const int tok = t0 + sgm * SEG;
        const int phys = __builtin_amdgcn_readlane(bt_lane, min(tok >> lbs, last_blk) - wb);
        const int64_t first_quad =
            (int64_t)phys * block_stride + (int64_t)(tok & (bs - 1)) * D * EB;
        rk[sgm] = make_rsrc(kc + first_quad, range);
        rv[sgm] = make_rsrc(vc + first_quad, range);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int sgm = (i * TPI) / SEG;
        const int l0 = (i * TPI) % SEG;  // first token of the instruction inside the segment
        buf.k[i] = load_key(rk[sgm], koff, (l0 >> 2) * CPR * 64 + (l0 & 3) * 16, &buf.k[i]);
      }
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd)
          buf.v[qd][dd] = buf_ld_quad<EB>(rv[qd >> 1], voff[dd], (qd & 1) * D * 4 * EB);
    };

    float m[G], lrow[G], acc[G][DPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      lrow[g] = 0.0f;
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) acc[g][dd] = 0.0f;
    }

    auto compute = [&](T& buf, int t0, int t_stop) {
      // ---- scores ----------------------------------------------------------
      float s[G][NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float kf[EPL];
        widen_key<KV>(buf.k[i], kf);
        const int t = t0 + i * TPI + row;
        const bool valid = t < t_stop;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float part_dot = 0.0f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) part_dot = fmaf(qf[g][e], kf[e], part_dot);
          const float dot = group_sum<RL>(part_dot);
          s[g][i] = valid && t < lim_lo + g / Gh ? dot * a.scale_log2 : -INFINITY;
        }
      }

      // ---- online softmax (wave-uniform max per head) ---------------------
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = s[g][0];
#pragma unroll
        for (int i = 1; i < NI; ++i) mx = fmaxf(mx, s[g][i]);
        mx = across_groups_max<RL>(mx);
        const float m_new = fmaxf(m[g], mx);
        // a row with every score so far masked keeps m = -inf: exponents are
        // then taken against 0 so that they give 0, not NaN
        const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m[g] - m_ref);
        m[g] = m_new;
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          s[g][i] = fast_exp2(s[g][i] - m_ref);
          psum += s[g][i];
        }
        lrow[g] = lrow[g] * alpha + psum;
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) acc[g][dd] *= alpha;
      }
      wave_lds_sync();  // the previous tile's probabilities have been read
      if (c == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int i = 0; i < NI; ++i) p_lds[g][i * TPI + row] = s[g][i];
      }
      wave_lds_sync();

      // ---- p . V -------------------------------------------------------------
      const int nv = min(kTile, t_stop - t0);  // valid tokens in this tile
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) {
          float vf[4];
          widen_quad<KV>(buf.v[qd][dd], vf);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = qd * 4 + r;
            if (t < nv) {
#pragma unroll
              for (int g = 0; g < G; ++g) acc[g][dd] = fmaf(p_lds[g][t], vf[r], acc[g][dd]);
            }
          }
        }
      }
    };

    // Walk the partition in windows of 64 blocks; inside a window this wave
    // takes every W-th tile, loading its next tile while the current one is
    // computed.  Only the last window can hold fewer than W tiles.
    T b0, b1;
    const int window = 64 * bs;
    const int stride = W * kTile;
    for (int w0 = t_begin; w0 < t_end; w0 += window) {
      const int w1 = min(w0 + window, t_end);
      if (w0 != t_begin) {
        wb = w0 >> lbs;
        bt_lane = (int)clamp_block(bt[min(wb + lane, last_blk)], a.num_blocks);
      }
      const int nt = (w1 - w0 + kTile - 1) / kTile;
      if (wave >= nt) continue;
      const int nk = (nt - wave + W - 1) / W;  // tiles of this wave
      const int first_t0 = w0 + wave * kTile;
      const int last_t0 = first_t0 + (nk - 1) * stride;
      issue(b0, first_t0, false);
      for (int i = 0; i < nk; i += 2) {
        const int t0 = first_t0 + i * stride;
        issue(b1, min(t0 + stride, last_t0), t0 + stride > last_t0);
        compute(b0, t0, w1);
        if (i + 1 >= nk) break;
        issue(b0, min(t0 + 2 * stride, last_t0), t0 + 2 * stride > last_t0);
        compute(b1, t0 + stride, w1);
      }
    }

    // ---- finish the work item ------------------------------------------------
    float lsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) lsum[g] = across_groups_sum<RL>(lrow[g]);
    if (W > 1) {
      // Merge the waves by log-sum-exp (a wave without tokens for a row has
      // m = -inf, l = 0 and zero accumulators; when no wave has any, the row's
      // l is 0 and exponents are taken against 0): every wave parks its m, l
      // and accumulators in LDS, then the whole workgroup rescales, sums and
      // stores.
      float* red_m = red;               // [W][G]
      float* red_l = red + 4 * G;       // [W][G]
      float* red_o = red + 8 * G;       // [W][G][D]
      if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          red_m[wave * G + g] = m[g];
          red_l[wave * G + g] = lsum[g];
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) red_o[(wave * G + g) * D + dd * 64 + lane] = acc[g][dd];
      __syncthreads();
      for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
        const int g = e / D, d = e - g * D;
        float Mg = -INFINITY;
        for (int w = 0; w < W; ++w) Mg = fmaxf(Mg, red_m[w * G + g]);
        const float Mref = Mg == -INFINITY ? 0.0f : Mg;
        float lt = 0.0f, x = 0.0f;
        for (int w = 0; w < W; ++w) {
          const float sc = fast_exp2(red_m[w * G + g] - Mref);
          lt += red_l[w * G + g] * sc;
          x += red_o[(w * G + g) * D + d] * sc;
        }
        const int64_t row_id = row_of(g);
        if (n_parts == 1) {
          store_elem(a.out, row_id * D + d, lt > 0.0f ? x * a.v_scale / lt : 0.0f, a.out_dtype);
        } else {
          const int64_t slot = row_id * a.max_partitions + part;
          a.ws_acc[slot * D + d] = x * a.v_scale;
          if (d == 0) {
            a.ws_ml[slot * 2] = Mg;
            a.ws_ml[slot * 2 + 1] = lt;
          }
        }
      }
      __syncthreads();  // the merge area is free for the next item
      goto next_item;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float l = lsum[g];
      const int64_t row_id = row_of(g);
      if (n_parts == 1) {
        const float inv = l > 0.0f ? a.v_scale / l : 0.0f;  // l = 0: a query before position 0
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd)
          store_elem(a.out, row_id * D + dd * 64 + lane, acc[g][dd] * inv, a.out_dtype);
      } else {
        const int64_t slot = row_id * a.max_partitions + part;
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd)
          a.ws_acc[slot * D + dd * 64 + lane] = acc[g][dd] * a.v_scale;
        if (lane == 0) {
          a.ws_ml[slot * 2] = m[g];
          a.ws_ml[slot * 2 + 1] = l;
        }
      }
    }
    }
  next_item:
    if (KernArgs& a = *fresh_args(); a.order_ctr) {
      // A dynamic deal asks for the next item here, at the end of this one:
      // asked for with the start-up loads instead, the counter's latency
      // under contention held them back (measured 10% slower).
      if (threadIdx.x == 0) ticket_lds[round & 1] = take_ticket(a.order_ctr);
      if (a.waves > 1) __syncthreads();
      it = (int)gridDim.x + ticket_lds[round & 1];
      ++round;
      continue;
    }
    if (!listed && !fresh_args()->order_static) break;
    ++round;
    it = round * step + ((round & 1) ? step - 1 - bx : bx);
  }  // work items
}

// LDS of the wave merge: m and l of up to 4 waves, then every wave's
// accumulators.
size_t merge_lds_bytes(int waves, int heads, int head_dim) {
  if (waves <= 1) return 0;
  return ((size_t)8 * heads + (size_t)waves * heads * head_dim) * sizeof(float);
}

template <Elem KV, int D>
hipError_t dispatch_g(const DecodeArgs& a, int64_t items_x, hipStream_t s) {
  const int rows = a.num_queries * a.heads_per_item;  // rows per item (template G)
  const size_t lds = (size_t)a.list_ints * sizeof(int) + merge_lds_bytes(a.waves, rows, D);
  const void* fn = nullptr;
  switch (rows) {
#define PA_CASE(GG)                                                       \
  case GG:                                                                \
    fn = reinterpret_cast<const void*>(&decode_valu_kernel<KV, D, GG>);   \
    break;
    PA_CASE(1) PA_CASE(2) PA_CASE(3) PA_CASE(4) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(8)
#undef PA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return launch_decode_grid(fn, a, items_x, lds, s);
}

template <Elem KV>
hipError_t dispatch_d(const DecodeArgs& a, int head_dim, int64_t items_x, hipStream_t s) {
  if (head_dim == 64) return dispatch_g<KV, 64>(a, items_x, s);
  if (head_dim == 128) return dispatch_g<KV, 128>(a, items_x, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, int kv_dtype, int head_dim, hipStream_t s) {
  const int64_t items_x = (int64_t)a.num_seqs * a.num_kv_heads * (a.group / a.heads_per_item);
  switch (kv_dtype) {
    case 0: return dispatch_d<Elem::F32>(a, head_dim, items_x, s);
    case 1: return dispatch_d<Elem::F16>(a, head_dim, items_x, s);
    case 2: return dispatch_d<Elem::BF16>(a, head_dim, items_x, s);
    case 3: return dispatch_d<Elem::FP8>(a, head_dim, items_x, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
