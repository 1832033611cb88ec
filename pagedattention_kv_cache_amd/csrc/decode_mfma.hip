// decode_mfma.hip -- paged decode attention for a GQA head group on the matrix
// cores (v_mfma_f32_16x16x32_{bf16,f16}), for 16-bit KV caches and for E4M3
// caches (widened exactly to bfloat16 in registers).
//
// A grouped-query head group is a real dense tile: the g query heads that
// share a kv head multiply the same keys and values, so per 16-token chunk
//   S[token][head]   = K[token][:] . Q[head][:]
//   O^T[dim][head]  += V^T[dim][token] . P^T[token][head]
// are small GEMMs with N = g (up to 16) columns.  Keys and values are still
// read from HBM once per kv head; the matrix cores take the multiply-adds off
// the vector ALUs, which then only run the online softmax ("vLLM Project
// Update" talk: PagedAttention over KV blocks; second kernel: sequences split
// into partitions merged the way flash decoding merges them).
//
// Lane layout (per wave of a (sequence, kv head, partition) work item):
//   lane = 16*j + n, n in [0,16), j in [0,4).
//   Chunks of 16 tokens.
//   QK^T (16x16x32): A = keys, row n = token n of the chunk, k-slots = the 8
//         dims of key chunk 4c + j (the key cache keeps a 16-byte chunk of
//         four consecutive tokens contiguous and the chunks of a token quad
//         side by side, so the four lanes n of a quad and the four groups j
//         read one 256-byte run per quad); B = queries, column n = head n,
//         same k-slots.  Result: lane (n, j) holds head n's scores of tokens
//         4j .. 4j+3.
//   P.V (16x16x16): A = values from the [quad][dim][4] value layout, row
//         n = dim 16c + n, k-slots = tokens 4j .. 4j+3 (quad j of the chunk:
//         one 8-byte run); B = probabilities, column n = head n, k-slots = the
//         same tokens -- exactly the registers the QK^T result left in the
//         lane, so no shuffle is needed.  Result: lane (n, j) holds
//         O^T[16c + 4j + r][n].
//   Every per-head quantity (running max, sum, rescale factor) therefore
//   lives in the lanes of column n.
//
// Precision: probabilities go to the matrix cores as hi + lo 16-bit parts
// (p = hi + lo with |lo| <= 2^-9 |p| for bf16), so P.V keeps ~16 significant
// bits; all accumulation is fp32.  p = 1 and p = 0 stay exact.
//
// Memory: the block ids of the current 64-block window are held one per lane
// and fetched with a lane read; the keys and values of a wave's next chunk are
// loaded while its current chunk is computed (two register buffers).
//
// A work item may run on 1, 2 or 4 waves (one workgroup).  Wave w takes the
// chunks w, w + W, w + 2W, ... of the partition with its own running max, sum
// and accumulators, and at the end the waves' partial results are merged
// through LDS with the same log-sum-exp rule that merges partitions.  More
// waves per item shorten the longest items (one long sequence among short
// ones) at the price of a few more start-up loads.
#include "pa_device.hpp"
#include "pa_launch.hpp"
#include "work_list.hpp"

namespace pa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

template <Elem E> struct Mma;
template <> struct Mma<Elem::BF16> {
  using vec8 = bf16x8_t;
  using vec4 = bf16x4_t;
  using scalar = __bf16;
  // S += K(16x32) . Q(32x16)
  static __device__ __forceinline__ f32x4_t qk(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // O^T += V^T(16x16) . P^T(16x16)
  static __device__ __forceinline__ f32x4_t pv(vec4 a, vec4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<Elem::F16> {
  using vec8 = f16x8_t;
  using vec4 = f16x4_t;
  using scalar = _Float16;
  static __device__ __forceinline__ f32x4_t qk(vec8 a, vec8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(vec4 a, vec4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kChunk = 16;  // tokens per iteration: one 16-row QK^T tile

// Cache-policy bits of buffer loads: non-temporal.  A chunk consumes its key
// quads (256-byte runs) and its value quads (one 4 KiB run per 16-bit block)
// whole, and nothing reads them again in the launch.  Measured (decode
// kernel): keys on the default policy instead cost 9-10% on the GQA and MHA
// workloads; values non-temporal gained 0.6% (GQA lognormal batch) and 3% (MHA
// batch) and lost 0.5% on long contexts; E4M3 values on the default policy
// cost 3.7% (GQA lognormal batch) and 1.2% (long contexts).
constexpr int kNonTemporal = 2;


// How a lane's matrix operands of one chunk are stored in the caches, loaded
// and widened to the multiply type.  16-bit caches, per lane and 32-dim
// k-chunk c: the 8 dims 32c + 8j .. 32c + 8j + 7 of key token n (one 16-byte
// load); per 32-dim value group c: dims 32c + 2n and 32c + 2n + 1 of value
// tokens 4j .. 4j + 3 (one token quad, one 16-byte load), which feed the
// P.V row chunks 2c and 2c + 1.  E4M3 caches permute the dims within 64-dim
// groups (below).  Every operand load is 16 bytes: 8-byte value loads (one
// dim per lane) measured 0.3% slower on the GQA lognormal batch and 2.9% on
// the skewed batch.
template <Elem KV> struct Store;
template <Elem KV> struct Store16 {  // f16 / bf16: loaded as the multiply type
  using Math = Mma<KV>;
  using KRaw = typename Math::vec8;
  using VRaw = uint4;  // two dims x four tokens
  static constexpr int EB = 2;
  static constexpr int kstep = 256;  // bytes between k-chunks (4 key chunks of a quad row)
  static constexpr int vstep = 256;  // bytes between 32-dim value groups
  // one key load per 32-dim k-chunk c: lane group j holds dims 32c + 8j .. + 7
  static constexpr bool kPairK = false;
  static constexpr int kloads(int D) { return D / 32; }
  static __device__ __forceinline__ int qdim(int c, int j) { return 32 * c + 8 * j; }
  // one value load per 32-dim group: dims 2n, 2n + 1 of group c feed row
  // chunks 2c and 2c + 1; output row 4j + r of row chunk 2c + h is dim
  // 32c + 8j + 2r + h
  static constexpr int kVDims = 2;
  static constexpr int vloads(int D) { return D / 32; }
  static __device__ __forceinline__ int dim(int rc, int j, int r) {
    return 32 * (rc >> 1) + 8 * j + 2 * r + (rc & 1);
  }
  // offsets from the chunk's first token quad
  static __device__ __forceinline__ int koff(int n, int j, int D) {
    return ((n >> 2) * (D / 8) + j) * 64 + (n & 3) * 16;
  }
  static __device__ __forceinline__ int voff(int n, int j, int D) { return (j * D + 2 * n) * 8; }
  static __device__ __forceinline__ KRaw load_k(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(KRaw,
                              __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
  }
  static __device__ __forceinline__ VRaw load_v(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(VRaw,
                              __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
  }
  static __device__ __forceinline__ KRaw load_k(const char* p) {
    return __builtin_bit_cast(KRaw, ld16_nt(p));
  }
  static __device__ __forceinline__ VRaw load_v(const char* p) { return ld16(p); }
  static __device__ __forceinline__ typename Math::vec8 k(KRaw r, int) { return r; }
  // the four tokens of dim 2n + h
  static __device__ __forceinline__ typename Math::vec4 v(VRaw r, int h) {
    const uint2 w = h ? uint2{r.z, r.w} : uint2{r.x, r.y};
    return __builtin_bit_cast(typename Math::vec4, w);
  }
};
template <> struct Store<Elem::BF16> : Store16<Elem::BF16> {};
template <> struct Store<Elem::F16> : Store16<Elem::F16> {};
// E4M3: half the bytes per operand; widened exactly to bfloat16 (the queries
// are bfloat16) before the matrix cores see them.  Every load is 16 bytes, so
// a chunk takes half the load instructions of 8-byte pieces (measured: 1.6%
// on the GQA lognormal batch for the keys, 0.6% more for the values).
template <> struct Store<Elem::FP8> {
  using Math = Mma<Elem::BF16>;
  using KRaw = uint4;
  using VRaw = uint4;
  static constexpr int EB = 1;
  // Keys: one 16-byte load per lane covers two k-chunks.  Lane group j loads
  // key chunk 4p + j (dims 64p + 16j .. + 15) of its token; its first 8
  // codes feed k-chunk 2p, the last 8 k-chunk 2p + 1, and the queries are
  // loaded with the same dims (qdim), so each k-chunk still sums 32 dims.
  static constexpr bool kPairK = true;
  static constexpr int kloads(int D) { return D / 64; }
  static __device__ __forceinline__ int qdim(int c, int j) {
    return 64 * (c >> 1) + 16 * j + 8 * (c & 1);
  }
  static constexpr int kstep = 256;  // bytes between key loads (4 key chunks of a quad row)
  static constexpr int vstep = 256;  // bytes between 64-dim value groups
  // Values: one 16-byte load per lane covers four adjacent dims (4n .. 4n + 3
  // of a 64-dim group) of its token quad, so the 16 lanes of a quad read 256
  // contiguous bytes; the four dims feed four P.V products (row chunks 4c + h)
  static constexpr int kVDims = 4;
  static constexpr int vloads(int D) { return D / 64; }
  // row chunk rc = 4c + h holds dims 64c + 4n + h; output row 4j + r of it is
  // dim 64c + 16j + 4r + h
  static __device__ __forceinline__ int dim(int rc, int j, int r) {
    return 64 * (rc >> 2) + 16 * j + 4 * r + (rc & 3);
  }
  static __device__ __forceinline__ int koff(int n, int j, int D) {
    return ((n >> 2) * (D / 16) + j) * 64 + (n & 3) * 16;
  }
  static __device__ __forceinline__ int voff(int n, int j, int D) { return (j * D + 4 * n) * 4; }
  static __device__ __forceinline__ KRaw load_k(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(KRaw,
                              __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
  }
  static __device__ __forceinline__ VRaw load_v(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(VRaw,
                              __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
  }
  static __device__ __forceinline__ KRaw load_k(const char* p) { return ld16_nt(p); }
  static __device__ __forceinline__ VRaw load_v(const char* p) { return ld16(p); }
  // gfx950 widens two E4M3 codes straight to a bfloat16 pair (scale 1: no
  // scaling); every E4M3 value is exact in bfloat16.
  template <bool HI>
  static __device__ __forceinline__ uint32_t pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
  // k-chunk 2p + h: codes 8h .. 8h + 7 of the load
  static __device__ __forceinline__ Math::vec8 k(KRaw r, int h) {
    const uint32_t x = h ? r.z : r.x, y = h ? r.w : r.y;
    const uint4 w = {pair<false>(x), pair<true>(x), pair<false>(y), pair<true>(y)};
    return __builtin_bit_cast(Math::vec8, w);
  }
  // the four tokens of dim 4n + h
  static __device__ __forceinline__ Math::vec4 v(VRaw r, int h) {
    const uint32_t x = h == 0 ? r.x : h == 1 ? r.y : h == 2 ? r.z : r.w;
    const uint2 w = {pair<false>(x), pair<true>(x)};
    return __builtin_bit_cast(Math::vec4, w);
  }
};

template <Elem KV, int D>
struct Buffers {
  typename Store<KV>::KRaw k[Store<KV>::kloads(D)];  // key row pieces of this lane's token
  typename Store<KV>::VRaw v[Store<KV>::vloads(D)];  // 4-token value runs of the row chunks
};

// UB: every 16-token chunk lies in one cache block (block_size >= 16), so the
// chunk's base address is wave-uniform (scalar registers) and each lane only
// adds a fixed 32-bit offset; otherwise (block_size 8) lanes address their
// own blocks.
template <Elem KV, int D, int G, bool UB>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs args) {
  using St = Store<KV>;
  using M = typename St::Math;
  using vec8 = typename M::vec8;
  using vec4 = typename M::vec4;
  using scalar = typename M::scalar;
  constexpr int KC = D / 32;  // QK^T k-chunks
  constexpr int KL = St::kloads(D);  // key loads per chunk
  constexpr int VC = D / 16;  // P.V row chunks
  constexpr int VL = St::vloads(D);  // value loads per chunk
  constexpr int NT = (G + 15) / 16;  // 16-column tiles: every key and value load feeds all


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
    // columns: G = Q x Gh, column n = (query n / Gh, head hq0 + n % Gh)
    const int Q = a.num_queries;
    const int Gh = a.heads_per_item;
    const int chunks = a.group / Gh;
    const int per_seq = a.num_kv_heads * chunks;
    const int W = a.waves;
    const int tid = fresh_tid();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    float* red = reinterpret_cast<float*>(dyn_lds + a.list_ints);  // wave merge area
    const int lbs = a.log2_block_size;
    const int bs = a.block_size;
    int P = a.partition_size;  // or the ordering kernel's pick (below)
    const int64_t head_tile = (int64_t)bs * D * St::EB;  // bytes of one (block, head) tile
    const int64_t block_stride = (int64_t)a.num_kv_heads * head_tile;
    const int n = lane & 15;
    const int j = lane >> 4;
    // per-lane byte offsets from the chunk's first token quad: key token n
    // (quad n/4, row n%4), the dims of lane group j; value quad j, dim n.
    // k-chunk c and value row chunk c add St::kstep * c and St::vstep * c.
    const int koff = St::koff(n, j, D);
    const int voff = St::voff(n, j, D);
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
    // An item's start-up loads and its first two chunks are issued at the
    // highest wave priority, then the wave drops back: the hardware otherwise
    // issues the oldest wave's loads first, and an item that starts on a young
    // wave waits for its first bytes while older waves stream (on a skewed
    // batch from HBM, the median item computed its first chunk 12 us into a
    // 33 us launch).  Measured on the 16-bit
    // caches, decode kernel: 0.1-2% faster on every workload, most on the
    // skewed one; on E4M3 caches neutral to 1.2% slower, so they keep it off.
    constexpr bool kStartPrio = KV != Elem::FP8;
    if constexpr (kStartPrio) __builtin_amdgcn_s_setprio(3);
    const int h = hc / chunks;
    const int hq0 = h * a.group + (hc % chunks) * Gh;
    // the q / out row of column c: query c / Gh, head hq0 + c % Gh
    auto row_of = [&](int c) -> int64_t {
      const int qc = c / Gh;
      return ((int64_t)b * Q + qc) * a.num_q_heads + hq0 + (c - qc * Gh);
    };

    // Start-up loads that do not depend on the context length go out together
    // with it: the first block-id window (clamped to the table width; entries
    // past the sequence are never used) and the queries.
    const int t_begin = part * P;
    const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
    const int L_in = a.context_lens[b];
    const int bt_first = bt[min((t_begin >> lbs) + lane, a.max_blocks_per_seq - 1)];

    // queries: column 16t + n of tile t = query row row_of(16t + n) (zero beyond the G
    // columns)
    vec8 qv[NT][KC];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if (16 * t + n < G) {
          const char* qp = reinterpret_cast<const char*>(a.q) +
                           (row_of(16 * t + n) * D + St::qdim(c, j)) * 2;
          qv[t][c] = *reinterpret_cast<const vec8*>(qp);
        } else {
#pragma unroll
          for (int r = 0; r < 8; ++r) qv[t][c][r] = (scalar)0.0f;
        }
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
    // query qi sits at position L - Q + qi and sees the positions up to its own
    const int lim_lo = L - Q + 1;        // the smallest column limit (uniform)
    const int lim_n = lim_lo + n / Gh;  // this lane's column of tile 0
    const char* kc = reinterpret_cast<const char*>(a.k_cache) + (int64_t)h * head_tile;
    const char* vc = reinterpret_cast<const char*>(a.v_cache) + (int64_t)h * head_tile;

    int wb = t_begin >> lbs;  // first logical block of the current block-id window
    int bt_lane = (int)clamp_block(bt_first, a.num_blocks);  // lane i: block of wb + i

    // Loads of one 16-token chunk.  Issued unconditionally, so every path
    // through the loop has the same loads in flight and the compiler's wait
    // counts stay exact; the prefetch past the last chunk (`none`) reads
    // through an empty buffer range, which returns zeros without touching
    // memory (or re-reads the last chunk where plain global loads are used).
    auto issue = [&](Buffers<KV, D>& buf, int t0, bool none) {
      if constexpr (UB) {
        // one block: a buffer resource based at the chunk's key / value tile,
        // per-lane 32-bit offsets, the 16-dim row stride as the scalar offset
        const int phys = __builtin_amdgcn_readlane(bt_lane, min(t0 >> lbs, last_blk) - wb);
        const int64_t first_quad =
            (int64_t)phys * block_stride + (int64_t)(t0 & (bs - 1)) * D * St::EB;
        const int range = none ? 0 : 0x7fffffff;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc + first_quad, range);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vc + first_quad, range);
        // opaque copies of the lane offsets: the per-chunk constants then fold
        // into the loads' immediate offsets instead of being hoisted out of
        // the loop into one register per load (12 VGPRs at head_dim 128)
        int ko = koff, vo = voff;
        asm volatile("" : "+v"(ko), "+v"(vo));
#pragma unroll
        for (int c = 0; c < KL; ++c) buf.k[c] = St::load_k(rk, ko + St::kstep * c);
#pragma unroll
        for (int c = 0; c < VL; ++c) buf.v[c] = St::load_v(rv, vo + St::vstep * c);
      } else {
        const int tk = t0 + n;      // this lane's key token
        const int tv = t0 + 4 * j;  // first token of this lane's value quad
        const int pk = __shfl(bt_lane, min(tk >> lbs, last_blk) - wb);
        const int pv = __shfl(bt_lane, min(tv >> lbs, last_blk) - wb);
        const int ik = tk & (bs - 1), iv = tv & (bs - 1);
        // the quad of token ik (iv) within its block, then the lane's piece
        const char* kp = kc + (int64_t)pk * block_stride + (ik >> 2) * 4 * D * St::EB +
                         St::koff(ik & 3, j, D);
        const char* vp = vc + (int64_t)pv * block_stride + (iv >> 2) * 4 * D * St::EB +
                         St::voff(n, 0, D);
#pragma unroll
        for (int c = 0; c < KL; ++c) buf.k[c] = St::load_k(kp + St::kstep * c);
#pragma unroll
        for (int c = 0; c < VL; ++c) buf.v[c] = St::load_v(vp + St::vstep * c);
      }
    };

    f32x4_t o[NT][VC];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int c = 0; c < VC; ++c) o[t][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // this lane's accumulators of tile t, times sc, into the D floats at base
    // (16-byte aligned): dim St::dim(c, j, r) holds o[t][c][r]
    auto store_acc = [&](float* base, int t, float sc) {
      if constexpr (St::kVDims == 1) {
#pragma unroll
        for (int c = 0; c < VC; ++c) {
          f32x4_t x = o[t][c];
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] *= sc;
          *reinterpret_cast<f32x4_t*>(base + 16 * c + 4 * j) = x;
        }
      } else {
        // group c: lane group j holds the V * 4 dims from 16Vc + 4Vj, dim
        // 16Vc + 4Vj + Vr + h in o[t][Vc + h][r] (V dims per value load)
        constexpr int V = St::kVDims;
#pragma unroll
        for (int c = 0; c < VC / V; ++c) {
          float x[4 * V];
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int h = 0; h < V; ++h) x[V * r + h] = o[t][V * c + h][r] * sc;
#pragma unroll
          for (int u = 0; u < V; ++u)
            *reinterpret_cast<f32x4_t*>(base + 16 * V * c + 4 * V * j + 4 * u) =
                f32x4_t{x[4 * u], x[4 * u + 1], x[4 * u + 2], x[4 * u + 3]};
        }
      }
    };
    float m[NT];     // running max of column 16t + n (log2 domain), uniform over j
    float lsum[NT];  // this lane's share of that column's sum
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      m[t] = -INFINITY;
      lsum[t] = 0.0f;
    }

    auto compute = [&](Buffers<KV, D>& buf, int t0, int t_stop) {
      vec4 vv[VC];
#pragma unroll
      for (int c = 0; c < VC; ++c) vv[c] = St::v(buf.v[c / St::kVDims], c % St::kVDims);
      // uniform: the chunk reaches the context end, the partition end or a query's limit
      const bool edge = t0 + kChunk > min(t_stop, lim_lo);
      if (edge) {
        // values past the context are zeroed (they may hold anything)
        const int nv = t_stop - t0 - 4 * j;  // tokens of this lane's run inside the range
#pragma unroll
        for (int c = 0; c < VC; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r >= nv) vv[c][r] = (scalar)0.0f;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < KC; ++c)
          sacc = M::qk(St::k(buf.k[St::kPairK ? c >> 1 : c], c & 1), qv[t][c], sacc);
        float s[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = sacc[r] * a.scale_log2;
        if (edge) {  // scores past the range or past the column's query are masked
          const int lim = t == 0 ? lim_n : lim_lo + (16 * t + n) / Gh;
          const int ns = min(t_stop, lim) - t0 - 4 * j;
#pragma unroll
          for (int r = 0; r < 4; ++r) s[r] = r < ns ? s[r] : -INFINITY;
        }
        float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m[t], mx);
        // a column with every score so far masked keeps m = -inf; exponents are
        // then taken against 0 so that they give 0, not NaN
        const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m[t] - m_ref);
        m[t] = m_new;
        vec4 phi, plo;
        float ps = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(s[r] - m_ref);
          ps += p;
          const scalar hi = (scalar)p;
          phi[r] = hi;
          plo[r] = (scalar)(p - (float)hi);
        }
        lsum[t] = lsum[t] * alpha + ps;
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int c = 0; c < VC; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[t][c][r] *= alpha;
        }
#pragma unroll
        for (int c = 0; c < VC; ++c) {
          o[t][c] = M::pv(vv[c], phi, o[t][c]);
          o[t][c] = M::pv(vv[c], plo, o[t][c]);
        }
      }
    };

    // Walk the partition in windows of 64 blocks (one block id per lane); inside
    // a window this wave takes every W-th chunk, loading its next chunk while
    // the current one is computed.  Only the last window can hold fewer than W
    // chunks (a full window has at least 32).
    Buffers<KV, D> b0, b1;
    const int window = 64 * bs;
    const int stride = W * kChunk;
    for (int w0 = t_begin; w0 < t_end; w0 += window) {
      const int w1 = min(w0 + window, t_end);
      if (w0 != t_begin) {  // later windows (one-pass over long contexts)
        wb = w0 >> lbs;
        bt_lane = (int)clamp_block(bt[min(wb + lane, last_blk)], a.num_blocks);
      }
      const int nc = (w1 - w0 + kChunk - 1) / kChunk;
      if (wave >= nc) continue;
      const int nk = (nc - wave + W - 1) / W;  // chunks of this wave
      const int first_t0 = w0 + wave * kChunk;
      const int last_t0 = first_t0 + (nk - 1) * stride;
      issue(b0, first_t0, false);
      for (int i = 0; i < nk; i += 2) {
        const int t0 = first_t0 + i * stride;
        issue(b1, min(t0 + stride, last_t0), t0 + stride > last_t0);
        compute(b0, t0, w1);
        if (i + 1 >= nk) break;
        issue(b0, min(t0 + 2 * stride, last_t0), t0 + 2 * stride > last_t0);
        if (kStartPrio && i == 0) __builtin_amdgcn_s_setprio(0);
        compute(b1, t0 + stride, w1);
      }
    }

    // ---- finish the work item ------------------------------------------------
    float l[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      l[t] = lsum[t] + __shfl_xor(lsum[t], 16);
      l[t] += __shfl_xor(l[t], 32);
    }
    if (W > 1) {
      // Merge the waves: M = max_w m_w, l = sum_w 2^(m_w - M) l_w, and the
      // accumulators likewise.  A wave without tokens for a column has m =
      // -inf, l = 0 and zero accumulators; when no wave has any (a query
      // whose position lies before this partition), the column's l is 0 and
      // exponents are taken against 0.  Every wave parks its rescaled
      // accumulators in LDS, then the whole workgroup sums them and stores.
      constexpr int CW = 16 * NT;  // columns per wave row of red_m / red_l
      float* red_m = red;               // [W][CW]
      float* red_l = red + 4 * CW;      // [W][CW]
      float* red_o = red + 8 * CW;      // [W][G][D + 4] (rows padded against bank conflicts)
      constexpr int RS = D + 4;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (j == 0) {
          red_m[wave * CW + 16 * t + n] = m[t];
          red_l[wave * CW + 16 * t + n] = l[t];
        }
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float M = -INFINITY;
        for (int w = 0; w < W; ++w) M = fmaxf(M, red_m[w * CW + 16 * t + n]);
        const float sc = fast_exp2(m[t] - (M == -INFINITY ? 0.0f : M));
        if (16 * t + n < G) store_acc(red_o + (wave * G + 16 * t + n) * RS, t, sc);
      }
      __syncthreads();
      for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
        const int g = e / D, d = e - g * D;
        float Mg = -INFINITY;
        for (int w = 0; w < W; ++w) Mg = fmaxf(Mg, red_m[w * CW + g]);
        const float Mref = Mg == -INFINITY ? 0.0f : Mg;
        float lt = 0.0f, x = 0.0f;
        for (int w = 0; w < W; ++w) {
          lt += red_l[w * CW + g] * fast_exp2(red_m[w * CW + g] - Mref);
          x += red_o[(w * G + g) * RS + d];
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
    for (int t = 0; t < NT; ++t) {
      const int col = 16 * t + (fresh_tid() & 15);  // re-derived: not held through the loop
      if (col < G) {
        const int64_t row_id = row_of(col);
        if (n_parts == 1) {
          // l = 0: a query before position 0
          const float inv = l[t] > 0.0f ? a.v_scale / l[t] : 0.0f;
#pragma unroll
          for (int c = 0; c < VC; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              store_elem(a.out, row_id * D + St::dim(c, j, r), o[t][c][r] * inv, a.out_dtype);
        } else {
          const int64_t slot = row_id * a.max_partitions + part;
          store_acc(a.ws_acc + slot * D, t, a.v_scale);
          if (j == 0) {
            a.ws_ml[slot * 2] = m[t];
            a.ws_ml[slot * 2 + 1] = l[t];
          }
        }
      }
    }
    }
  next_item:
    if constexpr (KV != Elem::FP8) __builtin_amdgcn_s_setprio(0);
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

// LDS of the wave merge: m and l of 16 columns per tile for up to 4 waves,
// then every wave's padded accumulators.
size_t merge_lds_bytes(int waves, int cols, int head_dim) {
  if (waves <= 1) return 0;
  const size_t cw = 16 * (size_t)((cols + 15) / 16);
  return (8 * cw + (size_t)waves * cols * (head_dim + 4)) * sizeof(float);
}

template <Elem KV, int D>
hipError_t dispatch_g(const DecodeArgs& a, int64_t items_x, hipStream_t s) {
  const bool ub = a.block_size >= 16;
  const int cols = a.num_queries * a.heads_per_item;  // tile columns (template G)
  const size_t lds = (size_t)a.list_ints * sizeof(int) + merge_lds_bytes(a.waves, cols, D);
  const void* fn = nullptr;
  switch (cols) {
#define PA_CASE(GG)                                                                   \
  case GG:                                                                            \
    fn = ub ? reinterpret_cast<const void*>(&decode_mfma_kernel<KV, D, GG, true>)     \
            : reinterpret_cast<const void*>(&decode_mfma_kernel<KV, D, GG, false>);   \
    break;
    PA_CASE(1) PA_CASE(2) PA_CASE(4) PA_CASE(8) PA_CASE(16)
    PA_CASE(3) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(10) PA_CASE(12) PA_CASE(24) PA_CASE(32)
#undef PA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return launch_decode_grid(fn, a, items_x, lds, s);
}

}  // namespace

bool mfma_supports_heads(int heads_per_item) {
  switch (heads_per_item) {
    case 1: case 2: case 3: case 4: case 5: case 6: case 7: case 8: case 10: case 12: case 16:
    case 24: case 32:
      return true;
    default:
      return false;
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int kv_dtype, int head_dim, hipStream_t s) {
  const int64_t items_x = (int64_t)a.num_seqs * a.num_kv_heads * (a.group / a.heads_per_item);
  if (kv_dtype == 2) {
    if (head_dim == 128) return dispatch_g<Elem::BF16, 128>(a, items_x, s);
    if (head_dim == 64) return dispatch_g<Elem::BF16, 64>(a, items_x, s);
  } else if (kv_dtype == 3) {  // E4M3 caches, bfloat16 queries
    if (head_dim == 128) return dispatch_g<Elem::FP8, 128>(a, items_x, s);
    if (head_dim == 64) return dispatch_g<Elem::FP8, 64>(a, items_x, s);
  } else if (kv_dtype == 1) {
    if (head_dim == 128) return dispatch_g<Elem::F16, 128>(a, items_x, s);
    if (head_dim == 64) return dispatch_g<Elem::F16, 64>(a, items_x, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
