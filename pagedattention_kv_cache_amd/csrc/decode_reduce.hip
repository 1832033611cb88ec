// decode_reduce.hip -- log-sum-exp merge of a sequence's partition results.
//
// The second PagedAttention kernel of the "vLLM Project Update" talk splits
// each sequence into pieces spread across the GPU and combines them the way
// flash decoding does; the talk gives no formula.  With per-partition running
// max m_p (log2 domain), sum l_p = sum_t 2^(s_t - m_p) and unnormalised
// output a_p = sum_t 2^(s_t - m_p) v_t, the exact merge is
//     M = max_p m_p,  w_p = 2^(m_p - M),
//     out = (sum_p w_p a_p) / (sum_p w_p l_p),
// which equals softmax(s).V over the whole sequence.
//
// One workgroup of 256 threads per 256 / D (query, q head) rows of a
// sequence, one thread per output element; the grid's second dimension holds
// at most 65535 sequences and steps over larger batches.  Rows with a single partition were
// finished by the decode kernel and are skipped.  Partitions are merged four
// at a time: the four (m, l) pairs and the four partial outputs are loaded
// together, then folded into the running result with the same rule
// (rescaling what was merged before by 2^(M_old - M_new)), so the loads of a
// batch wait neither on each other nor on its maximum.  A partition holding
// no token a row may see (a query before it) has m = -inf, l = 0 and weight
// 0; a row with no token at all gives 0.
#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {
namespace {

constexpr int kReduceThreads = 256;

template <int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int kRows = kReduceThreads / D;  // rows per workgroup
  const int P = partition_of(a);
  const int rows = a.num_queries * a.num_q_heads;
  const int qh = (int)blockIdx.x * kRows + (int)threadIdx.x / D;  // query * num_q_heads + q head
  const int e = (int)threadIdx.x % D;
  if (qh >= rows) return;
  for (int b = blockIdx.y; b < a.num_seqs; b += gridDim.y) {
    const int L = clamp_len(a.context_lens[b], a.max_blocks_per_seq, a.block_size);
    const int n_parts = L > 0 ? (L + P - 1) / P : 0;
    if (n_parts <= 1) continue;
    const int64_t row_id = (int64_t)b * rows + qh;
    const float* ml = a.ws_ml + row_id * a.max_partitions * 2;
    const float* accs = a.ws_acc + row_id * a.max_partitions * D + e;
    float M = -INFINITY, num = 0.0f, den = 0.0f;
    for (int p0 = 0; p0 < n_parts; p0 += 4) {
      float mp[4], lp[4], xp[4];
      // unconditional loads of clamped partitions (no branch between them),
      // masked after
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int p = min(p0 + k, n_parts - 1);
        const float2 pair = *reinterpret_cast<const float2*>(ml + 2 * p);
        const float x = accs[(int64_t)p * D];
        const bool in = p0 + k < n_parts;
        mp[k] = in ? pair.x : -INFINITY;
        lp[k] = in ? pair.y : 0.0f;
        xp[k] = in ? x : 0.0f;
      }
      const float Mn = fmaxf(fmaxf(M, fmaxf(mp[0], mp[1])), fmaxf(mp[2], mp[3]));
      const float Mref = Mn == -INFINITY ? 0.0f : Mn;
      const float sc = fast_exp2(M - Mref);  // 0 on the first batch (M = -inf)
      num *= sc;
      den *= sc;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float w = fast_exp2(mp[k] - Mref);
        den = fmaf(w, lp[k], den);
        num = fmaf(w, xp[k], num);
      }
      M = Mn;
    }
    store_elem(a.out, row_id * D + e, den > 0.0f ? num / den : 0.0f, a.out_dtype);
  }
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeArgs& a, int head_dim, hipStream_t s) {
  if (a.max_partitions <= 1) return hipSuccess;
  const int rows = a.num_queries * a.num_q_heads;
  const int rows_per_wg = kReduceThreads / head_dim;
  const int seqs_y = a.num_seqs < 65535 ? a.num_seqs : 65535;  // the kernel steps over the rest
  dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg), (unsigned)seqs_y);
  if (head_dim == 64) {
    hipLaunchKernelGGL(decode_reduce_kernel<64>, grid, dim3(kReduceThreads), 0, s, a);
  } else if (head_dim == 128) {
    hipLaunchKernelGGL(decode_reduce_kernel<128>, grid, dim3(kReduceThreads), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
