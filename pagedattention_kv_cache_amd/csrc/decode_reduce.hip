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
// One workgroup per (query, q head) row of a sequence; one thread per output
// dim.  Rows with a single partition were finished by the decode kernel and
// are skipped.  A partition holding no token a row may see (a query before
// it) has m = -inf, l = 0 and weight 0; a row with no token at all gives 0.
#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {
namespace {

template <int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeArgs a) {
  const int qh = blockIdx.x;  // query * num_q_heads + q head
  const int b = blockIdx.y;
  const int e = threadIdx.x;
  const int L = clamp_len(a.context_lens[b], a.max_blocks_per_seq, a.block_size);
  const int n_parts = L > 0 ? (L + a.partition_size - 1) / a.partition_size : 0;
  if (n_parts <= 1) return;
  const int64_t row_id = (int64_t)b * a.num_queries * a.num_q_heads + qh;
  const float* ml = a.ws_ml + row_id * a.max_partitions * 2;
  const float* accs = a.ws_acc + row_id * a.max_partitions * D + e;

  float M = -INFINITY;
  for (int p = 0; p < n_parts; ++p) M = fmaxf(M, ml[2 * p]);
  if (M == -INFINITY) M = 0.0f;
  float num = 0.0f, den = 0.0f;
  for (int p = 0; p < n_parts; ++p) {
    const float w = fast_exp2(ml[2 * p] - M);
    den = fmaf(w, ml[2 * p + 1], den);
    num = fmaf(w, accs[(int64_t)p * D], num);
  }
  store_elem(a.out, row_id * D + e, den > 0.0f ? num / den : 0.0f, a.out_dtype);
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeArgs& a, int head_dim, hipStream_t s) {
  if (a.max_partitions <= 1) return hipSuccess;
  dim3 grid((unsigned)(a.num_queries * a.num_q_heads), (unsigned)a.num_seqs);
  if (head_dim == 64) {
    hipLaunchKernelGGL(decode_reduce_kernel<64>, grid, dim3(64), 0, s, a);
  } else if (head_dim == 128) {
    hipLaunchKernelGGL(decode_reduce_kernel<128>, grid, dim3(128), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
