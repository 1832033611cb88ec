// decode_order.hip -- longest-first order of a partitioned decode's work items.
//
// The host does not read the context lengths, so a partitioned decode
// launches one workgroup per *possible* (sequence, partition) item, most of
// which are empty on a batch of mixed lengths.  Dispatched in grid order,
// empty workgroups that come first hold back the start of the real ones, and
// full-size items that come last stretch the end of the launch.  This kernel
// (one workgroup, run just before the decode on the same stream) writes the
// non-empty items in order of decreasing token count, then -1 for the rest;
// decode workgroup i takes entry i, so the grid starts with the longest
// items and ends with the empty ones, which exit at once.
//
// Entry = b * max_partitions + partition.  Items of equal size (in 16-token
// chunks) may come in any order: an item's result does not depend on the
// workgroup that computes it.
#include "cache_write.hpp"
#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {
namespace {

// One workgroup of 256 threads orders; in the write + order launch the other
// workgroups write, 256 threads each, as the write kernel does.  With 1024
// threads per workgroup (the order's histogram scan one bin per thread) the
// write ran on a quarter as many CUs: the launch took 10.1-10.5 us at the GQA
// lognormal and MHA batches, 5.8-6.0 us now (rocprofv3).
constexpr int kThreads = 256;
constexpr int kBins = 1024;  // item sizes in 16-token chunks; larger ones share the last bin
constexpr int kBinsPerThread = kBins / kThreads;

// Size bin of partition `part` of a sequence of L tokens: its 16-token chunks.
__device__ __forceinline__ int item_bin(int L, int part, int P) {
  return min((min(L - part * P, P) + 15) / 16, kBins - 1);
}

// Items of a sequence of (clamped) length L: its partitions; an empty
// sequence still has one, which writes its zero rows.
__device__ __forceinline__ int seq_items(int L, int P, int np) {
  return L <= 0 ? 1 : min((L + P - 1) / P, np);
}

// The partition the library picks on the device (DecodeArgs::part_dev) from
// the clamped context lengths: their total, their maximum and the batch size.
// A batch whose longest context is at most twice the mean keeps the host's
// pick c (its items are alike: larger ones would not even out).  Otherwise the
// pick is the largest of c / 2, c, 2c that is at most a third of one compute
// unit's share of the token-heads (a CU runs three 4-wave workgroups, so an
// item then takes at most about as long as the CU's whole share), 2c only
// while the longest context still spans two partitions and 2c <= 8192.
// Measured against the host's pick alone: GQA lognormal batch of 256
// (share/3 ~ 4200) 2048 -> 4096, decode kernel 259.1 -> 256.1 us; the same
// lengths over 64 sequences (share/3 ~ 1000) 2048 -> 1024, 66.3 -> 65.5 us and
// one 8192-token sequence among 63 short ones 2048 -> 1024, 38.4 -> 30.4 us
// (ordering + decode); uniform batches keep the host's pick (4 x 32k and
// 16 x 16k at 4096, 64 x 4k-32k at 8192) and their time.
__device__ __forceinline__ int device_partition(const DecodeArgs& a, int64_t total, int lmax) {
  const int c = a.partition_size;
  const int64_t B = a.num_seqs;
  if (lmax <= 0 || (int64_t)lmax * B <= 2 * total) return c;
  const int64_t items = (int64_t)a.num_kv_heads * (a.group / a.heads_per_item);
  const int64_t third = total * items / (3 * (int64_t)max(a.num_cus, 1));
  int p = c / 2;
  if (third >= c) p = c;
  if (third >= 2LL * c && 4LL * c <= lmax && 2 * c <= 8192) p = 2 * c;
  return p;
}

// The order, by one workgroup of kThreads threads.
__device__ __forceinline__ void order_items(const DecodeArgs& a, int32_t* order) {
  __shared__ int hist[kBins];
  __shared__ int start[kBins];
  __shared__ unsigned long long len_total;
  __shared__ int len_max, picked;
  const int tid = threadIdx.x;
  const int np = a.max_partitions, B = a.num_seqs;
  for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
  if (tid == 0) {
    len_total = 0;
    len_max = 0;
  }
  __syncthreads();
  int L_own = 0;  // the length of sequence tid, kept for the later passes
  int64_t my_total = 0;
  int my_max = 0;
  for (int b = tid; b < B; b += kThreads) {
    const int L = clamp_len(a.context_lens[b], a.max_blocks_per_seq, a.block_size);
    if (b == tid) L_own = L;
    my_total += max(L, 0);
    my_max = max(my_max, L);
  }
  int P = a.partition_size;
  if (a.part_dev && a.part_pick) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      my_total += __shfl_xor(my_total, off, 64);
      my_max = max(my_max, __shfl_xor(my_max, off, 64));
    }
    if ((tid & 63) == 0) {
      atomicAdd(&len_total, (unsigned long long)my_total);
      atomicMax(&len_max, my_max);
    }
    __syncthreads();
    if (tid == 0) {
      picked = device_partition(a, (int64_t)len_total, len_max);
      *a.part_dev = picked;  // read by the decode and merge launches that follow
    }
    __syncthreads();
    P = picked;
  } else if (a.part_dev && tid == 0) {
    *a.part_dev = P;
  }
  for (int b = tid; b < B; b += kThreads) {
    const int L =
        b == tid ? L_own : clamp_len(a.context_lens[b], a.max_blocks_per_seq, a.block_size);
    const int n = seq_items(L, P, np);
    for (int p = 0; p < n; ++p) atomicAdd(&hist[L <= 0 ? 0 : item_bin(L, p, P)], 1);
  }
  __syncthreads();
  // start[bin] = items in larger bins.  Thread tid takes the bins at
  // positions kBinsPerThread * tid .. + kBinsPerThread - 1 of the descending
  // order (bin kBins - 1 - position), so an inclusive prefix sum of the
  // threads' totals counts the largest bins up to its own; within a wave by
  // lane shuffles, across waves through LDS.
  __shared__ int wave_sum[kThreads / 64];
  const int lane = tid & 63, wave = tid >> 6;
  int cnt[kBinsPerThread], own = 0;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    cnt[i] = hist[kBins - 1 - (kBinsPerThread * tid + i)];
    own += cnt[i];
  }
  int v = own;
#pragma unroll
  for (int off = 1; off < 64; off *= 2) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wave_sum[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += wave_sum[w];
  int run = v - own;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    start[kBins - 1 - (kBinsPerThread * tid + i)] = run;
    run += cnt[i];
  }
  __syncthreads();
  const int total = start[0] + hist[0];
  __syncthreads();
  for (int b = tid; b < B; b += kThreads) {
    const int L =
        b == tid ? L_own : clamp_len(a.context_lens[b], a.max_blocks_per_seq, a.block_size);
    const int n = seq_items(L, P, np);
    for (int p = 0; p < n; ++p)
      order[atomicAdd(&start[L <= 0 ? 0 : item_bin(L, p, P)], 1)] = b * np + p;
  }
  for (int e = total + tid; e < B * np; e += kThreads) order[e] = -1;
  if (tid == 0 && a.part_dev) a.part_dev[1] = total;  // the entries, for the decode's deal
  if (tid == 0 && a.order_ctr) *a.order_ctr = 0;
}

__global__ __launch_bounds__(kThreads) void decode_order_kernel(DecodeArgs a, int32_t* order) {
  order_items(a, order);
}

// A decode step's cache write and the order in one launch: workgroup 0
// orders (it reads only the context lengths), the others write the step's
// new tokens, one 16-byte chunk per thread.  The decode that follows on the
// stream sees both.
template <int EB>
__global__ __launch_bounds__(kThreads) void decode_prologue_kernel(DecodeArgs a, int32_t* order,
                                                                   CacheWriteArgs w,
                                                                   int chunks_per_row) {
  if (blockIdx.x == 0) {
    order_items(a, order);
  } else {
    cache_write_chunk<EB>(w, (int64_t)(blockIdx.x - 1) * kThreads + threadIdx.x,
                          chunks_per_row);
  }
}

// The same with the quantizing write into E4M3 caches (source type SRC).
template <Elem SRC>
__global__ __launch_bounds__(kThreads) void decode_prologue_fp8_kernel(DecodeArgs a,
                                                                       int32_t* order,
                                                                       CacheWriteArgs w,
                                                                       int chunks_per_row) {
  if (blockIdx.x == 0) {
    order_items(a, order);
  } else {
    cache_write_fp8_chunk<SRC>(w, (int64_t)(blockIdx.x - 1) * kThreads + threadIdx.x,
                               chunks_per_row);
  }
}

}  // namespace

hipError_t launch_decode_order(const DecodeArgs& a, int32_t* order, const CacheWriteArgs* write,
                               hipStream_t s) {
  if (!write || write->num_tokens == 0) {
    hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(kThreads), 0, s, a, order);
    return hipGetLastError();
  }
  // E4M3: one thread per 16 elements; else per 16 bytes
  const int chunks = write->elem_bytes == 1 ? write->head_dim / 16
                                            : write->head_dim * write->elem_bytes / 16;
  const int64_t total = write->num_tokens * write->num_kv_heads * chunks;
  const int64_t blocks = 1 + (total + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (write->elem_bytes == 1) {
    switch (write->src_dtype) {
      case 0:
        hipLaunchKernelGGL(decode_prologue_fp8_kernel<Elem::F32>, dim3((unsigned)blocks),
                           dim3(kThreads), 0, s, a, order, *write, chunks);
        break;
      case 1:
        hipLaunchKernelGGL(decode_prologue_fp8_kernel<Elem::F16>, dim3((unsigned)blocks),
                           dim3(kThreads), 0, s, a, order, *write, chunks);
        break;
      case 2:
        hipLaunchKernelGGL(decode_prologue_fp8_kernel<Elem::BF16>, dim3((unsigned)blocks),
                           dim3(kThreads), 0, s, a, order, *write, chunks);
        break;
      default:
        return hipErrorInvalidValue;
    }
  } else if (write->elem_bytes == 4) {
    hipLaunchKernelGGL(decode_prologue_kernel<4>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       a, order, *write, chunks);
  } else {
    hipLaunchKernelGGL(decode_prologue_kernel<2>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       a, order, *write, chunks);
  }
  return hipGetLastError();
}

}  // namespace pa
