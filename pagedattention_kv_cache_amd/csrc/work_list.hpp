// work_list.hpp -- the (sequence, partition) work list a persistent decode
// launch walks.
//
// A decode launch over partitions has up to num_seqs * max_partitions work
// items per head chunk, but only sum_b ceil(L_b / P) of them hold tokens (one
// for an empty sequence, which writes zeros); the host does not know the
// context lengths.  Instead of one workgroup per possible item -- most of
// which would only read a length and exit -- a fixed grid of workgroups each
// builds the list of real items in LDS from the context lengths and takes
// every gridDim.x-th entry.  The list is ordered longest sequences first:
// items with a higher partition index come first, and inside one partition
// index the sequences with more partitions come first, so full partitions of
// long contexts start early and the short remainders fill in at the end.
// Every workgroup must build exactly the same list (each takes its own share
// of the entries), so its construction is deterministic.
#pragma once

#include "pa_device.hpp"
#include "pa_launch.hpp"

namespace pa {

// Items of sequence b: its partitions, or one (zero output) when empty.
__device__ __forceinline__ int items_of_seq(const DecodeArgs& a, int b) {
  const int L = clamp_len(a.context_lens[b], a.max_blocks_per_seq, a.block_size);
  return L <= 0 ? 1 : (L + a.partition_size - 1) / a.partition_size;
}

// x[i] <- sum_{i' >= i} x[i'] for i in [0, len); called by all lanes of one wave.
__device__ __forceinline__ void wave_suffix_sum(int* x, int len) {
  const int lane = threadIdx.x & 63;
  const int per = (len + 63) / 64;
  const int lo = min(lane * per, len), hi = min(lo + per, len);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += x[i];
  int incl = s;  // sum over lanes >= lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_down(incl, off);
    if (lane + off < 64) incl += o;
  }
  int run = incl - s;
  for (int i = hi - 1; i >= lo; --i) {
    run += x[i];
    x[i] = run;
  }
}

// The kernel argument block, read afresh: each call yields an opaque copy of
// the kernarg pointer, so a persistent loop re-reads the arguments it needs
// per item instead of holding all of them in scalar registers for the whole
// launch.  The decode kernels take DecodeArgs as their only argument, at
// offset 0 of the kernarg segment.
using KernArgs = const __attribute__((address_space(4))) DecodeArgs;
__device__ __forceinline__ KernArgs* fresh_args() {
  KernArgs* p = (KernArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}

// The thread index through an opaque copy: per-lane offsets derived from it
// inside a persistent loop are then computed per item instead of being
// hoisted out of the loop and held in vector registers for the whole launch.
__device__ __forceinline__ int fresh_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Dynamic deal: the next item index of a workgroup from the launch's counter
// (one lane asks).  The answer goes through two LDS ints used alternately, so
// a wave that runs ahead to the next item cannot overwrite a value another
// wave has not read yet.
__device__ __forceinline__ int take_ticket(int32_t* ctr) {
  return __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS layout of the list (ints): cnt[NP + 2], tot[NP + 2], base[NP + 1],
// fill[NP + 1], sorted[B], items[B].
__device__ __forceinline__ const int* list_base(const int* lds, int np) {
  return lds + 2 * (np + 2);
}
__device__ __forceinline__ const int* list_sorted(const int* lds, int np) {
  return lds + 2 * (np + 2) + 2 * (np + 1);
}

// Builds the list in `lds` and returns its length (items); every thread of
// the workgroup must call it.  Every workgroup of the launch builds the same
// list: the counts are order-free sums, and inside one item count the
// sequences keep their index order (a stable counting sort run by wave 0).
__device__ inline int build_work_list(const DecodeArgs& a, int* lds) {
  const int NP = a.max_partitions, B = a.num_seqs;
  const int tid = threadIdx.x, T = blockDim.x;
  int* cnt = lds;                // cnt[n]: sequences with n items, n in [1, NP]
  int* tot = cnt + NP + 2;       // suffix sums of cnt
  int* base = tot + NP + 2;
  int* fill = base + NP + 1;
  int* sorted = fill + NP + 1;
  int* items = sorted + B;       // items of each sequence
  for (int i = tid; i < NP + 2; i += T) cnt[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += T) {
    const int n = items_of_seq(a, b);
    items[b] = n;
    atomicAdd(&cnt[n], 1);
  }
  __syncthreads();
  if (tid < 64) {
    // cnt[n] <- S[n] = #{b : n_b >= n}, so partition p has S[p + 1] items;
    // tot[n] <- sum_{n' >= n} S[n'] (the items of partitions >= n - 1).
    wave_suffix_sum(cnt + 1, NP);
    wave_lds_sync();
    for (int n = 1 + tid; n <= NP + 1; n += 64) tot[n] = n <= NP ? cnt[n] : 0;
    wave_lds_sync();
    wave_suffix_sum(tot + 1, NP);
    wave_lds_sync();
    // rank k = NP - 1 - p lists partition p; it starts after the items of
    // all higher partitions: base[k] = tot[NP - k + 1] (tot[NP + 1] = 0).
    for (int k = tid; k <= NP; k += 64) base[k] = k == 0 ? 0 : tot[NP - k + 1];
    // sequences with n items go after those with more: positions from S[n + 1]
    for (int n = 1 + tid; n <= NP; n += 64) fill[n] = n < NP ? cnt[n + 1] : 0;
    wave_lds_sync();
    // stable placement, 64 sequences at a time: the lanes holding one item
    // count take consecutive positions in lane (= sequence) order
    const int lane = tid;
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int b = b0 + lane;
      const bool live = b < B;
      const int n = live ? items[b] : 0;
      uint64_t pending = __ballot(live);
      while (pending) {
        const int x = __builtin_amdgcn_readlane(n, __builtin_ctzll(pending));
        const uint64_t same = __ballot(live && n == x);
        const int start = fill[x];
        if (live && n == x) sorted[start + __popcll(same & ((1ull << lane) - 1))] = b;
        wave_lds_sync();
        if (lane == 0) fill[x] = start + __popcll(same);
        wave_lds_sync();
        pending &= ~same;
      }
    }
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(base[NP]);
}

// List entry `item` -> (sequence, partition).  `k` is a cursor that only moves
// forward: the entries a workgroup takes increase.
__device__ __forceinline__ void work_item(const int* lds, int np, int item, int& k, int& b,
                                          int& part) {
  const int* base = list_base(lds, np);
  while (__builtin_amdgcn_readfirstlane(base[k + 1]) <= item) ++k;
  part = np - 1 - k;
  b = __builtin_amdgcn_readfirstlane(list_sorted(lds, np)[item - base[k]]);
}

}  // namespace pa
