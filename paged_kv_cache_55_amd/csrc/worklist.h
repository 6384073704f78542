// Work list of a split-K paged decode, built by every workgroup of a
// persistent grid.
//
// A work item is (sequence b, partition p, KV head) for every partition
// that holds at least one token: partition p of sequence b covers tokens
// [p * P, min(L_b, (p + 1) * P)). Items are numbered j * Hkv + kvh where
// j = prefix[b] + p and prefix is the exclusive prefix sum over sequences of
// ceil(L_b / P). The grid is sized to the number of workgroups the GPU can
// hold at once, and workgroup w takes items w, w + grid, w + 2 grid, ...,
// so no workgroup is launched without work and none exits empty-handed:
// per-workgroup dispatch cost, not the data, dominates a grid of many
// short or empty workgroups.
#pragma once

#include "device_common.h"

namespace pagedkv {

constexpr int kMaxSeqs = 4096;  // sequences per call (prefix lives in LDS)

// Exclusive prefix over a block of kThreads threads (a multiple of 64);
// `v` is this thread's value, `scratch` holds kThreads / 64 ints. Returns
// the exclusive prefix; *total gets the sum.
template <int kThreads = 256>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  constexpr int kW = kThreads / 64;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int n = __shfl_up(inc, off, 64);
    if (lane >= off) inc += n;
  }
  if (lane == 63) scratch[w] = inc;
  __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int i = 0; i < kW; ++i) {
    const int s = scratch[i];
    base += i < w ? s : 0;
    sum += s;
  }
  __syncthreads();
  *total = sum;
  return base + inc - v;
}

// prefix[0..B] <- exclusive prefix of the counts already in prefix[0..B-1].
// Needs blockDim.x == kThreads and B <= kMaxSeqs; each thread scans a
// contiguous chunk. Ends with a barrier.
template <int kThreads = 256>
__device__ __forceinline__ void scan_counts_in_place(int B, int* prefix, int* scratch) {
  constexpr int kMaxChunk = (kMaxSeqs + kThreads - 1) / kThreads;
  const int chunk = (B + kThreads - 1) / kThreads;  // <= kMaxChunk
  const int first = threadIdx.x * chunk;
  int counts[kMaxChunk];
  int local = 0;
#pragma unroll
  for (int i = 0; i < kMaxChunk; ++i) {
    const int c = (i < chunk && first + i < B) ? prefix[first + i] : 0;
    counts[i] = c;
    local += c;
  }
  int total;
  int run = block_exclusive_scan<kThreads>(local, scratch, &total);
#pragma unroll
  for (int i = 0; i < kMaxChunk; ++i) {
    if (i < chunk && first + i < B) {
      prefix[first + i] = run;
      run += counts[i];
    }
  }
  if (threadIdx.x == 0) prefix[B] = total;
  __syncthreads();
}

// prefix[0..B] <- exclusive prefix of ceil(L_b / part_tokens) (0 for L_b <= 0).
// Needs blockDim.x == 256 and B <= kMaxSeqs. The lengths are read with
// coalesced loads into LDS, then scanned. Ends with a barrier.
__device__ __forceinline__ void build_partition_prefix(const int32_t* __restrict__ seq_lens, int B,
                                                       int part_tokens, int* prefix,
                                                       int* scratch) {
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    const int L = seq_lens[i];
    prefix[i] = L > 0 ? (L + part_tokens - 1) / part_tokens : 0;
  }
  __syncthreads();
  scan_counts_in_place(B, prefix, scratch);
}

// Sequence owning partition index j: the largest b with prefix[b] <= j.
__device__ __forceinline__ int find_sequence(const int* prefix, int B, int j) {
  int lo = 0, hi = B;  // prefix[lo] <= j < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= j) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace pagedkv
