// Dispatch: per-expert histogram, LDS prefix scan, stable scatter into an
// expert-contiguous permutation of the kept slots (sorted by expert, then token).
//
// This is the token-to-expert grouping that a grouped GEMM over
// expert-contiguous rows consumes [SpecForge PR #943, "Modifications":
// grouped_mm dispatch]; the per-expert counts are the analogue of the received
// token counters of [DeepGEMM PR #381, description].
#include "kernels.h"

namespace moe {

// Slots whose id lies outside [0, E) (-1: dropped by the budget or the top-p
// trim) are skipped by every kernel here.
//
// One workgroup of 1024 threads (16 waves).
//  1. counts[e] via LDS atomics over all slots.
//  2. Exclusive scan of counts in LDS -> offsets[0..E].
//  3. Tokens are taken 1024 at a time, one per thread in token order.  For each
//     expert every wave builds a 64-bit mask of its lanes (tokens) routed there;
//     a slot's rank among earlier tokens of the chunk is the popcount of the
//     masks of earlier waves plus its own wave's mask below its lane.  Because a
//     token never lists one expert twice, (expert, token) order is exactly this
//     rank.  A running cursor per expert carries the count across chunks.
__global__ void __launch_bounds__(1024) dispatch_kernel(
    const int32_t* __restrict__ ids, int T, int E, int K, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm) {
  constexpr int kWaves = 16;
  __shared__ unsigned long long mask[kWaves][kMaxExperts];  // 64 KiB
  __shared__ int cnt[kMaxExperts];
  __shared__ int cursor[kMaxExperts];
  __shared__ int scan_tmp[1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int e = tid; e < kMaxExperts; e += 1024) cnt[e] = 0;
  __syncthreads();
  const int nslots = T * K;
  for (int s = tid; s < nslots; s += 1024) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // Inclusive Hillis-Steele scan over E <= 512 <= 1024 entries.
  scan_tmp[tid] = (tid < E) ? cnt[tid] : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = (tid >= o) ? scan_tmp[tid - o] : 0;
    __syncthreads();
    scan_tmp[tid] += add;
    __syncthreads();
  }
  if (tid < E) {
    const int excl = scan_tmp[tid] - cnt[tid];
    cursor[tid] = excl;
    counts[tid] = cnt[tid];
    offsets[tid] = excl;
  }
  if (tid == 0) offsets[E] = scan_tmp[E - 1];
  __syncthreads();

  for (int c0 = 0; c0 < T; c0 += 1024) {
    for (int i = tid; i < kWaves * kMaxExperts; i += 1024) (&mask[0][0])[i] = 0ull;
    __syncthreads();
    const int t = c0 + tid;
    const bool live = t < T;
    const int32_t* row = ids + static_cast<size_t>(t) * K;
    if (live) {
      for (int k = 0; k < K; ++k) {
        const int e = row[k];
        if (e >= 0 && e < E) atomicOr(&mask[wave][e], 1ull << lane);
      }
    }
    __syncthreads();
    if (live) {
      const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      for (int k = 0; k < K; ++k) {
        const int e = row[k];
        if (e < 0 || e >= E) continue;
        int rank = cursor[e] + __popcll(mask[wave][e] & below);
        for (int q = 0; q < wave; ++q) rank += __popcll(mask[q][e]);
        perm[rank] = t * K + k;
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += 1024) {
      int add = 0;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) add += __popcll(mask[q][e]);
      cursor[e] += add;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- many-chunk dispatch
//
// For T > 1024 the same ranking runs with one workgroup per 1024-token chunk:
//  A. dispatch_chunk_kernel: per chunk, the per-expert count (chunk_counts[c][e])
//     and every kept slot's rank among the chunk's earlier tokens (slot_rank);
//  B. dispatch_scan_kernel (one workgroup): counts, offsets and, in place, each
//     chunk's first position per expert = offsets[e] + sum of earlier chunks;
//  C. dispatch_scatter_kernel: perm[chunk_base[c][e] + slot_rank[s]] = s.
// The result is identical to the single-workgroup kernel.

__global__ void __launch_bounds__(1024) dispatch_chunk_kernel(
    const int32_t* __restrict__ ids, int T, int E, int K, int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ slot_rank) {
  constexpr int kWaves = 16;
  __shared__ unsigned long long mask[kWaves][kMaxExperts];  // 64 KiB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  for (int i = tid; i < kWaves * kMaxExperts; i += 1024) (&mask[0][0])[i] = 0ull;
  __syncthreads();
  const int t = c * 1024 + tid;
  const bool live = t < T;
  const int32_t* row = ids + static_cast<size_t>(t) * K;
  if (live) {
    for (int k = 0; k < K; ++k) {
      const int e = row[k];
      if (e >= 0 && e < E) atomicOr(&mask[wave][e], 1ull << lane);
    }
  }
  __syncthreads();
  if (live) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int k = 0; k < K; ++k) {
      const int e = row[k];
      if (e < 0 || e >= E) continue;
      int rank = __popcll(mask[wave][e] & below);
      for (int q = 0; q < wave; ++q) rank += __popcll(mask[q][e]);
      slot_rank[static_cast<size_t>(t) * K + k] = rank;
    }
  }
  for (int e = tid; e < E; e += 1024) {
    int n = 0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) n += __popcll(mask[q][e]);
    chunk_counts[static_cast<size_t>(c) * E + e] = n;
  }
}

__global__ void __launch_bounds__(1024) dispatch_scan_kernel(int nchunks, int E,
                                                             int32_t* __restrict__ chunk_counts,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets) {
  __shared__ int scan_tmp[1024];
  const int tid = threadIdx.x;
  int total = 0;
  if (tid < E)
    for (int c = 0; c < nchunks; ++c) total += chunk_counts[static_cast<size_t>(c) * E + tid];
  scan_tmp[tid] = (tid < E) ? total : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = (tid >= o) ? scan_tmp[tid - o] : 0;
    __syncthreads();
    scan_tmp[tid] += add;
    __syncthreads();
  }
  if (tid < E) {
    int base = scan_tmp[tid] - total;
    counts[tid] = total;
    offsets[tid] = base;
    for (int c = 0; c < nchunks; ++c) {
      int32_t* p = chunk_counts + static_cast<size_t>(c) * E + tid;
      const int n = *p;
      *p = base;
      base += n;
    }
  }
  if (tid == 0) offsets[E] = scan_tmp[E - 1];
}

__global__ void __launch_bounds__(256) dispatch_scatter_kernel(const int32_t* __restrict__ ids, int T,
                                                               int E, int K,
                                                               const int32_t* __restrict__ chunk_base,
                                                               const int32_t* __restrict__ slot_rank,
                                                               int32_t* __restrict__ perm) {
  const int nslots = T * K;
  for (int s = blockIdx.x * 256 + threadIdx.x; s < nslots; s += gridDim.x * 256) {
    const int e = ids[s];
    if (e < 0 || e >= E) continue;
    const int c = (s / K) / 1024;
    perm[chunk_base[static_cast<size_t>(c) * E + e] + slot_rank[s]] = s;
  }
}

}  // namespace moe
