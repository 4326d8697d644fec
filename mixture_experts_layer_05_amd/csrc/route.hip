// Router: logits GEMV, softmax top-k with renormalisation, expert budget.
//
// Logits z[t,e] = x_t . W_r[e] are accumulated in float32; the shared-expert gate
// logit x_t . w_g rides along as one extra column.  Selection follows the
// "softmax, renormalised top-k" preset of [SpecForge PR #943, "Modifications"];
// the budget follows [colibri issue_budget.md, "How it works", steps 1-5].
#include "kernels.h"

namespace moe {

// ------------------------------------------------------------------ logits, bf16 (MFMA)
//
// One workgroup = 4 waves computes a 16-token x 32-column tile (two 16-column
// MFMA blocks sharing the token fragments) over one of P contiguous parts of the
// hidden dimension; the waves split the part into four ranges and their partial
// tiles are summed through LDS.  Part p writes its partial logits to plane p of
// z (p * plane floats further on); the top-k kernel adds the planes in order
// 0..P-1, so the result does not depend on timing.  Splitting the contraction
// gives a decode-sized batch enough workgroups to keep its loads in flight.
// Column c < E is W_r[c], column E (if present) is w_g, the rest of the padded
// tile is computed on a repeated column and not stored.  Every product of two
// bf16 values is exact in float32 and the MFMA accumulates in float32.
__global__ void __launch_bounds__(256) router_logits_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_router,
    const uint16_t* __restrict__ w_gate_col, int T, int H, int E, int ncols,
    float* __restrict__ z, int ldz, size_t plane) {
  __shared__ f32x4 red[4][2][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * 16, c0 = blockIdx.y * 32;
  const int part = blockIdx.z, parts = gridDim.z;
  const int t = min(t0 + r, T - 1);
  const uint16_t* arow = x + static_cast<size_t>(t) * H;
  const uint16_t* brow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = min(c0 + 16 * j + r, ncols - 1);
    brow[j] = (c < E) ? w_router + static_cast<size_t>(c) * H : w_gate_col;
  }
  const int nch = H / 128;
  const int pb = (part * nch) / parts, pe = ((part + 1) * nch) / parts;
  const int kb = pb + (wave * (pe - pb)) / 4, ke = pb + ((wave + 1) * (pe - pb)) / 4;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int kc = kb; kc < ke; ++kc) {
    const int k = kc * 128 + 32 * g;
    uint4 a[4], b[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = *reinterpret_cast<const uint4*>(arow + k + 8 * q);
      b[0][q] = *reinterpret_cast<const uint4*>(brow[0] + k + 8 * q);
      b[1][q] = *reinterpret_cast<const uint4*>(brow[1] + k + 8 * q);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[0] = mfma_bf16_16x16x32(a[q], b[0][q], acc[0]);
      acc[1] = mfma_bf16_16x16x32(a[q], b[1][q], acc[1]);
    }
  }
  red[wave][0][lane] = acc[0];
  red[wave][1][lane] = acc[1];
  __syncthreads();
  if (wave < 2) {
    const int j = wave;
    f32x4 sum = red[0][j][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 o = red[w][j][lane];
      sum[0] += o[0]; sum[1] += o[1]; sum[2] += o[2]; sum[3] += o[3];
    }
    const int col = c0 + 16 * j + mfma16_col(lane);
    float* zp = z + static_cast<size_t>(part) * plane;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = t0 + mfma16_row(lane, i);
      if (row < T && col < ncols) zp[static_cast<size_t>(row) * ldz + col] = sum[i];
    }
  }
}

// ------------------------------------------------------------------ logits, f32 (FMA)
//
// One wave per (token, column): lanes stride the hidden dimension, then a wave sum.
__global__ void __launch_bounds__(256) router_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w_router,
    const float* __restrict__ w_gate_col, int T, int H, int E, int ncols,
    float* __restrict__ z, int ldz) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= T * ncols) return;
  const int t = item / ncols, c = item % ncols;
  const float* a = x + static_cast<size_t>(t) * H;
  const float* b = (c < E) ? w_router + static_cast<size_t>(c) * H : w_gate_col;
  float s = 0.f;
  for (int h = lane; h < H; h += kWave) s = fmaf(a[h], b[h], s);
  s = wave_sum(s);
  if (lane == 0) z[static_cast<size_t>(t) * ldz + c] = s;
}

// ------------------------------------------------------------------ top-k
//
// One wave per token.  Lane l holds experts l, l+64, ... (up to 8 each).  K rounds
// of a wave-wide argmax on (logit desc, id asc) pick the ids in descending
// order.  A NaN logit counts as -inf; a picked expert is marked taken (a per-lane
// bit mask) and leaves the candidates, so even -inf logits (experts masked through
// the bias) are picked at most once and every id lies in [0, E).  Weights: exp(z_k - z_max) over the K picks, divided by their sum
// (renormalised top-k) or by the sum over all E experts (plain softmax).
// top_p in (0, 1): pick k survives iff the picks before it hold less than top_p
// of the K picks' summed weight (so pick 0 always survives); the others become
// id -1 / weight 0 and a renormalised top-k is taken over the survivors only.
// The prefix sums run in pick order, the same for every lane.
__global__ void __launch_bounds__(256) topk_kernel(
    const float* __restrict__ z, int ldz, int parts, size_t plane, const float* __restrict__ bias, int T,
    int E, int K, int norm_topk, float top_p, int has_shared, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, float* __restrict__ shared_gate, unsigned long long* __restrict__ budget_agg,
    int32_t* __restrict__ budget_present) {
  // The expert budget's accumulators start at zero in every call (the budget pass
  // runs after this kernel on the same stream).
  if (budget_agg && blockIdx.x == 0) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      budget_agg[e] = 0ull;
      budget_present[e] = 0;
    }
  }
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* zr = z + static_cast<size_t>(t) * ldz;
  // Logit of column c: the partial planes added in order 0..parts-1.
  auto logit = [&](int c) {
    float s = zr[c];
    for (int p = 1; p < parts; ++p) s += zr[static_cast<size_t>(p) * plane + c];
    return s;
  };
  // The shared-expert gate logit is read up front, next to the expert logits.
  const float gate_logit = (has_shared && lane == 0) ? logit(E) : 0.f;
  float v[kMaxExperts / kWave];
#pragma unroll
  for (int j = 0; j < kMaxExperts / kWave; ++j) {
    const int e = lane + kWave * j;
    float val = -INFINITY;
    if (e < E) {
      val = logit(e);
      if (bias) val += bias[static_cast<size_t>(t) * E + e];
      if (val != val) val = -INFINITY;   // NaN
    }
    v[j] = val;
  }
  // Plain-softmax denominator (only needed without renormalisation).
  float zmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMaxExperts / kWave; ++j) zmax = fmaxf(zmax, v[j]);
  zmax = wave_max(zmax);
  float denom_all = 0.f;
  if (!norm_topk) {
#pragma unroll
    for (int j = 0; j < kMaxExperts / kWave; ++j)
      if (lane + kWave * j < E) denom_all += expf(v[j] - zmax);
    denom_all = wave_sum(denom_all);
  }
  int my_id = -1;
  float my_z = 0.f;
  unsigned taken = 0;   // bit j: expert lane + 64 j already picked
  for (int k = 0; k < K; ++k) {
    // Lane-local best among the untaken: largest value, lowest id on ties (ids
    // grow with j).  be = 0x7fffffff marks a lane with no candidate left.
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kMaxExperts / kWave; ++j) {
      const int e = lane + kWave * j;
      if (e < E && !((taken >> j) & 1u) && (v[j] > bv || (v[j] == bv && e < be))) { bv = v[j]; be = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oe = __shfl_xor(be, o, kWave);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    // K <= E, so some lane still had a candidate and be is a valid id.
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == k) { my_id = be; my_z = bv; }
  }
  // The first pick is the maximum logit.
  const float zmax_k = __shfl(my_z, 0, kWave);
  float p = (lane < K) ? expf(my_z - zmax_k) : 0.f;
  bool kept = lane < K;
  if (top_p > 0.f) {
    float before = 0.f, all = 0.f;   // weight of the picks before this lane's, of all K
    for (int k = 0; k < K; ++k) {
      const float pk = __shfl(p, k, kWave);
      if (k < lane) before += pk;
      all += pk;
    }
    kept = kept && (lane == 0 || before < top_p * all);
  }
  const float pk = kept ? p : 0.f;
  float denom = norm_topk ? wave_sum(pk) : denom_all * expf(zmax - zmax_k);
  if (lane < K) {
    topk_ids[static_cast<size_t>(t) * K + lane] = kept ? my_id : -1;
    topk_w[static_cast<size_t>(t) * K + lane] = pk / denom;
  }
  if (has_shared && lane == 0) shared_gate[t] = 1.0f / (1.0f + expf(-gate_logit));
}

// ------------------------------------------------------------------ expert budget
//
// Two passes over the batch.  The aggregate gate weight of an expert is an exact
// sum of fixed-point weights (each float32 weight rounded to a multiple of 2^-33,
// summed as 64-bit integers), so it does not depend on the order the slots are
// added in, and the keep-set is a pure function of the routing whatever the
// timing.  Its distance to the float64 sum is at most T * K * 2^-34 (4e-6 at
// 65536 slots), far inside the gaps the ranking is decided on.
//  1. budget_aggregate_kernel, one workgroup per 256-token chunk: integer atomics
//     into LDS per expert, then one global 64-bit atomic per touched expert (the
//     accumulators are zeroed by the top-k kernel of the same call)
//     [colibri issue_budget.md, "How it works" step 1];
//  2. budget_apply_kernel, one workgroup per 256 tokens: every workgroup ranks the
//     union by (aggregate desc, id asc) and keeps rank < B [steps 2-3] (the same
//     few microseconds in each, instead of a third launch); then one thread per
//     token compacts its kept slots to the front in
//     their original order, -1 / 0 into the tail, and renormalises the kept
//     weights if norm_topk (not when none is left) [steps 4-5].  Workgroup 0
//     writes statistics 0-1; dropped slots and emptied tokens go into statistics
//     2-3 by integer atomics (zeroed by the first pass).
// With B = 0 or union <= B the routing is left as it is and only the statistics
// {union, union, 0, 0} are written.
constexpr int kBudgetChunk = kBudgetChunkTokens;   // tokens per workgroup of both passes
constexpr double kBudgetFixed = 8589934592.0;   // 2^33

__global__ void __launch_bounds__(kBudgetChunk) budget_aggregate_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int T, int E, int K,
    unsigned long long* __restrict__ agg_fixed, int32_t* __restrict__ present, int32_t* __restrict__ stats) {
  __shared__ unsigned long long lagg[kMaxExperts];
  __shared__ int lcnt[kMaxExperts];
  const int tid = threadIdx.x;
  if (stats && blockIdx.x == 0 && tid < 2) stats[2 + tid] = 0;
  for (int e = tid; e < kMaxExperts; e += kBudgetChunk) {
    lagg[e] = 0ull;
    lcnt[e] = 0;
  }
  __syncthreads();
  const size_t s0 = static_cast<size_t>(blockIdx.x) * kBudgetChunk * K;
  const int nslot = max(0, min(kBudgetChunk, T - static_cast<int>(blockIdx.x) * kBudgetChunk)) * K;
  for (int i = tid; i < nslot; i += kBudgetChunk) {
    const int e = ids[s0 + i];
    if (e >= 0 && e < E) {
      const unsigned long long f =
          static_cast<unsigned long long>(llrint(static_cast<double>(w[s0 + i]) * kBudgetFixed));
      atomicAdd(&lagg[e], f);
      lcnt[e] = 1;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kBudgetChunk)
    if (lcnt[e]) {
      if (lagg[e]) atomicAdd(&agg_fixed[e], lagg[e]);
      present[e] = 1;
    }
}

__global__ void __launch_bounds__(kBudgetChunk) budget_apply_kernel(
    int32_t* __restrict__ ids, float* __restrict__ w, int T, int E, int K, int budget, int norm_topk,
    const unsigned long long* __restrict__ agg_fixed, const int32_t* __restrict__ present,
    int32_t* __restrict__ stats) {
  __shared__ double key[kMaxExperts];
  __shared__ int keep[kMaxExperts];
  __shared__ int s_union, s_dropped, s_empty;
  const int tid = threadIdx.x;
  if (tid == 0) { s_union = 0; s_dropped = 0; s_empty = 0; }
  __syncthreads();
  // The union ranked by (aggregate desc, id asc); an absent expert gets key -1,
  // below every present one.
  for (int e = tid; e < kMaxExperts; e += kBudgetChunk) {
    const bool p = e < E && present[e] != 0;
    key[e] = p ? static_cast<double>(agg_fixed[e]) : -1.0;
    if (p) atomicAdd(&s_union, 1);
  }
  __syncthreads();
  const int nu = s_union;
  const bool active = budget > 0 && nu > budget;
  if (blockIdx.x == 0 && tid == 0 && stats) {
    stats[0] = nu;
    stats[1] = active ? budget : nu;
  }
  if (!active) return;   // uniform
  // Rank of each present expert: the present experts with a larger aggregate, or
  // an equal one and a lower id (every thread reads the same key at a time).
  for (int e = tid; e < E; e += kBudgetChunk) {
    const double a = key[e];
    int r = 0;
    if (a >= 0.0) {
#pragma unroll 8
      for (int o = 0; o < E; ++o) {
        const double b = key[o];
        r += (b > a || (b == a && o < e)) ? 1 : 0;
      }
    }
    keep[e] = (a >= 0.0 && r < budget) ? 1 : 0;
  }
  __syncthreads();
  const int t = blockIdx.x * kBudgetChunk + tid;
  if (t < T) {
    int32_t* ir = ids + static_cast<size_t>(t) * K;
    float* wr = w + static_cast<size_t>(t) * K;
    int nk = 0, nd = 0;
    float sum = 0.f;
    for (int k = 0; k < K; ++k) {
      const int e = ir[k];
      if (e < 0 || e >= E) continue;
      if (keep[e]) { sum += wr[k]; ++nk; } else { ++nd; }
    }
    if (nd) {
      // Compact in place: position j <= k has already been read when it is written.
      int j = 0;
      for (int k = 0; k < K; ++k) {
        const int e = ir[k];
        if (e >= 0 && e < E && keep[e]) {
          const float v = wr[k];
          ir[j] = e;
          wr[j] = norm_topk ? v / sum : v;
          ++j;
        }
      }
      for (; j < K; ++j) { ir[j] = -1; wr[j] = 0.f; }
      atomicAdd(&s_dropped, nd);
    }
    if (nk == 0) atomicAdd(&s_empty, 1);
  }
  __syncthreads();
  if (tid == 0 && stats) {
    if (s_dropped) atomicAdd(&stats[2], s_dropped);
    if (s_empty) atomicAdd(&stats[3], s_empty);
  }
}

}  // namespace moe
