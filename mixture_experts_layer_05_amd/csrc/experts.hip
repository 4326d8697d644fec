// Routed and shared SwiGLU experts: kernel choice, the float32 kernels and the
// fp8 activation quantiser.
//
//   h[i,:] = silu(x_t W_gate[e]^T) * (x_t W_up[e]^T)      for dispatch row i = (t, e)
//   y[t,:] += w_{t,k} * h[i,:] W_down[e]^T
// and the shared expert as one more group whose rows are all T tokens and whose
// combine weight is sigmoid(x_t . w_g) [SpecForge PR #943, "Modifications":
// shared expert, sigmoid-gated].
//
// bf16 and fp8 weights run on MFMA kernels: stream_gemm.hip (decode-sized M,
// bound by streaming the touched experts' weights) or tile_gemm.hip
// (prefill-sized M, bound by MFMA throughput).  float32 weights (the small
// reference-precision configuration) run on the FMA kernels below, one output
// element per thread.
#include <algorithm>

#include "kernels.h"
#include "schedule.h"

namespace moe {

namespace {

// ---------------------------------------------------------------- float32 experts (FMA)

// Tile of 16 rows x 16 columns, one output per thread of a 256-thread block.
__global__ void __launch_bounds__(256) gate_up_f32_kernel(ExpertArgs a) {
  __shared__ int prefix[kSchedInts];
  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int total = build_tile_prefix(prefix, a.counts, a.offsets, a.E, a.T, has_shared, 16, (a.I + 15) / 16,
                                      has_shared ? (a.S + 15) / 16 : 0);
  const int H = a.H;
  const float* x = static_cast<const float*>(a.x);
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const TileInfo t = find_tile(prefix, G, tile, a, 16);
    const int width = t.shared ? a.S : a.I;
    const int m = t.m0 + (threadIdx.x >> 4);
    const int col = t.nt * 16 + (threadIdx.x & 15);
    if (m >= t.rows || col >= width) continue;
    const float* wg = static_cast<const float*>(t.shared ? a.ws_gate : a.w_gate);
    const float* wu = static_cast<const float*>(t.shared ? a.ws_up : a.w_up);
    if (!t.shared) {
      wg += static_cast<size_t>(t.group) * a.I * H;
      wu += static_cast<size_t>(t.group) * a.I * H;
    }
    const float* xr = x + static_cast<size_t>(row_token(a, t, m)) * H;
    const float* gr = wg + static_cast<size_t>(col) * H;
    const float* ur = wu + static_cast<size_t>(col) * H;
    float sg = 0.f, su = 0.f;
    for (int k = 0; k < H; ++k) {
      sg = fmaf(xr[k], gr[k], sg);
      su = fmaf(xr[k], ur[k], su);
    }
    const size_t idx = t.shared ? a.h_shared + static_cast<size_t>(m) * width + col
                                : static_cast<size_t>(t.rowbase + m) * width + col;
    static_cast<float*>(a.h)[idx] = silu_f32(sg) * su;
  }
}

__global__ void __launch_bounds__(256) down_f32_kernel(ExpertArgs a) {
  __shared__ int prefix[kSchedInts];
  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int H = a.H;
  const int total = build_tile_prefix(prefix, a.counts, a.offsets, a.E, a.T, has_shared, 16, (H + 15) / 16,
                                      has_shared ? (H + 15) / 16 : 0);
  const float* hb = static_cast<const float*>(a.h);
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const TileInfo t = find_tile(prefix, G, tile, a, 16);
    const int kdim = t.shared ? a.S : a.I;
    const int m = t.m0 + (threadIdx.x >> 4);
    const int col = t.nt * 16 + (threadIdx.x & 15);
    if (m >= t.rows || col >= H) continue;
    const float* wd = static_cast<const float*>(t.shared ? a.ws_down : a.w_down);
    if (!t.shared) wd += static_cast<size_t>(t.group) * H * a.I;
    const float* hr = hb + (t.shared ? a.h_shared + static_cast<size_t>(m) * kdim
                                     : static_cast<size_t>(t.rowbase + m) * kdim);
    const float* dr = wd + static_cast<size_t>(col) * kdim;
    float s = 0.f;
    for (int k = 0; k < kdim; ++k) s = fmaf(hr[k], dr[k], s);
    const DownDst dst = down_row(a, t, m);
    dst.row[col] = dst.w * s;
  }
}

// ---------------------------------------------------------------- combine

// y[t,:] (+)= sum over k of w[t,k] * o[t*K+k,:], k ascending, skipping dropped
// slots (weight 0, row never written).  `accumulate` adds onto the shared
// expert's term already stored in y.  If y_act is not null the same values also
// go there in the activation dtype.  A workgroup item is one token's run of
// 1024 columns (256 float4), so small T still spreads over every CU.  KT > 0: the
// kernel for K = KT with H a multiple of 4, in which a thread's K row loads are
// all issued before the first add (the weights are uniform over the item, so the
// skip of a dropped slot is a scalar branch) and marked non-temporal: each slot
// row is read once, and keeping it out of the caches ran the large layer's
// combine ~15 % faster (measured); KT = 0: any K and H.
constexpr int kCombineCols = 1024;   // 256 threads x one float4

__device__ __forceinline__ void store_act(void* y_act, int act_bf16, bool act_vec, size_t row, int c, float4 s) {
  if (!act_vec) {
    const float v[4] = {s.x, s.y, s.z, s.w};
    for (int e = 0; e < 4; ++e) {
      if (act_bf16) static_cast<uint16_t*>(y_act)[row + 4 * c + e] = f32_to_bf16_bits(v[e]);
      else static_cast<float*>(y_act)[row + 4 * c + e] = v[e];
    }
  } else if (act_bf16) {
    // bf16: round to nearest (ties to even).  Four values per store when y_act is
    // aligned for it (it need only be aligned to its element size).
    const uint32_t lo = f32_to_bf16_bits(s.x) | (static_cast<uint32_t>(f32_to_bf16_bits(s.y)) << 16);
    const uint32_t hi = f32_to_bf16_bits(s.z) | (static_cast<uint32_t>(f32_to_bf16_bits(s.w)) << 16);
    reinterpret_cast<uint2*>(static_cast<uint16_t*>(y_act) + row)[c] = uint2{lo, hi};
  } else {
    reinterpret_cast<float4*>(static_cast<float*>(y_act) + row)[c] = s;
  }
}

template <int KT>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ o,
                                                      const float* __restrict__ topk_w,
                                                      float* __restrict__ y, void* __restrict__ y_act,
                                                      int act_bf16, int T, int H, int K, int accumulate) {
  const int nchunk = (H + kCombineCols - 1) / kCombineCols;
  const bool act_vec = reinterpret_cast<uintptr_t>(y_act) % (act_bf16 ? 8 : 16) == 0;
  const int64_t items = static_cast<int64_t>(T) * nchunk;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int t = static_cast<int>(it / nchunk);
    const int c0 = static_cast<int>(it - static_cast<int64_t>(t) * nchunk) * kCombineCols;
    const float* wr = topk_w + static_cast<size_t>(t) * K;
    const float* orow = o + static_cast<size_t>(t) * K * H;
    float* yr = y + static_cast<size_t>(t) * H;
    const size_t row = static_cast<size_t>(t) * H;
    if constexpr (KT > 0) {
      const int c = c0 / 4 + static_cast<int>(threadIdx.x);
      if (c < min(H, c0 + kCombineCols) / 4) {
        float w[KT];
        float4 v[KT];
#pragma unroll
        for (int k = 0; k < KT; ++k) w[k] = wr[k];
#pragma unroll
        for (int k = 0; k < KT; ++k)
          if (w[k] != 0.f) {
            const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(orow + static_cast<size_t>(k) * H) + c);
            v[k] = float4{q[0], q[1], q[2], q[3]};
          }
        float4 s = accumulate ? reinterpret_cast<const float4*>(yr)[c] : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          if (w[k] == 0.f) continue;
          s.x = fmaf(w[k], v[k].x, s.x);
          s.y = fmaf(w[k], v[k].y, s.y);
          s.z = fmaf(w[k], v[k].z, s.z);
          s.w = fmaf(w[k], v[k].w, s.w);
        }
        reinterpret_cast<float4*>(yr)[c] = s;
        if (y_act) store_act(y_act, act_bf16, act_vec, row, c, s);
      }
    } else if ((H & 3) == 0) {
      const int cend = min(H, c0 + kCombineCols) / 4;
      for (int c = c0 / 4 + static_cast<int>(threadIdx.x); c < cend; c += blockDim.x) {
        float4 s = accumulate ? reinterpret_cast<const float4*>(yr)[c] : float4{0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < K; ++k) {
          const float w = wr[k];
          if (w == 0.f) continue;
          const float4 v = reinterpret_cast<const float4*>(orow + static_cast<size_t>(k) * H)[c];
          s.x = fmaf(w, v.x, s.x);
          s.y = fmaf(w, v.y, s.y);
          s.z = fmaf(w, v.z, s.z);
          s.w = fmaf(w, v.w, s.w);
        }
        reinterpret_cast<float4*>(yr)[c] = s;
        if (y_act) store_act(y_act, act_bf16, act_vec, row, c, s);
      }
    } else {
      for (int c = c0 + static_cast<int>(threadIdx.x); c < min(H, c0 + kCombineCols); c += blockDim.x) {
        float s = accumulate ? yr[c] : 0.f;
        for (int k = 0; k < K; ++k) {
          const float w = wr[k];
          if (w != 0.f) s = fmaf(w, orow[static_cast<size_t>(k) * H + c], s);
        }
        yr[c] = s;
        if (y_act) {
          if (act_bf16) static_cast<uint16_t*>(y_act)[row + c] = f32_to_bf16_bits(s);
          else static_cast<float*>(y_act)[row + c] = s;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fp8 activation quantiser

// Per row and per 128-element group: amax, s = amax / 448 (1 if amax = 0),
// q = e4m3(RNE(clamp(v / s, +-448))).  32 lanes (half a wave) per group, four
// elements per lane.  Rows [0, rows_host) of src, or [0, *rows_dev) if rows_dev,
// then, if seg1_items > 0, seg1_items more groups starting at element seg1 (the
// shared expert's rows of h, in the same launch).
template <bool SRC_BF16>
__global__ void __launch_bounds__(256) quant_g128_kernel(const void* __restrict__ src, int rows_host,
                                                         const int32_t* __restrict__ rows_dev, int cols,
                                                         size_t seg1, size_t seg1_items,
                                                         uint8_t* __restrict__ q, float* __restrict__ s) {
  const int rows = rows_dev ? *rows_dev : rows_host;
  const int ng = cols / kGroup;
  const size_t items0 = static_cast<size_t>(rows) * ng;
  const size_t items = items0 + seg1_items;
  const int half = threadIdx.x >> 5, hl = threadIdx.x & 31;
  for (size_t it = static_cast<size_t>(blockIdx.x) * 8 + half; it < items;
       it += static_cast<size_t>(gridDim.x) * 8) {
    // Rows are contiguous: (row, group) -> element it*128 of its segment.
    const size_t g0 = it < items0 ? it * kGroup : seg1 + (it - items0) * kGroup;
    const size_t base = g0 + 4 * hl;
    float v[4];
    if constexpr (SRC_BF16) {
      const uint2 p = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + base);
      v[0] = bf16_bits_to_f32(p.x & 0xffffu);
      v[1] = bf16_bits_to_f32(p.x >> 16);
      v[2] = bf16_bits_to_f32(p.y & 0xffffu);
      v[3] = bf16_bits_to_f32(p.y >> 16);
    } else {
      const float4 p = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + base);
      v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
    }
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = fminf(fmaxf(v[e] / sc, -448.0f), 448.0f);
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], packed, true);
    *reinterpret_cast<int*>(q + base) = packed;
    if (hl == 0) s[g0 / kGroup] = sc;
  }
}

// MXFP8 activations for the MXFP4 contraction [OCP MX v1.0 scale rule]: per row
// and 32-element block, amax, shared exponent s = floor(log2(amax)) - 8 clamped to
// >= -127 (0 for an all-zero block), scale byte s + 127, element = e4m3 RNE of
// clamp(v * 2^-s, +-448).  2^-s is built from its exponent bits, so the product is
// exact.  Eight lanes per block, four elements per lane.  Rows [0, rows_host) of
// src, or [0, *rows_dev) if rows_dev, then seg1_items more blocks from element
// seg1 (as quant_g128_kernel).
template <bool SRC_BF16>
__global__ void __launch_bounds__(256) quant_mx8_kernel(const void* __restrict__ src, int rows_host,
                                                        const int32_t* __restrict__ rows_dev, int cols,
                                                        size_t seg1, size_t seg1_items,
                                                        uint8_t* __restrict__ q, uint8_t* __restrict__ e8) {
  const int rows = rows_dev ? *rows_dev : rows_host;
  const size_t items0 = static_cast<size_t>(rows) * (cols / kMxBlock);
  const size_t items = items0 + seg1_items;
  const int blk = threadIdx.x >> 3, bl = threadIdx.x & 7;
  for (size_t it = static_cast<size_t>(blockIdx.x) * 32 + blk; it < items;
       it += static_cast<size_t>(gridDim.x) * 32) {
    // Rows are contiguous: (row, block) -> element it*32 of its segment.
    const size_t b0 = it < items0 ? it * kMxBlock : seg1 + (it - items0) * kMxBlock;
    const size_t base = b0 + 4 * bl;
    float v[4];
    if constexpr (SRC_BF16) {
      const uint2 p = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + base);
      v[0] = bf16_bits_to_f32(p.x & 0xffffu);
      v[1] = bf16_bits_to_f32(p.x >> 16);
      v[2] = bf16_bits_to_f32(p.y & 0xffffu);
      v[3] = bf16_bits_to_f32(p.y >> 16);
    } else {
      const float4 p = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + base);
      v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
    }
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
    for (int o = 4; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    const int ebits = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
    int s = 0;
    if (amax > 0.f) s = (ebits == 0) ? -127 : max(ebits - 127 - 8, -127);
    const float mul = __uint_as_float(static_cast<uint32_t>(127 - s) << 23);   // 2^-s
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = fminf(fmaxf(v[e] * mul, -448.0f), 448.0f);
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], packed, true);
    *reinterpret_cast<int*>(q + base) = packed;
    if (bl == 0) e8[b0 / kMxBlock] = static_cast<uint8_t>(s + 127);
  }
}

// ---------------------------------------------------------------- launch helpers

constexpr int kMaxGrid = 2048;

int tile_bound(const ExpertArgs& a, int BM, int nt_routed, int nt_shared) {
  const int64_t slots = static_cast<int64_t>(a.T) * a.K;
  const int64_t mt = slots / BM + std::min<int64_t>(a.E, slots);
  int64_t b = mt * nt_routed;
  if (a.S > 0) b += ceil_div(a.T, BM) * nt_shared;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(b, kMaxGrid)));
}

// Rows per expert decide the kernels.  The average expert sees rho = T*K/E rows
// (the load measure of the small-M / large-M family choice of [DeepGEMM fork
// PR #5, "Dynamic family selection"]).  By default the weight-streaming kernels
// alone (stream_gemm.hip, which pick their tile height from rho).  A call whose
// rows could fill the GPU with 256-row tiles (T*K*I >= 256 CUs x 256 rows x 128
// columns) and whose experts see at least kMixRows rows on average is instead
// divided by its realised counts, read on the device (schedule.h,
// build_tile_prefix), whatever its weight format: rows that fill a 256-row
// tile at least half go to the LDS-tiled MFMA kernels (tile_gemm.hip), short
// groups and the short tails of long ones to the streaming kernel.  Two launches,
// disjoint rows.  Measured: the large layer at T = 512-1024 with Zipf skew
// alpha >= 1 runs 22-30 % faster split; a call too small to fill the GPU with
// 256-row tiles runs them nearly alone (the drafter at T = 224, whose shared
// expert would be one 224-row group: 1.7x slower).
constexpr int64_t kMixRows = 16;

bool split_call(const ExpertArgs& a, int weight_dtype, int64_t rho) {
  return rho >= kMixRows &&
         static_cast<int64_t>(a.T) * a.K * a.I >= int64_t{256} * 256 * 128 && tall_tiles_fit(a);
}

// Tile height for the streaming kernel's share of a split call, through the rows
// per expert it is given: from 192 rows per expert on average that share is mostly
// short tails and cold groups, which 64-row tiles serve better (5 % faster at
// T = 8192, alpha = 0, measured); below, it holds groups just short of 128 rows,
// which 128-row tiles serve better (12 % at T = 4096, alpha = 0).  From 192 rows
// the share is divided once more by group (schedule.h, splits 3 and 4): groups
// left with more than 64 rows take 128-row tiles, the rest 64-row ones.
int64_t rest_rows(int64_t rho) { return rho >= 192 ? 47 : rho; }
constexpr int64_t kMidTileRho = 48;   // selects 128-row streaming tiles

template <typename F>
hipError_t launch_rest(const ExpertArgs& a, int weight_dtype, int64_t rho, F&& launch) {
  ExpertArgs rest = a;
  if (rest_rows(rho) == rho) {
    rest.split = 2;
    return launch(rest, weight_dtype, rho);
  }
  rest.split = 3;
  const hipError_t e = launch(rest, weight_dtype, kMidTileRho);
  if (e != hipSuccess) return e;
  rest.split = 4;
  return launch(rest, weight_dtype, rest_rows(rho));
}

int64_t rows_per_expert(const ExpertArgs& a) { return static_cast<int64_t>(a.T) * a.K / a.E; }

// A forced streaming tile height as the rows per expert that select it (see
// launch_stream_rho in stream_gemm.hip: <= 12 -> 16 rows, <= 24 -> 32, < 48 -> 64,
// else 128).
int64_t forced_rho(int force_tile) {
  switch (force_tile) {
    case 16: return 1;
    case 32: return 20;
    case 64: return 40;
    default: return 48;
  }
}

}  // namespace

bool split_allowed(const ExpertArgs& a, int weight_dtype) {
  return (weight_dtype == kDtypeBf16 || weight_dtype == kDtypeFp8 || weight_dtype == kDtypeMxfp4) && tall_tiles_fit(a);
}

hipError_t launch_gate_up(const ExpertArgs& a, int weight_dtype, hipStream_t stream) {
  if (weight_dtype == kDtypeF32) {
    const int grid = tile_bound(a, 16, (a.I + 15) / 16, (a.S + 15) / 16);
    gate_up_f32_kernel<<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
  }
  const int64_t rho = rows_per_expert(a);
  if (a.force_tile > 0) return launch_gate_up_stream(a, weight_dtype, forced_rho(a.force_tile), stream);
  if (a.force_tile == kForceSplit || split_call(a, weight_dtype, rho)) {
    ExpertArgs tall = a;
    tall.split = 1;
    const hipError_t e = launch_gate_up_tall(tall, weight_dtype, stream);
    if (e != hipSuccess) return e;
    return launch_rest(a, weight_dtype, rho, [&](const ExpertArgs& r, int dt, int64_t rr) {
      return launch_gate_up_stream(r, dt, rr, stream);
    });
  }
  ExpertArgs s = a;
  s.kparts = gate_up_kparts(a.T, a.K, a.E, a.H, a.I, a.S, weight_dtype);
  // The partial sums must fit the workspace's region for them (sized by the same
  // estimate); a call it was not sized for runs unsplit rather than past its end.
  if (s.kparts > 1 && static_cast<size_t>(s.kparts) * gate_up_part_floats(a.T, a.K, a.I, a.S) > a.gpart_floats)
    s.kparts = 1;
  return launch_gate_up_stream(s, weight_dtype, rho, stream);
}

hipError_t launch_down(const ExpertArgs& a, int weight_dtype, hipStream_t stream) {
  if (weight_dtype == kDtypeF32) {
    const int grid = tile_bound(a, 16, (a.H + 15) / 16, (a.H + 15) / 16);
    down_f32_kernel<<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
  }
  const int64_t rho = rows_per_expert(a);
  if (a.force_tile > 0) return launch_down_stream(a, weight_dtype, forced_rho(a.force_tile), stream);
  if ((a.force_tile == kForceSplit || split_call(a, weight_dtype, rho)) && a.H % 256 == 0) {
    ExpertArgs tall = a;
    tall.split = 1;
    const hipError_t e = launch_down_tall(tall, weight_dtype, stream);
    if (e != hipSuccess) return e;
    return launch_rest(a, weight_dtype, rho, [&](const ExpertArgs& r, int dt, int64_t rr) {
      return launch_down_stream(r, dt, rr, stream);
    });
  }
  return launch_down_stream(a, weight_dtype, rho, stream);
}

hipError_t launch_combine(const ExpertArgs& a, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(a.T) * ceil_div(a.H, kCombineCols);
  const int grid = static_cast<int>(std::min<int64_t>(items, 65536));
  const int acc = a.S > 0 ? 1 : 0;
#define MOE_COMBINE(KT) combine_kernel<KT><<<grid, 256, 0, stream>>>(a.o, a.topk_w, a.y, a.y_act, a.act_bf16, a.T, \
                                                                 a.H, a.K, acc)
  switch (a.H % 4 == 0 ? a.K : 0) {
    case 1: MOE_COMBINE(1); break;
    case 2: MOE_COMBINE(2); break;
    case 4: MOE_COMBINE(4); break;
    case 6: MOE_COMBINE(6); break;
    case 8: MOE_COMBINE(8); break;
    case 10: MOE_COMBINE(10); break;
    default: MOE_COMBINE(0); break;
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

hipError_t launch_quant_x(const ExpertArgs& a, uint8_t* xq, float* xs, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(a.T) * (a.H / kGroup);
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ceil_div(items, 8), 4096)));
  quant_g128_kernel<true><<<grid, 256, 0, stream>>>(a.x, a.T, nullptr, a.H, 0, 0, xq, xs);
  return hipGetLastError();
}

hipError_t launch_quant_x_mx(const ExpertArgs& a, uint8_t* xq, uint8_t* xe8, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(a.T) * (a.H / kMxBlock);
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ceil_div(items, 32), 4096)));
  quant_mx8_kernel<true><<<grid, 256, 0, stream>>>(a.x, a.T, nullptr, a.H, 0, 0, xq, xe8);
  return hipGetLastError();
}

// One launch over h: the routed rows the dispatch kept (their count read on the
// device from offsets[E]), then the shared expert's T rows at h_shared.
hipError_t launch_quant_h_mx(const ExpertArgs& a, uint8_t* hq, uint8_t* he8, hipStream_t stream) {
  const int64_t items_s = a.S > 0 ? static_cast<int64_t>(a.T) * (a.S / kMxBlock) : 0;
  const int64_t items = static_cast<int64_t>(a.T) * a.K * (a.I / kMxBlock) + items_s;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ceil_div(items, 32), 4096)));
  quant_mx8_kernel<false><<<grid, 256, 0, stream>>>(a.h, 0, a.offsets + a.E, a.I, a.h_shared,
                                                    static_cast<size_t>(items_s), hq, he8);
  return hipGetLastError();
}

hipError_t launch_quant_h(const ExpertArgs& a, uint8_t* hq, float* hs, hipStream_t stream) {
  const int64_t items_s = a.S > 0 ? static_cast<int64_t>(a.T) * (a.S / kGroup) : 0;
  const int64_t items = static_cast<int64_t>(a.T) * a.K * (a.I / kGroup) + items_s;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ceil_div(items, 8), 4096)));
  quant_g128_kernel<false><<<grid, 256, 0, stream>>>(a.h, 0, a.offsets + a.E, a.I, a.h_shared,
                                                     static_cast<size_t>(items_s), hq, hs);
  return hipGetLastError();
}

}  // namespace moe
