// Routed and shared SwiGLU experts: grouped gate/up with fused SwiGLU, then
// grouped down with the gate-weighted combine.
//
//   h[i,:] = silu(x_t W_gate[e]^T) * (x_t W_up[e]^T)      for dispatch row i = (t, e)
//   y[t,:] += w_{t,k} * h[i,:] W_down[e]^T
// and the shared expert as one more group whose rows are all T tokens and whose
// combine weight is sigmoid(x_t . w_g) [SpecForge PR #943, "Modifications":
// shared expert, sigmoid-gated].
//
// Work decomposition.  A "group" is a routed expert (rows = its dispatch
// segment) or the shared expert (rows = every token).  A tile is (group,
// m-tile of BM rows, n-tile of output columns).  Each launch is persistent: a
// workgroup builds the per-group tile prefix from expert_counts in LDS (no
// host round trip) and strides over the tile list, where the m-tiles of one
// (group, n-tile) are adjacent so that the weight slab they share is fetched
// from HBM once and served from L2 to the rest.
//
// Inside a tile the waves of the workgroup split the contraction dimension into
// contiguous ranges; each wave streams its weight rows straight from HBM into
// registers with 16-byte loads (lane groups of four cover 256 contiguous bytes
// of a row per step), multiplies with MFMA, and the partial tiles are summed in
// LDS.  The down kernel stages the finished tile in LDS so that each wave
// issues its float32 atomic adds as whole 64-column (256-byte) row segments,
// rather than scattered 16-byte pieces -- the row-staged scatter idea of
// [DeepGEMM fork PR #5, "What changed -- large M", L2 scatter].
#include <algorithm>

#include "kernels.h"
#include "schedule.h"

namespace moe {

namespace {

// ---------------------------------------------------------------- wave-level MFMA streams
//
// Contraction chunks are 128 elements.  For bf16, chunk step s (0..3) covers
// elements [32s, 32s+32); lane group g = lane/16 holds elements [32s+8g, +8) of its
// row, so the four lanes of a row read 64 contiguous bytes per load instruction.
// The next chunk's loads are issued before the current chunk's MFMAs (register
// double buffering), so every wave keeps a full chunk of weight bytes in flight.

template <int RM, int CN>
struct Bf16Chunk {
  uint4 a[RM][4], b[CN][4];
  __device__ __forceinline__ void load(const uint16_t* const (&arow)[RM], const uint16_t* const (&brow)[CN],
                                       int kc, int g) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kc * 128 + 32 * s + 8 * g;
#pragma unroll
      for (int j = 0; j < CN; ++j) b[j][s] = ld16_stream(brow[j] + k);
#pragma unroll
      for (int i = 0; i < RM; ++i) a[i][s] = ld16(arow[i] + k);
    }
  }
  __device__ __forceinline__ void mma(f32x4 (&acc)[RM][CN]) const {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < CN; ++j) acc[i][j] = mfma_bf16_16x16x32(a[i][s], b[j][s], acc[i][j]);
  }
};

// acc[i][j] += A(row block i) . B(column block j) over chunks [kb, ke).
// arow[i] / brow[j] point at this lane's row (lane % 16) of each block.
template <int RM, int CN>
__device__ __forceinline__ void wave_mma_bf16(const uint16_t* const (&arow)[RM],
                                              const uint16_t* const (&brow)[CN], int kb, int ke, int g,
                                              f32x4 (&acc)[RM][CN]) {
  if (kb >= ke) return;
  Bf16Chunk<RM, CN> c0, c1;
  c0.load(arow, brow, kb, g);
  int kc = kb;
  for (; kc + 1 < ke; kc += 2) {
    c1.load(arow, brow, kc + 1, g);
    c0.mma(acc);
    if (kc + 2 < ke) c0.load(arow, brow, kc + 2, g);
    c1.mma(acc);
  }
  if (kc < ke) c0.mma(acc);
}

// fp8: one MFMA per 128-element chunk = one scale group.  Lane group g holds bytes
// [16g, 16g+16) and [64+16g, 64+16g+16) of its row's chunk (two 64-byte runs across
// the four lanes of a row).  ascale[i][e] points at the scale row of output row
// 4*(lane/16)+e of block i, bscale[j] at the scale row of this lane's output column;
// partial products are rescaled in float32.
template <int RM, int CN>
struct Fp8Chunk {
  i32x8 a[RM], b[CN];
  float sa[RM][4], sb[CN];
  __device__ __forceinline__ static i32x8 pack(uint4 lo, uint4 hi) {
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  __device__ __forceinline__ void load(const uint8_t* const (&arow)[RM], const float* const (&ascale)[RM][4],
                                       const uint8_t* const (&brow)[CN], const float* const (&bscale)[CN],
                                       int kc, int g) {
    const int k = kc * 128 + 16 * g;
#pragma unroll
    for (int j = 0; j < CN; ++j) b[j] = pack(ld16_stream(brow[j] + k), ld16_stream(brow[j] + k + 64));
#pragma unroll
    for (int i = 0; i < RM; ++i) a[i] = pack(ld16(arow[i] + k), ld16(arow[i] + k + 64));
#pragma unroll
    for (int j = 0; j < CN; ++j) sb[j] = bscale[j][kc];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sa[i][e] = ascale[i][e][kc];
  }
  __device__ __forceinline__ void mma(f32x4 (&acc)[RM][CN]) const {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < CN; ++j) {
        const f32x4 p = mfma_fp8_16x16x128(a[i], b[j], zero);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(p[e], sa[i][e] * sb[j], acc[i][j][e]);
      }
  }
};

template <int RM, int CN>
__device__ __forceinline__ void wave_mma_fp8(const uint8_t* const (&arow)[RM],
                                             const float* const (&ascale)[RM][4],
                                             const uint8_t* const (&brow)[CN],
                                             const float* const (&bscale)[CN], int kb, int ke, int g,
                                             f32x4 (&acc)[RM][CN]) {
  if (kb >= ke) return;
  Fp8Chunk<RM, CN> c0, c1;
  c0.load(arow, ascale, brow, bscale, kb, g);
  int kc = kb;
  for (; kc + 1 < ke; kc += 2) {
    c1.load(arow, ascale, brow, bscale, kc + 1, g);
    c0.mma(acc);
    if (kc + 2 < ke) c0.load(arow, ascale, brow, bscale, kc + 2, g);
    c1.mma(acc);
  }
  if (kc < ke) c0.mma(acc);
}

// ---------------------------------------------------------------- gate/up + SwiGLU (MFMA)

// Tile: BM = 16*RM rows x 16*CNH intermediate columns (CNH gate blocks and the
// CNH up blocks of the same columns), NWK waves splitting the hidden dimension.
template <int RM, int CNH, int NWK, bool FP8>
__global__ void __launch_bounds__(64 * NWK) gate_up_mfma_kernel(ExpertArgs a) {
  constexpr int BM = 16 * RM, BNH = 16 * CNH, CN = 2 * CNH;
  __shared__ int prefix[kMaxExperts + 2];
  __shared__ f32x4 red[NWK][RM][CN][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;

  zero_output(a);
  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int total = build_tile_prefix(prefix, a.counts, a.E, a.T, has_shared, BM, a.I / BNH,
                                      has_shared ? a.S / BNH : 0);
  const int H = a.H;
  const int nch = H / 128;
  const int kb = (wave * nch) / NWK, ke = ((wave + 1) * nch) / NWK;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const TileInfo t = find_tile(prefix, G, tile, a, BM);
    const int width = t.shared ? a.S : a.I;
    const int n0 = t.nt * BNH;
    f32x4 acc[RM][CN];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < CN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if constexpr (!FP8) {
      const uint16_t* x = static_cast<const uint16_t*>(a.x);
      const uint16_t* wg = static_cast<const uint16_t*>(t.shared ? a.ws_gate : a.w_gate);
      const uint16_t* wu = static_cast<const uint16_t*>(t.shared ? a.ws_up : a.w_up);
      if (!t.shared) {
        wg += static_cast<size_t>(t.group) * a.I * H;
        wu += static_cast<size_t>(t.group) * a.I * H;
      }
      const uint16_t* arow[RM];
#pragma unroll
      for (int i = 0; i < RM; ++i) {
        const int m = min(t.m0 + 16 * i + r, t.rows - 1);
        arow[i] = x + static_cast<size_t>(row_token(a, t, m)) * H;
      }
      const uint16_t* brow[CN];
#pragma unroll
      for (int j = 0; j < CNH; ++j) {
        brow[j] = wg + static_cast<size_t>(n0 + 16 * j + r) * H;
        brow[CNH + j] = wu + static_cast<size_t>(n0 + 16 * j + r) * H;
      }
      wave_mma_bf16<RM, CN>(arow, brow, kb, ke, g, acc);
    } else {
      const int ng = H / kGroup;
      const uint8_t* wg = static_cast<const uint8_t*>(t.shared ? a.ws_gate : a.w_gate);
      const uint8_t* wu = static_cast<const uint8_t*>(t.shared ? a.ws_up : a.w_up);
      const float* sg = t.shared ? a.ss_gate : a.s_gate;
      const float* su = t.shared ? a.ss_up : a.s_up;
      if (!t.shared) {
        wg += static_cast<size_t>(t.group) * a.I * H;
        wu += static_cast<size_t>(t.group) * a.I * H;
        sg += static_cast<size_t>(t.group) * a.I * ng;
        su += static_cast<size_t>(t.group) * a.I * ng;
      }
      const uint8_t* arow[RM];
      const float* ascale[RM][4];
#pragma unroll
      for (int i = 0; i < RM; ++i) {
        const int m = min(t.m0 + 16 * i + r, t.rows - 1);
        arow[i] = a.xq + static_cast<size_t>(row_token(a, t, m)) * H;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int me = min(t.m0 + 16 * i + mfma16_row(lane, e), t.rows - 1);
          ascale[i][e] = a.xs + static_cast<size_t>(row_token(a, t, me)) * ng;
        }
      }
      const uint8_t* brow[CN];
      const float* bscale[CN];
#pragma unroll
      for (int j = 0; j < CNH; ++j) {
        brow[j] = wg + static_cast<size_t>(n0 + 16 * j + r) * H;
        brow[CNH + j] = wu + static_cast<size_t>(n0 + 16 * j + r) * H;
        bscale[j] = sg + static_cast<size_t>(n0 + 16 * j + mfma16_col(lane)) * ng;
        bscale[CNH + j] = su + static_cast<size_t>(n0 + 16 * j + mfma16_col(lane)) * ng;
      }
      wave_mma_fp8<RM, CN>(arow, ascale, brow, bscale, kb, ke, g, acc);
    }

#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < CN; ++j) red[wave][i][j][lane] = acc[i][j];
    __syncthreads();
    for (int p = wave; p < RM * CNH; p += NWK) {
      const int i = p / CNH, jh = p % CNH;
      f32x4 gs = red[0][i][jh][lane], us = red[0][i][CNH + jh][lane];
#pragma unroll
      for (int w = 1; w < NWK; ++w) {
        const f32x4 go = red[w][i][jh][lane], uo = red[w][i][CNH + jh][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) { gs[e] += go[e]; us[e] += uo[e]; }
      }
      const int col = n0 + 16 * jh + mfma16_col(lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = t.m0 + 16 * i + mfma16_row(lane, e);
        if (m < t.rows) {
          const float hv = silu_f32(gs[e]) * us[e];
          const size_t idx = t.shared ? a.h_shared + static_cast<size_t>(m) * width + col
                                      : static_cast<size_t>(t.rowbase + m) * width + col;
          if constexpr (FP8) static_cast<float*>(a.h)[idx] = hv;
          else static_cast<uint16_t*>(a.h)[idx] = f32_to_bf16_bits(hv);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- down + combine (MFMA)

// Tile: BM = 16*RM rows x 16*CN hidden columns, NWK waves splitting the
// intermediate dimension.  The summed tile is staged in LDS and each wave then
// adds whole row segments of y with float32 atomics.
template <int RM, int CN, int NWK, bool FP8>
__global__ void __launch_bounds__(64 * NWK) down_mfma_kernel(ExpertArgs a) {
  constexpr int BM = 16 * RM, BN = 16 * CN;
  __shared__ int prefix[kMaxExperts + 2];
  __shared__ f32x4 red[NWK][RM][CN][kWave];
  __shared__ float out[BM][BN + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;

  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int H = a.H;
  const int total = build_tile_prefix(prefix, a.counts, a.E, a.T, has_shared, BM, H / BN,
                                      has_shared ? H / BN : 0);

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const TileInfo t = find_tile(prefix, G, tile, a, BM);
    const int kdim = t.shared ? a.S : a.I;
    const int n0 = t.nt * BN;
    const int nch = kdim / 128;
    const int kb = (wave * nch) / NWK, ke = ((wave + 1) * nch) / NWK;
    f32x4 acc[RM][CN];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < CN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Row m of the tile lives at h row (rowbase + m) of the routed region, or row m
    // of the shared region.
    auto hrow = [&](int m) -> size_t {
      return t.shared ? a.h_shared + static_cast<size_t>(m) * kdim
                      : static_cast<size_t>(t.rowbase + m) * kdim;
    };
    if constexpr (!FP8) {
      const uint16_t* hb = static_cast<const uint16_t*>(a.h);
      const uint16_t* wd = static_cast<const uint16_t*>(t.shared ? a.ws_down : a.w_down);
      if (!t.shared) wd += static_cast<size_t>(t.group) * H * a.I;
      const uint16_t* arow[RM];
#pragma unroll
      for (int i = 0; i < RM; ++i) arow[i] = hb + hrow(min(t.m0 + 16 * i + r, t.rows - 1));
      const uint16_t* brow[CN];
#pragma unroll
      for (int j = 0; j < CN; ++j) brow[j] = wd + static_cast<size_t>(n0 + 16 * j + r) * kdim;
      wave_mma_bf16<RM, CN>(arow, brow, kb, ke, g, acc);
    } else {
      const int ng = kdim / kGroup;
      const uint8_t* wd = static_cast<const uint8_t*>(t.shared ? a.ws_down : a.w_down);
      const float* sd = t.shared ? a.ss_down : a.s_down;
      if (!t.shared) {
        wd += static_cast<size_t>(t.group) * H * a.I;
        sd += static_cast<size_t>(t.group) * H * ng;
      }
      const uint8_t* arow[RM];
      const float* ascale[RM][4];
#pragma unroll
      for (int i = 0; i < RM; ++i) {
        arow[i] = a.hq + hrow(min(t.m0 + 16 * i + r, t.rows - 1));
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ascale[i][e] = a.hs + hrow(min(t.m0 + 16 * i + mfma16_row(lane, e), t.rows - 1)) / kGroup;
      }
      const uint8_t* brow[CN];
      const float* bscale[CN];
#pragma unroll
      for (int j = 0; j < CN; ++j) {
        brow[j] = wd + static_cast<size_t>(n0 + 16 * j + r) * kdim;
        bscale[j] = sd + static_cast<size_t>(n0 + 16 * j + mfma16_col(lane)) * ng;
      }
      wave_mma_fp8<RM, CN>(arow, ascale, brow, bscale, kb, ke, g, acc);
    }

#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < CN; ++j) red[wave][i][j][lane] = acc[i][j];
    __syncthreads();
    for (int p = wave; p < RM * CN; p += NWK) {
      const int i = p / CN, j = p % CN;
      f32x4 s = red[0][i][j][lane];
#pragma unroll
      for (int w = 1; w < NWK; ++w) {
        const f32x4 o = red[w][i][j][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += o[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) out[16 * i + mfma16_row(lane, e)][16 * j + mfma16_col(lane)] = s[e];
    }
    __syncthreads();
    // Weighted combine, one 16*CN-column row segment per wave instruction.
    for (int q = wave; q < BM; q += NWK) {
      const int m = t.m0 + q;
      if (m >= t.rows) break;
      int tok;
      float wgt;
      if (t.shared) {
        tok = m;
        wgt = a.shared_gate[m];
      } else {
        const int slot = a.perm[t.rowbase + m];
        tok = slot / a.K;
        wgt = a.topk_w[slot];
      }
      float* yr = a.y + static_cast<size_t>(tok) * H + n0;
      for (int c = lane; c < BN; c += kWave) atomicAdd(yr + c, wgt * out[q][c]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- float32 experts (FMA)

// Tile of 16 rows x 16 columns, one output per thread of a 256-thread block.
__global__ void __launch_bounds__(256) gate_up_f32_kernel(ExpertArgs a) {
  __shared__ int prefix[kMaxExperts + 2];
  zero_output(a);
  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int total = build_tile_prefix(prefix, a.counts, a.E, a.T, has_shared, 16, (a.I + 15) / 16,
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
  __shared__ int prefix[kMaxExperts + 2];
  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int H = a.H;
  const int total = build_tile_prefix(prefix, a.counts, a.E, a.T, has_shared, 16, (H + 15) / 16,
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
    int tok;
    float wgt;
    if (t.shared) { tok = m; wgt = a.shared_gate[m]; }
    else { const int slot = a.perm[t.rowbase + m]; tok = slot / a.K; wgt = a.topk_w[slot]; }
    atomicAdd(a.y + static_cast<size_t>(tok) * H + col, wgt * s);
  }
}

// ---------------------------------------------------------------- fp8 activation quantiser

// Per row and per 128-element group: amax, s = amax / 448 (1 if amax = 0),
// q = e4m3(RNE(clamp(v / s, +-448))).  32 lanes (half a wave) per group, four
// elements per lane.  Rows [0, rows_host) of src, or [0, *rows_dev) if rows_dev.
template <bool SRC_BF16>
__global__ void __launch_bounds__(256) quant_g128_kernel(const void* __restrict__ src, int rows_host,
                                                         const int32_t* __restrict__ rows_dev, int cols,
                                                         uint8_t* __restrict__ q, float* __restrict__ s) {
  const int rows = rows_dev ? *rows_dev : rows_host;
  const int ng = cols / kGroup;
  const size_t items = static_cast<size_t>(rows) * ng;
  const int half = threadIdx.x >> 5, hl = threadIdx.x & 31;
  for (size_t it = static_cast<size_t>(blockIdx.x) * 8 + half; it < items;
       it += static_cast<size_t>(gridDim.x) * 8) {
    const size_t base = it * kGroup + 4 * hl;  // rows are contiguous: (row, group) -> it*128
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
    if (hl == 0) s[it] = sc;
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

// Rows per expert decide the kernel: the average expert sees rho = T*K/E rows
// (the same load measure as the small-M / large-M family choice of
// [DeepGEMM fork PR #5, "Dynamic family selection"]).  Up to 16 rows: 16-row
// streaming tiles; up to kTiledRows: 32-row streaming tiles; above: LDS-tiled
// MFMA kernels, 128-row tiles, and 256-row tiles from kTallRows.
constexpr int64_t kTiledRows = 48, kTallRows = 160;

int64_t rows_per_expert(const ExpertArgs& a) { return static_cast<int64_t>(a.T) * a.K / a.E; }
bool tall_tiles(const ExpertArgs& a) { return static_cast<int64_t>(a.T) * a.K > 16LL * a.E; }

}  // namespace

hipError_t launch_gate_up(const ExpertArgs& a, int weight_dtype, hipStream_t stream) {
  if (weight_dtype == kDtypeF32) {
    const int grid = tile_bound(a, 16, (a.I + 15) / 16, (a.S + 15) / 16);
    gate_up_f32_kernel<<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
  }
  const bool fp8 = weight_dtype == kDtypeFp8;
  const int64_t rho = rows_per_expert(a);
  if (rho >= kTiledRows) return launch_gate_up_tiled(a, fp8, rho >= kTallRows, stream);
  if (tall_tiles(a)) {
    const int grid = tile_bound(a, 32, a.I / 32, a.S / 32);
    if (fp8) gate_up_mfma_kernel<2, 2, 4, true><<<grid, 256, 0, stream>>>(a);
    else gate_up_mfma_kernel<2, 2, 4, false><<<grid, 256, 0, stream>>>(a);
  } else {
    const int grid = tile_bound(a, 16, a.I / 32, a.S / 32);
    if (fp8) gate_up_mfma_kernel<1, 2, 4, true><<<grid, 256, 0, stream>>>(a);
    else gate_up_mfma_kernel<1, 2, 4, false><<<grid, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_down(const ExpertArgs& a, int weight_dtype, hipStream_t stream) {
  if (weight_dtype == kDtypeF32) {
    const int grid = tile_bound(a, 16, (a.H + 15) / 16, (a.H + 15) / 16);
    down_f32_kernel<<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
  }
  const bool fp8 = weight_dtype == kDtypeFp8;
  const int64_t rho = rows_per_expert(a);
  if (rho >= kTiledRows && a.H % 256 == 0) return launch_down_tiled(a, fp8, rho >= kTallRows, stream);
  if (tall_tiles(a)) {
    const int grid = tile_bound(a, 32, a.H / 64, a.H / 64);
    if (fp8) down_mfma_kernel<2, 4, 4, true><<<grid, 256, 0, stream>>>(a);
    else down_mfma_kernel<2, 4, 4, false><<<grid, 256, 0, stream>>>(a);
  } else {
    const int grid = tile_bound(a, 16, a.H / 64, a.H / 64);
    if (fp8) down_mfma_kernel<1, 4, 4, true><<<grid, 256, 0, stream>>>(a);
    else down_mfma_kernel<1, 4, 4, false><<<grid, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_quant_x(const ExpertArgs& a, uint8_t* xq, float* xs, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(a.T) * (a.H / kGroup);
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ceil_div(items, 8), 4096)));
  quant_g128_kernel<true><<<grid, 256, 0, stream>>>(a.x, a.T, nullptr, a.H, xq, xs);
  return hipGetLastError();
}

hipError_t launch_quant_h(const ExpertArgs& a, uint8_t* hq, float* hs, hipStream_t stream) {
  // Routed rows: as many as the dispatch kept (read on the device from offsets[E]).
  const int64_t items = static_cast<int64_t>(a.T) * a.K * (a.I / kGroup);
  int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ceil_div(items, 8), 4096)));
  quant_g128_kernel<false><<<grid, 256, 0, stream>>>(a.h, 0, a.offsets + a.E, a.I, hq, hs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.S == 0) return err;
  const int64_t items_s = static_cast<int64_t>(a.T) * (a.S / kGroup);
  grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ceil_div(items_s, 8), 4096)));
  quant_g128_kernel<false><<<grid, 256, 0, stream>>>(static_cast<const float*>(a.h) + a.h_shared, a.T,
                                                     nullptr, a.S, hq + a.h_shared,
                                                     hs + a.h_shared / kGroup);
  return hipGetLastError();
}

}  // namespace moe
