// Weight-streaming grouped expert GEMMs: decode-sized M (few rows per expert) and,
// with 128-row tiles, the middle range up to the 256-row LDS-tiled kernels.
//
// At decode sizes every routed expert sees a handful of tokens, so the layer is
// bound by reading each touched expert's weights once from HBM [SpecForge PR
// #943, "Motivation": each draft step streams the touched experts' weights].
// The kernel is built around keeping enough of that stream in flight:
//
//   * a tile is BN weight rows of one group (routed expert or shared expert)
//     against BM rows of tokens; the contraction runs in stages that give every
//     row 256 contiguous bytes where the contraction allows: 128 elements of
//     bf16, 256 of fp8 (two 128-groups; one group, 128 bytes, when a contraction
//     is not a multiple of 256), 512 of MXFP4 weights (256 bytes of codes per
//     weight row, 512 per MXFP8 activation row; 256 elements when a contraction
//     is not a multiple of 512).  Per workgroup, 256-byte row pieces load ~40 %
//     more bytes per clock than 128-byte ones (measured); larger ones gain
//     nothing;
//   * a workgroup is 8 waves with two roles.  Four loader waves only load: they
//     keep NS stages in flight in registers and write one stage per step into a
//     double-buffered LDS stage.  Four compute waves read the other LDS buffer,
//     run the MFMAs (16x16x32 bf16; 16x16x128 fp8 with the row and column group
//     scales applied to each group's partial sum in float32; the block-scaled
//     16x16x128 fp8 x fp4 MFMA for MXFP4, which applies the E8M0 scales itself)
//     and write the results.  One barrier per stage hands the buffers over;
//   * the split keeps the loaders' wait counts exact: a wave's vector-memory
//     counter covers its loads and its stores alike, and the compiler waits for
//     everything once a store is pending, so a wave that also wrote results would
//     drain its whole stream at every tile.  Loaders therefore never store to
//     global memory, and every load they issue is unconditional: rows outside the
//     group are read through a buffer descriptor at an offset past its end (zeros),
//     the stages past the workgroup's last one re-read that stage, and the dispatch
//     rows of a tile are fetched a whole tile before their first use;
//   * one workgroup per CU, 256 VGPRs per lane: the loaders hold NS = 2..6
//     stages (~100-150 KB per CU in flight); measured, deeper staging no longer
//     moves the rate: a CU keeps ~11 KB of loads outstanding, so its rate is
//     that over the latency (~10 B/clk from HBM, more from L2), and the
//     remaining lever is fewer bytes per tile;
//   * tiles are spread by their cost in stages (see balanced_walk);
//   * gate/up tiles fuse SwiGLU and write h; down tiles write each routed slot's
//     output row (unweighted) and the shared expert's rows (weighted by sigmoid(g)).
#include "kernels.h"
#include "schedule.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kLoadWaves = 4;
constexpr int kComputeWaves = 4;
constexpr int kLoadThreads = kLoadWaves * kWave;
constexpr int kStreamThreads = (kLoadWaves + kComputeWaves) * kWave;
constexpr int kXcdCount = 8;   // the tile walk assumes grids that are multiples of 8
// A-buffer offset that marks a row outside its group: every A buffer is smaller
// (the host limits x and h to 3 GiB), so such loads return zeros.
constexpr uint32_t kDeadRow = 0xC0000000u;

// LDS rows of a stage are stored unpadded, with the 16-byte pieces of a row
// permuted so that both the loaders' 16-byte stores (16 lanes: one row's
// consecutive pieces, or two 128-byte rows) and the MFMA fragment reads (16 lanes:
// one piece of 16 consecutive rows) touch every bank once per 16 lanes.  A 256- or
// 512-byte row keeps piece p at p ^ (row mod 16) (the low four bits; a row starts
// at bank 0); a 128-byte row (two per 256-byte bank line) at p ^ ((row / 2) mod 8).
// Byte offset of piece p of row `row` in rows of RB bytes.
template <int RB>
__device__ __forceinline__ int lds_at(int row, int p) {
  static_assert(RB == 128 || RB == 256 || RB == 512, "row size");
  const int q = RB == 128 ? (p ^ ((row >> 1) & 7)) : (p ^ (row & 15));
  return row * RB + 16 * q;
}

// GateUp: h = SwiGLU(x W_gate^T, x W_up^T); Down: o / y = h W_down^T; Router: the
// router logits z = x [W_r; w_g]^T over all T tokens (one group of T rows).
enum class SMode { GateUp, Down, Router };

// FMT is the weight format: kDtypeBf16; kDtypeFp8 (e4m3 codes, float32 scale per
// row and 128-group, activations quantised the same way) in stages of one group,
// or kFp8Wide, the same in stages of two groups (contractions that are multiples
// of 256), or kFp8Quad, in stages of four groups (multiples of 512: one 16-byte
// scale load per row per stage instead of two 8-byte ones); kDtypeMxfp4 (E2M1 codes two per byte, E8M0 scale per 32 elements,
// activations MXFP8) in stages of 256 elements, or kMxWide, the same in stages of
// 512 (contractions that are multiples of 512).
constexpr int kFp8Wide = 0x12;
constexpr int kMxWide = 0x13;
constexpr int kFp8Quad = 0x14;

template <SMode MODE, int BM, int BN, int WM, int FMT>
struct StreamCfg {
  static constexpr bool kQ = FMT != kDtypeBf16;                // 8-bit activation codes + scales
  static constexpr bool kMX = FMT == kDtypeMxfp4 || FMT == kMxWide;
  static constexpr bool kWide = kMX || FMT == kFp8Wide || FMT == kFp8Quad;   // 8-bit A in stages of >= 256
  static constexpr int kWM = WM;                               // compute waves along rows
  static constexpr int kWN = kComputeWaves / WM;               // compute waves along weight rows
  // Contraction elements per stage: 128 (one bf16 row slice of 256 bytes, or one fp8
  // 128-group), 256 for wide fp8 and for MX (a weight row gives 128 contiguous
  // bytes): 256-byte pieces load faster per byte than 128-byte ones.
  static constexpr int kElems = (FMT == kMxWide || FMT == kFp8Quad) ? 512 : kWide ? 256 : 128;
  static constexpr int kRowDataA = kQ ? kElems : 256;          // A bytes per row per stage
  static constexpr int kRowDataB = kMX ? kElems / 2 : kRowDataA;   // B bytes per row per stage
  static constexpr int kSub = kQ ? kElems / 128 : 4;           // MFMA k-steps per stage
  static constexpr int kRowStrideA = kRowDataA;                // unpadded LDS rows, pieces swizzled
  static constexpr int kRowStrideB = kRowDataB;
  static constexpr int kLanesPerRowA = kRowDataA / 16;
  static constexpr int kLanesPerRowB = kRowDataB / 16;
  static constexpr int kRowsPerPassA = kLoadThreads / kLanesPerRowA;
  static constexpr int kRowsPerPassB = kLoadThreads / kLanesPerRowB;
  static constexpr int kAPasses = (BM + kRowsPerPassA - 1) / kRowsPerPassA;
  static constexpr int kBPasses = BN / kRowsPerPassB;
  static constexpr int kRM = BM / WM / 16;                     // row blocks per compute wave
  static constexpr int kCB = BN / kWN / 16;                    // column blocks per compute wave
  static constexpr int kBOff = BM * kRowStrideA;               // B rows inside a stage buffer
  static constexpr int kSlot = kBOff + BN * kRowStrideB;       // one LDS stage buffer
  static constexpr int kScales = BM + BN;                      // one scale word per row (below)
  // Scale word of a row per stage: the fp8 float32 group scale (two of them for
  // wide fp8, four in quad stages), or the MX row's E8M0 bytes (one per 32
  // elements: 8 or 16).
  using ScaleWord = std::conditional_t<FMT == kMxWide || FMT == kFp8Quad, uint4,
                                       std::conditional_t<kWide, uint2, uint32_t>>;
  static_assert(BN % kRowsPerPassB == 0, "BN must be a multiple of the rows per pass");
  static_assert(MODE == SMode::Down || kCB % 2 == 0, "gate/up needs gate and up blocks");
  static_assert(kRM >= 1 && BM % (16 * WM) == 0, "rows per wave must be a multiple of 16");
  // Scale words a loader thread stages per stage: rows tid and tid + 256 (the
  // activation rows first, then the weight rows).
  static constexpr int kScaleWords = (BM + BN + kLoadThreads - 1) / kLoadThreads;
  static_assert(!kQ || (BM <= kLoadThreads && kScaleWords <= 2), "at most two scale rows per loader thread");
};

// Register stages a loader keeps in flight: as many as fit ~160 VGPRs (more make
// the register allocator copy in-flight load destinations, which forces waits).
constexpr int stream_stages(int pieces_per_stage) {
  const int n = 160 / (4 * pieces_per_stage);
  return n < 2 ? 2 : (n > 6 ? 6 : n);
}

// Weight row of the LDS B tile read by column block j of the compute wave in
// weight-row column wn of kWN (lane row r).  Gate/up tiles hold BN/2 gate rows then
// the BN/2 up rows of the same intermediate columns; wave column wn takes the gate
// and up rows of columns [wn*BN/(2*kWN), (wn+1)*BN/(2*kWN)).
template <SMode MODE, int BN, int kWN, int kCB>
__device__ __forceinline__ int stream_b_row(int wn, int j, int r) {
  if constexpr (MODE == SMode::GateUp) {
    const int half = kCB / 2;
    const int jh = (j < half) ? j : j - half;
    return ((j < half) ? 0 : BN / 2) + wn * (BN / (2 * kWN)) + 16 * jh + r;
  } else {
    return wn * (BN / kWN) + 16 * j + r;
  }
}

// Calls f(integral_constant<J>) for J = 0..N-1 in order while it returns true.
template <int J, int N>
struct Unrolled {
  template <class F>
  __device__ __forceinline__ static bool run(F& f) {
    if (!f(std::integral_constant<int, J>{})) return false;
    return Unrolled<J + 1, N>::run(f);
  }
};
template <int N>
struct Unrolled<N, N> {
  template <class F>
  __device__ __forceinline__ static bool run(F&) { return true; }
};

// The tiles a workgroup runs: [tile, end) in steps of `step`.
struct Walk {
  int tile, end, step;
};

// Cost-balanced walk over the tiles of a grouped launch.  A tile costs its number
// of stages: measured per workgroup, a stage takes about the same time whatever
// the tile's row count (the token rows come from L2 next to the weight stream).
// Each XCD (workgroup b runs on XCD b % 8) takes the contiguous run of tiles whose
// start cost falls in its eighth of the total, and its workgroups stride through
// that run, so the m-tiles of a weight slab (neighbours in the tile order) run at
// the same time on one XCD and share its L2.  Cutting by tile count instead would
// hand the shared expert's longer down tiles (contraction S instead of I) to the
// last XCDs only.
// cpre (G + 1 entries of CostT) receives the cost prefix; a group's tile cost is
// nk_routed or nk_shared stages.
template <typename CostT>
__device__ Walk balanced_walk(const int* sched, CostT* cpre, int G, int E, int nk_routed, int nk_shared) {
  const int* prefix = sched;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    long long carry = 0;
    for (int base = 0; base < G; base += kWave) {
      const int g = base + lane;
      long long v = 0;
      if (g < G) {
        const int c = (g < E) ? nk_routed : nk_shared;
        v = static_cast<long long>(c) * (prefix[g + 1] - prefix[g]);
      }
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const long long n = __shfl_up(v, o, kWave);
        if (lane >= o) v += n;
      }
      if (g < G) cpre[g + 1] = static_cast<CostT>(carry + v);
      carry += __shfl(v, kWave - 1, kWave);
    }
    if (lane == 0) cpre[0] = 0;
  }
  __syncthreads();
  const int total = prefix[G];
  const long long ctot = static_cast<long long>(cpre[G]);
  // First tile whose start cost is >= c.  The last group g with cpre[g] <= c < ctot
  // holds tiles (cpre[g + 1] > c), so the quotient stays inside it or at its end.
  auto first_at = [&](long long c) -> int {
    if (c >= ctot) return total;
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (static_cast<long long>(cpre[mid]) <= c) lo = mid; else hi = mid;
    }
    const long long off = c - static_cast<long long>(cpre[lo]);
    const int cost = (lo < E) ? nk_routed : nk_shared;
    return prefix[lo] + static_cast<int>((off + cost - 1) / cost);
  };
  const int xcd = blockIdx.x % 8;
  const int begin = first_at(ctot * xcd / 8);
  return Walk{begin + static_cast<int>(blockIdx.x / 8), first_at(ctot * (xcd + 1) / 8),
              static_cast<int>(gridDim.x / 8)};
}

template <SMode MODE, int BM, int BN, int WM, int FMT, int NS>
__global__ void __launch_bounds__(kStreamThreads, 1) stream_expert_kernel(ExpertArgs a) {
  using C = StreamCfg<MODE, BM, BN, WM, FMT>;
  constexpr bool FP8 = C::kQ;    // quantised: 8-bit activation codes with scales
  constexpr bool MX = C::kMX;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::kSlot];
  // Per stage and row: the fp8 float32 scale (as bits), or the MX row's eight E8M0
  // bytes for the stage's eight 32-element blocks.
  using SW = typename C::ScaleWord;
  __shared__ __attribute__((aligned(16))) SW sscale[FP8 ? 2 * C::kScales : 1];
  __shared__ int sched[kSchedInts];
  // Cost prefix of the tile walk.  32-bit in the four-group fp8 kernels, whose
  // 16 x 128 tile needs the LDS; their launcher checks that the costs fit.
  using CostT = std::conditional_t<FMT == kFp8Quad, int, long long>;
  __shared__ CostT cpre[kSchedStride];

  const int tid = threadIdx.x;
  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int H = a.H;
  const int bn_cols = (MODE == SMode::GateUp) ? BN / 2 : BN;
  // Contraction parts per (group, m-tile, n-tile) of a gate/up or router launch:
  // tile index n' = P n + p covers n-tile n over the p-th 1/P of the contraction.
  const int P = (MODE != SMode::Down) ? max(1, a.kparts) : 1;
  const size_t esz = FP8 ? 1 : 2;   // bytes per A (activation) element
  // Bytes of one weight row of `k` elements.
  auto b_row_bytes = [&](int k) -> size_t { return MX ? static_cast<size_t>(k) / 2 : static_cast<size_t>(k) * esz; };
  Walk walk;
  if constexpr (MODE == SMode::Router) {
    // Equal tiles: an equal run per XCD, strided by its workgroups.
    const int total = static_cast<int>(ceil_div(a.T, BM) * ceil_div(a.ncols, BN)) * P;
    const int xcd = blockIdx.x % 8;
    walk = Walk{total * xcd / 8 + static_cast<int>(blockIdx.x / 8), total * (xcd + 1) / 8,
                static_cast<int>(gridDim.x / 8)};
  } else {
    const int nt_r = ((MODE == SMode::GateUp) ? a.I / bn_cols : H / bn_cols) * P;
    const int nt_s = has_shared ? ((MODE == SMode::GateUp) ? a.S / bn_cols : H / bn_cols) * P : 0;
    // n-tiles per group of the 128 x 128 launch that serves split 3 (same value in
    // the split-4 launch, whatever its own tile width).
    const int mid_nt = (MODE == SMode::GateUp) ? a.I / 64 : H / 128;
    build_tile_prefix(sched, a.counts, a.offsets, a.E, a.T, has_shared, BM, nt_r, nt_s, a.split, mid_nt);
    const int nk_r = ((MODE == SMode::GateUp) ? H : a.I) / C::kElems / P;
    const int nk_s = ((MODE == SMode::GateUp) ? H : a.S) / C::kElems / P;
    walk = balanced_walk<CostT>(sched, cpre, G, a.E, nk_r, nk_s);
  }
  if (walk.tile >= walk.end) return;   // uniform across the workgroup

  // ---- tile geometry
  struct Tile {
    TileInfo t;
    int kdim, nk, n0;
    int part, kb;   // contraction part and its first stage
  };
  // gc: the caller's group cursor (a group at or before the tile's; tiles only move
  // forward, so each role keeps one and the lookup scans forward from it).
  auto make_tile = [&](int tile, int& gc) {
    Tile d;
    if constexpr (MODE == SMode::Router) {
      // One group of T rows read straight from x (the shared-expert row rule).
      const int mt = static_cast<int>(ceil_div(a.T, BM));
      d.t.group = 0;
      d.t.shared = true;
      d.t.rows = a.T;
      d.t.rowbase = 0;
      d.t.m0 = (tile % mt) * BM;
      d.t.nt = tile / mt;
    } else {
      gc = advance_group(sched, G, tile, gc);
      d.t = tile_in_group(sched, gc, tile, a, BM);
    }
    d.kdim = (MODE != SMode::Down) ? H : (d.t.shared ? a.S : a.I);
    d.part = d.t.nt % P;
    d.t.nt /= P;
    d.nk = d.kdim / C::kElems / P;
    d.kb = d.part * d.nk;
    d.n0 = d.t.nt * bn_cols;
    return d;
  };
  auto hrow = [&](const Tile& d, int m) -> size_t {   // element offset of row m in h / hq
    return d.t.shared ? a.h_shared + static_cast<size_t>(m) * d.kdim
                      : static_cast<size_t>(d.t.rowbase + m) * d.kdim;
  };

  // Both roles pass one barrier per stage of the workgroup's tiles.  Every routed
  // tile has the same stage count, and so does every shared-expert tile (the tiles
  // from prefix[E] on), so the total needs only the number of the walk's tiles in
  // that tail.
  const int last = walk.tile + (walk.end - 1 - walk.tile) / walk.step * walk.step;
  const int ntiles = (last - walk.tile) / walk.step + 1;
  int nstages = ntiles * (H / C::kElems / P);
  if constexpr (MODE != SMode::Router) {
    const int nk_r = ((MODE == SMode::GateUp) ? H : a.I) / C::kElems / P;
    const int nk_s = ((MODE == SMode::GateUp) ? H : a.S) / C::kElems / P;
    const int first_shared = has_shared ? sched[a.E] : walk.end;
    const int skip = first_shared <= walk.tile ? 0 : (first_shared - walk.tile + walk.step - 1) / walk.step;
    const int n_shared = max(0, ntiles - skip);
    nstages = (ntiles - n_shared) * nk_r + n_shared * nk_s;
  }

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave < kLoadWaves) {
    // ================================================================ loaders
    const int lrow = tid / C::kLanesPerRowA;           // A row inside a load pass
    const int lcol = (tid % C::kLanesPerRowA) * 16;    // byte offset inside the A stage slice
    const int lrowb = tid / C::kLanesPerRowB;          // the same for B
    const int lcolb = (tid % C::kLanesPerRowB) * 16;
    const uint8_t* abase;
    size_t aelems;
    if constexpr (MODE != SMode::Down) {
      abase = FP8 ? a.xq : static_cast<const uint8_t*>(a.x);
      aelems = static_cast<size_t>(a.T) * H;
    } else {
      abase = FP8 ? a.hq : static_cast<const uint8_t*>(a.h);
      aelems = a.h_shared + static_cast<size_t>(a.T) * a.S;
    }
    const __amdgpu_buffer_rsrc_t arsrc = buf_rsrc(abase, static_cast<uint32_t>(aelems * esz));

    // Dispatch entries behind a tile's A rows (and the fp8 scale row of thread
    // tid < BM), loaded unconditionally; only read a tile later.
    struct Pend {
      int pv[C::kAPasses];
      int ps;
    };
    auto fetch = [&](const Tile& d) {
      Pend p;
      const TileInfo& t = d.t;
#pragma unroll
      for (int q = 0; q < C::kAPasses; ++q) p.pv[q] = 0;
      p.ps = 0;
      if constexpr (MODE == SMode::GateUp) {
        const int base = t.shared ? 0 : t.rowbase;
#pragma unroll
        for (int q = 0; q < C::kAPasses; ++q) {
          const int mc = min(t.m0 + lrow + q * C::kRowsPerPassA, t.rows - 1);
          p.pv[q] = t.shared ? a.perm[base + mc] : slot_clamp(a.perm[base + mc], a);
        }
        if constexpr (FP8) p.ps = slot_clamp(a.perm[base + min(t.m0 + min(tid, BM - 1), t.rows - 1)], a);
      }
      return p;
    };
    // A row offsets and this thread's scale row of a tile (bytes; the stage's
    // scale word is at sizeof(SW) * stage).
    struct Src {
      uint32_t a[C::kAPasses];
      const uint8_t* s[C::kScaleWords];
    };
    auto resolve = [&](const Tile& d, const Pend& p) {
      Src S;
      const TileInfo& t = d.t;
#pragma unroll
      for (int q = 0; q < C::kAPasses; ++q) {
        const int row = lrow + q * C::kRowsPerPassA;
        const int m = t.m0 + row;
        const int mc = min(m, t.rows - 1);
        uint32_t off;
        if constexpr (MODE == SMode::Down) {
          off = static_cast<uint32_t>(hrow(d, mc) * esz);
        } else {
          const int tok = t.shared ? mc : p.pv[q] / a.K;
          off = static_cast<uint32_t>(tok) * static_cast<uint32_t>(H) * static_cast<uint32_t>(esz);
        }
        S.a[q] = (row < BM && m < t.rows) ? off : kDeadRow;
      }
#pragma unroll
      for (int w = 0; w < C::kScaleWords; ++w) S.s[w] = nullptr;
      if constexpr (FP8) {
        // Thread tid < BM stages the scale word of tile row tid, BM <= tid < BM+BN
        // that of B row tid-BM; the other threads re-read B row 0's (never stored).
        // fp8: ng float32 scales per row (one per 128); MX: K/32 E8M0 bytes per row.
        const int ng = d.kdim / kGroup;
        const size_t srow = MX ? static_cast<size_t>(d.kdim / kMxBlock) : static_cast<size_t>(ng) * 4;
        const uint8_t* sw0;
        const uint8_t* sw1 = nullptr;
        auto wscale = [&](const float* fs, const uint8_t* ms) {
          return MX ? ms : reinterpret_cast<const uint8_t*>(fs);
        };
        if constexpr (MODE == SMode::GateUp) {
          sw0 = t.shared ? wscale(a.ss_gate, a.e8s_gate)
                         : wscale(a.s_gate, a.e8_gate) + static_cast<size_t>(t.group) * a.I * srow;
          sw1 = t.shared ? wscale(a.ss_up, a.e8s_up)
                         : wscale(a.s_up, a.e8_up) + static_cast<size_t>(t.group) * a.I * srow;
        } else {
          sw0 = t.shared ? wscale(a.ss_down, a.e8s_down)
                         : wscale(a.s_down, a.e8_down) + static_cast<size_t>(t.group) * H * srow;
        }
        // Scale row tid + 256 w: activation rows [0, BM) (only in word 0, BM <= 256),
        // then weight rows; rows past BM + BN re-read weight row 0 (never stored).
#pragma unroll
        for (int w = 0; w < C::kScaleWords; ++w) {
          const int r = tid + kLoadThreads * w;
          if (w == 0 && tid < BM) {
            const int mc = min(t.m0 + tid, t.rows - 1);
            if constexpr (MODE == SMode::GateUp) {
              const int tok = t.shared ? mc : p.ps / a.K;
              S.s[w] = (MX ? a.xe8 : reinterpret_cast<const uint8_t*>(a.xs)) + static_cast<size_t>(tok) * srow;
            } else {
              // Element offset of the row in h, in scale units (one per 32 or per 128).
              S.s[w] = MX ? a.he8 + hrow(d, mc) / kMxBlock
                          : reinterpret_cast<const uint8_t*>(a.hs + hrow(d, mc) / kGroup);
            }
          } else {
            const int br = (r < BM + BN) ? r - BM : 0;
            if constexpr (MODE == SMode::GateUp)
              S.s[w] = (br < BN / 2) ? sw0 + static_cast<size_t>(d.n0 + br) * srow
                                     : sw1 + static_cast<size_t>(d.n0 + br - BN / 2) * srow;
            else
              S.s[w] = sw0 + static_cast<size_t>(d.n0 + br) * srow;
          }
        }
      }
      return S;
    };
    // Weight-row pointers of a tile (arithmetic only).
    struct BPtr {
      const uint8_t* b[C::kBPasses];
    };
    auto make_b = [&](const Tile& d) {
      BPtr P;
      const TileInfo& t = d.t;
      const uint8_t* w0;
      const uint8_t* w1 = nullptr;
      const size_t rb = b_row_bytes(d.kdim);
      if constexpr (MODE == SMode::GateUp) {
        w0 = static_cast<const uint8_t*>(t.shared ? a.ws_gate : a.w_gate);
        w1 = static_cast<const uint8_t*>(t.shared ? a.ws_up : a.w_up);
        if (!t.shared) {
          w0 += static_cast<size_t>(t.group) * a.I * rb;
          w1 += static_cast<size_t>(t.group) * a.I * rb;
        }
      } else if constexpr (MODE == SMode::Router) {
        w0 = static_cast<const uint8_t*>(a.w_router);
      } else {
        w0 = static_cast<const uint8_t*>(t.shared ? a.ws_down : a.w_down);
        if (!t.shared) w0 += static_cast<size_t>(t.group) * H * rb;
      }
#pragma unroll
      for (int q = 0; q < C::kBPasses; ++q) {
        const int br = lrowb + q * C::kRowsPerPassB;
        if constexpr (MODE == SMode::GateUp) {
          P.b[q] = (br < BN / 2) ? w0 + static_cast<size_t>(d.n0 + br) * rb
                                 : w1 + static_cast<size_t>(d.n0 + br - BN / 2) * rb;
        } else if constexpr (MODE == SMode::Router) {
          // Column c < E: router row c; c == E: the shared gate vector; columns past
          // the last one re-read a valid row and are never stored.
          const int c = min(d.n0 + br, a.ncols - 1);
          P.b[q] = (c < a.E) ? w0 + static_cast<size_t>(c) * rb : static_cast<const uint8_t*>(a.w_gcol);
        } else {
          P.b[q] = w0 + static_cast<size_t>(d.n0 + br) * rb;
        }
      }
      return P;
    };

    struct Regs {
      uint4 a[C::kAPasses], b[C::kBPasses];
      SW s[C::kScaleWords];
    };
    auto gload = [&](Regs& R, const BPtr& P, const Src& S, int ks) {
      const uint32_t off = static_cast<uint32_t>(ks) * C::kRowDataA + lcol;
      const uint32_t offb = static_cast<uint32_t>(ks) * C::kRowDataB + lcolb;
#pragma unroll
      for (int q = 0; q < C::kBPasses; ++q) R.b[q] = ld16_stream(P.b[q] + offb);
#pragma unroll
      for (int q = 0; q < C::kAPasses; ++q) R.a[q] = buf_ld16(arsrc, S.a[q] + off, 0);
      if constexpr (FP8) {
#pragma unroll
        for (int w = 0; w < C::kScaleWords; ++w) R.s[w] = *reinterpret_cast<const SW*>(S.s[w] + sizeof(SW) * ks);
      }
    };
    auto lstore = [&](const Regs& R, int slot) {
      uint8_t* base = smem + slot * C::kSlot;
#pragma unroll
      for (int q = 0; q < C::kAPasses; ++q)
        if (lrow + q * C::kRowsPerPassA < BM)
          *reinterpret_cast<uint4*>(base + lds_at<C::kRowStrideA>(lrow + q * C::kRowsPerPassA, lcol / 16)) = R.a[q];
#pragma unroll
      for (int q = 0; q < C::kBPasses; ++q)
        *reinterpret_cast<uint4*>(base + C::kBOff + lds_at<C::kRowStrideB>(lrowb + q * C::kRowsPerPassB, lcolb / 16)) =
            R.b[q];
      if constexpr (FP8) {
#pragma unroll
        for (int w = 0; w < C::kScaleWords; ++w)
          if (tid + kLoadThreads * w < C::kScales) sscale[slot * C::kScales + tid + kLoadThreads * w] = R.s[w];
      }
    };

    // The load cursor: stage ld_ks of tile ld; the next tile's dispatch rows are
    // already being fetched (np).
    int lg = 0;   // group cursor of the look-ahead tile nld
    Tile ld = make_tile(walk.tile, lg);
    Src ls = resolve(ld, fetch(ld));
    BPtr lb = make_b(ld);
    int ld_tile = walk.tile, ld_ks = 0;
    Tile nld = make_tile(min(walk.tile + walk.step, last), lg);
    Pend np = fetch(nld);
    auto issue = [&](Regs& R) {
      gload(R, lb, ls, ld.kb + ld_ks);
      if (ld_ks + 1 < ld.nk) {
        ++ld_ks;
      } else if (ld_tile < last) {
        ld_tile += walk.step;
        ld = nld;
        ls = resolve(ld, np);
        lb = make_b(ld);
        ld_ks = 0;
        nld = make_tile(min(ld_tile + walk.step, last), lg);
        np = fetch(nld);
      }
      // else: past the workgroup's last stage; that stage is loaded again, unused.
    };

    Regs R[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) issue(R[j]);   // stages 0 .. NS-1
    lstore(R[0], 0);                             // stage 0 -> buffer 0
    issue(R[0]);                                 // stage NS
    __syncthreads();
    // Step k: the compute waves read stage k from buffer k&1 while the loaders
    // store stage k+1 (register set (k+1) % NS) into buffer (k+1)&1 and refill that
    // set with stage k+1+NS.
    int k = 0;
    auto step = [&](auto J) {
      constexpr int j = decltype(J)::value;
      lstore(R[(j + 1) % NS], (k + 1) & 1);
      issue(R[(j + 1) % NS]);
      __syncthreads();
      return ++k < nstages;
    };
    while (Unrolled<0, NS>::run(step)) {
    }
  } else {
    // ================================================================ compute
    const int cw = wave - kLoadWaves;
    const int lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int wm = cw / C::kWN, wn = cw % C::kWN;
    const int wrow0 = wm * (BM / WM);   // first tile row of this wave

    f32x4 acc[C::kRM][C::kCB];
    auto clear_acc = [&]() {
#pragma unroll
      for (int i = 0; i < C::kRM; ++i)
#pragma unroll
        for (int j = 0; j < C::kCB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // 16-byte piece p of A row (wrow0 + 16 i + r), or of B row br.
    auto a_ld = [&](const uint8_t* base, int i, int p) {
      return *reinterpret_cast<const uint4*>(base + lds_at<C::kRowStrideA>(wrow0 + 16 * i + r, p));
    };
    auto b_ld = [&](const uint8_t* base, int br, int p) {
      return *reinterpret_cast<const uint4*>(base + C::kBOff + lds_at<C::kRowStrideB>(br, p));
    };
    auto compute = [&](int slot) {
      const uint8_t* base = smem + slot * C::kSlot;
      if constexpr (!FP8) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uint4 af[C::kRM], bf[C::kCB];
#pragma unroll
          for (int i = 0; i < C::kRM; ++i) af[i] = a_ld(base, i, 4 * s + g);
#pragma unroll
          for (int j = 0; j < C::kCB; ++j)
            bf[j] = b_ld(base, stream_b_row<MODE, BN, C::kWN, C::kCB>(wn, j, r), 4 * s + g);
#pragma unroll
          for (int i = 0; i < C::kRM; ++i)
#pragma unroll
            for (int j = 0; j < C::kCB; ++j) acc[i][j] = mfma_bf16_16x16x32(af[i], bf[j], acc[i][j]);
        }
      } else if constexpr (MX) {
        // Two 16x16x128 steps per stage (s = 0, 1: elements [128s, +128)), A = MXFP8
        // codes (8-bit layout: lane group g holds bytes [16g, +16) and [64+16g, +16)
        // of the step's 128 codes) and B = MXFP4 codes (4-bit layout: lane group g
        // holds the 32 codes [32g, +32), bytes [16g, +16) of the step's 64).  The E8M0
        // scale of K-block g of a step (its elements [32g, +32)) for the lane's row
        // comes from lane group g: byte g of the row's scale word s.
        const SW* sc = sscale + slot * C::kScales;
#pragma unroll
        for (int s = 0; s < C::kSub; ++s) {
          i32x8 af[C::kRM], bf[C::kCB];
          int sa[C::kRM], sb[C::kCB];
#pragma unroll
          for (int i = 0; i < C::kRM; ++i) {
            const uint4 lo = a_ld(base, i, 8 * s + g);
            const uint4 hi = a_ld(base, i, 8 * s + 4 + g);
            af[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const uint32_t w = reinterpret_cast<const uint32_t*>(&sc[wrow0 + 16 * i + r])[s];
            sa[i] = static_cast<int>((w >> (8 * g)) & 0xffu);
          }
#pragma unroll
          for (int j = 0; j < C::kCB; ++j) {
            const int br = stream_b_row<MODE, BN, C::kWN, C::kCB>(wn, j, r);
            const uint4 v = b_ld(base, br, 4 * s + g);
            bf[j] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            const uint32_t w = reinterpret_cast<const uint32_t*>(&sc[BM + br])[s];
            sb[j] = static_cast<int>((w >> (8 * g)) & 0xffu);
          }
#pragma unroll
          for (int i = 0; i < C::kRM; ++i)
#pragma unroll
            for (int j = 0; j < C::kCB; ++j)
              acc[i][j] = mfma_mxfp8_mxfp4_16x16x128(af[i], bf[j], acc[i][j], sa[i], sb[j]);
        }
      } else {
        // One 16x16x128 step per 128-group of the stage (two for wide fp8).  Lane
        // group g holds bytes [16g, +16) and [64+16g, +16) of its row's group.  The
        // row scales of the accumulator rows 4g..4g+3 are rescaled in float32 per
        // group.
        constexpr int kSub = C::kSub;
        const float* scf = reinterpret_cast<const float*>(sscale + slot * C::kScales);
#pragma unroll
        for (int s = 0; s < kSub; ++s) {
          i32x8 af[C::kRM], bf[C::kCB];
          f32x4 sa[C::kRM];
          float sb[C::kCB];
#pragma unroll
          for (int i = 0; i < C::kRM; ++i) {
            const uint4 lo = a_ld(base, i, 8 * s + g);
            const uint4 hi = a_ld(base, i, 8 * s + 4 + g);
            af[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const int row = wrow0 + 16 * i + 4 * g;
            if constexpr (kSub == 4) {
              // Four floats per row (groups 0..3 of the stage).
              sa[i] = f32x4{scf[4 * row + s], scf[4 * row + 4 + s], scf[4 * row + 8 + s], scf[4 * row + 12 + s]};
            } else if constexpr (C::kWide) {
              // Two floats per row (groups 0 and 1 of the stage).
              const f32x4 r01 = *reinterpret_cast<const f32x4*>(&scf[2 * row]);
              const f32x4 r23 = *reinterpret_cast<const f32x4*>(&scf[2 * row + 4]);
              sa[i] = s ? f32x4{r01[1], r01[3], r23[1], r23[3]} : f32x4{r01[0], r01[2], r23[0], r23[2]};
            } else {
              sa[i] = *reinterpret_cast<const f32x4*>(&scf[row]);
            }
          }
#pragma unroll
          for (int j = 0; j < C::kCB; ++j) {
            const int br = stream_b_row<MODE, BN, C::kWN, C::kCB>(wn, j, r);
            const uint4 lo = b_ld(base, br, 8 * s + g);
            const uint4 hi = b_ld(base, br, 8 * s + 4 + g);
            bf[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            sb[j] = scf[kSub * (BM + br) + s];
          }
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < C::kRM; ++i)
#pragma unroll
            for (int j = 0; j < C::kCB; ++j) {
              const f32x4 p = mfma_fp8_16x16x128(af[i], bf[j], zero);
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(p[e], sa[i][e] * sb[j], acc[i][j][e]);
            }
        }
      }
    };

    // Down tiles: the destination of each output row this lane writes (tile rows
    // wrow0 + 16i + 4g + e), fetched when the tile starts.  Routed rows go,
    // unweighted, to their slot's row of o; shared rows to y, weighted by sigmoid(g).
    // The loaded values are left untouched until the epilogue: an instruction that
    // used them at once would wait for every older memory operation of the wave,
    // the previous tile's output stores included (one counter covers both).
    int dslot[MODE == SMode::Down ? C::kRM : 1][4];
    float dgate[MODE == SMode::Down ? C::kRM : 1][4];
    auto fetch_dst = [&](const Tile& d) {
      if constexpr (MODE == SMode::Down) {
        const TileInfo& t = d.t;
        const int base = t.shared ? 0 : t.rowbase;
#pragma unroll
        for (int i = 0; i < C::kRM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int mc = min(t.m0 + wrow0 + 16 * i + 4 * g + e, t.rows - 1);
            dslot[i][e] = a.perm[base + mc];
            dgate[i][e] = has_shared ? a.shared_gate[min(mc, a.T - 1)] : 1.0f;
          }
      }
    };

    auto epilogue = [&](const Tile& d) {
      const TileInfo& t = d.t;
      if constexpr (MODE == SMode::Router) {
#pragma unroll
        for (int i = 0; i < C::kRM; ++i)
#pragma unroll
          for (int j = 0; j < C::kCB; ++j) {
            const int col = d.n0 + wn * (BN / C::kWN) + 16 * j + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = t.m0 + wrow0 + 16 * i + 4 * g + e;
              if (m < t.rows && col < a.ncols)
                a.z[static_cast<size_t>(d.part) * a.zplane + static_cast<size_t>(m) * a.ldz + col] = acc[i][j][e];
            }
          }
      } else if constexpr (MODE == SMode::GateUp) {
        const int width = t.shared ? a.S : a.I;
        if (P > 1) {
          // Raw gate and up sums of this contraction part (gate_up_part_floats layout).
          float* part = a.gpart + static_cast<size_t>(d.part) * gate_up_part_floats(a.T, a.K, a.I, a.S) +
                        (t.shared ? static_cast<size_t>(a.T) * a.K * 2 * a.I : 0);
#pragma unroll
          for (int i = 0; i < C::kRM; ++i)
#pragma unroll
            for (int jh = 0; jh < C::kCB / 2; ++jh) {
              const int col = d.n0 + wn * (BN / (2 * C::kWN)) + 16 * jh + r;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int m = t.m0 + wrow0 + 16 * i + 4 * g + e;
                if (m < t.rows) {
                  float* prow = part + static_cast<size_t>(t.shared ? m : t.rowbase + m) * 2 * width;
                  prow[col] = acc[i][jh][e];
                  prow[width + col] = acc[i][jh + C::kCB / 2][e];
                }
              }
            }
          return;
        }
#pragma unroll
        for (int i = 0; i < C::kRM; ++i)
#pragma unroll
          for (int jh = 0; jh < C::kCB / 2; ++jh) {
            const int col = d.n0 + wn * (BN / (2 * C::kWN)) + 16 * jh + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = t.m0 + wrow0 + 16 * i + 4 * g + e;
              if (m < t.rows) {
                const float hv = silu_f32(acc[i][jh][e]) * acc[i][jh + C::kCB / 2][e];
                const size_t idx = t.shared ? a.h_shared + static_cast<size_t>(m) * width + col
                                            : static_cast<size_t>(t.rowbase + m) * width + col;
                if constexpr (FP8) static_cast<float*>(a.h)[idx] = hv;
                else static_cast<uint16_t*>(a.h)[idx] = f32_to_bf16_bits(hv);
              }
            }
          }
      } else {
#pragma unroll
        for (int i = 0; i < C::kRM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = t.m0 + wrow0 + 16 * i + 4 * g + e;
            if (m < t.rows) {
              float* row = t.shared ? a.y + static_cast<size_t>(m) * H
                                    : a.o + static_cast<size_t>(slot_clamp(dslot[i][e], a)) * H;
              const float w = t.shared ? dgate[i][e] : 1.0f;
#pragma unroll
              for (int j = 0; j < C::kCB; ++j)
                row[d.n0 + wn * (BN / C::kWN) + 16 * j + r] = w * acc[i][j][e];
            }
          }
      }
    };

    int cg = 0;   // group cursor of the computed tile
    Tile cp = make_tile(walk.tile, cg);
    int cp_tile = walk.tile, cp_ks = 0;
    fetch_dst(cp);
    clear_acc();
    __syncthreads();   // stage 0 is in buffer 0
    for (int k = 0; k < nstages; ++k) {
      compute(k & 1);
      if (++cp_ks == cp.nk) {
        epilogue(cp);
        clear_acc();
        cp_ks = 0;
        cp_tile += walk.step;
        if (cp_tile <= last) {
          cp = make_tile(cp_tile, cg);
          fetch_dst(cp);
        }
      }
      __syncthreads();
    }
  }
}

// Finishing pass of a contraction-split gate/up launch: the parts' gate and up
// sums are added in order p = 0, 1, ... and h = SwiGLU is written where the
// unsplit kernel writes it.  Routed dispatch rows [0, offsets[E]) (I columns),
// then the shared expert's T rows (S columns); four columns per thread.
template <bool H_F32>
__global__ void __launch_bounds__(256) gate_up_finish_kernel(ExpertArgs a) {
  const size_t pf = gate_up_part_floats(a.T, a.K, a.I, a.S);
  const size_t shared0 = static_cast<size_t>(a.T) * a.K * 2 * a.I;
  const int64_t routed = static_cast<int64_t>(a.offsets[a.E]) * (a.I / 4);
  const int64_t items = routed + (a.S > 0 ? static_cast<int64_t>(a.T) * (a.S / 4) : 0);
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; it < items;
       it += static_cast<int64_t>(gridDim.x) * 256) {
    const bool sh = it >= routed;
    const int64_t j = sh ? it - routed : it;
    const int width = sh ? a.S : a.I;
    const int64_t row = j / (width / 4);
    const int c = static_cast<int>(j - row * (width / 4)) * 4;
    const float* src = a.gpart + (sh ? shared0 : 0) + static_cast<size_t>(row) * 2 * width + c;
    float4 gs = *reinterpret_cast<const float4*>(src);
    float4 us = *reinterpret_cast<const float4*>(src + width);
    for (int p = 1; p < a.kparts; ++p) {
      const float4 gv = *reinterpret_cast<const float4*>(src + p * pf);
      const float4 uv = *reinterpret_cast<const float4*>(src + p * pf + width);
      gs.x += gv.x; gs.y += gv.y; gs.z += gv.z; gs.w += gv.w;
      us.x += uv.x; us.y += uv.y; us.z += uv.z; us.w += uv.w;
    }
    const float hv[4] = {silu_f32(gs.x) * us.x, silu_f32(gs.y) * us.y, silu_f32(gs.z) * us.z,
                         silu_f32(gs.w) * us.w};
    const size_t idx = sh ? a.h_shared + static_cast<size_t>(row) * a.S + c : static_cast<size_t>(row) * a.I + c;
    if constexpr (H_F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(a.h) + idx) = float4{hv[0], hv[1], hv[2], hv[3]};
    } else {
      const uint32_t lo = f32_to_bf16_bits(hv[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(hv[1])) << 16);
      const uint32_t hi = f32_to_bf16_bits(hv[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(hv[3])) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h) + idx) = uint2{lo, hi};
    }
  }
}

// Upper bound of the tile count (host side; the device computes the exact one).
int64_t stream_tiles(const ExpertArgs& a, int BM, int nt_routed, int nt_shared) {
  const int64_t slots = static_cast<int64_t>(a.T) * a.K;
  int64_t b = (slots / BM + std::min<int64_t>(a.E, slots)) * nt_routed;
  if (a.S > 0) b += ceil_div(a.T, BM) * nt_shared;
  return b;
}

// One workgroup per CU (256 CUs), fewer if there are fewer tiles.
int stream_grid(int64_t tiles) {
  const int64_t b = std::min<int64_t>(tiles, 256);
  return static_cast<int>(std::max<int64_t>(kXcdCount, ceil_div(b, kXcdCount) * kXcdCount));
}

template <SMode MODE, int BM, int BN, int WM, int FMT>
hipError_t launch_stream(const ExpertArgs& a, hipStream_t stream) {
  using C = StreamCfg<MODE, BM, BN, WM, FMT>;
  constexpr int NS = stream_stages(C::kAPasses + C::kBPasses);
  const int bn_cols = (MODE == SMode::GateUp) ? BN / 2 : BN;
  const int nt_r = (MODE == SMode::GateUp) ? a.I / bn_cols : a.H / bn_cols;
  const int nt_s = (MODE == SMode::GateUp) ? a.S / bn_cols : a.H / bn_cols;
  const int parts = (MODE == SMode::GateUp) ? std::max(1, a.kparts) : 1;
  const int grid = stream_grid(stream_tiles(a, BM, nt_r, nt_s) * parts);
  stream_expert_kernel<MODE, BM, BN, WM, FMT, NS><<<grid, kStreamThreads, 0, stream>>>(a);
  return hipGetLastError();
}

constexpr int64_t kStreamTallRows = 48;   // rows per expert from which the tiles are 128 rows tall

// Tile shape from the average rows per expert rho = T*K/E: 16-row tiles up to 12
// rows, 32 up to 24, 64 up to 48, then 128 x 128 (below the 256-row LDS-tiled
// kernels' range, and for MXFP4 at every size).  Gate/up tiles of 32 or 64 rows use 64 weight rows
// (the compute waves split 2 x 2) when 128-row tiles would leave fewer than ~3
// tiles per CU: its tiles all have H/128 stages, so the count per workgroup sets
// the balance.  Down tiles keep 128 weight rows: they are short (I/128 stages),
// there are H/128 of them per row block, and wider tiles re-read fewer h rows.
// kFp8Quad where its double-buffered 512-byte row stages fit LDS next to the tile
// schedule (tiles of at most 144 token and weight rows: 16 x 128, 64 x 64,
// 32 x 64); larger tiles run kFp8Wide.  MXFP4 128 x 128 tiles run in 256-element
// stages.
template <int FMT, int BM, int BN>
constexpr int fit_fmt() {
  return FMT == kMxWide && BM + BN > 192 ? kDtypeMxfp4 : (FMT == kFp8Quad && BM + BN > 144) ? kFp8Wide : FMT;
}

// Contraction split of the gate/up projection for calls too small to give every
// CU a tile: one or a few tokens touch few experts, and with 64 intermediate
// columns per tile the launch has fewer tiles than CUs (the one-token drafter step:
// 64).  Each tile is cut into P parts of the contraction (P divides H/128, or
// H/512 with fp8 weights, so that the parts end on stage boundaries of every
// stage form), so that ~P times more CUs stream the weights; the parts write raw
// gate and up sums and gate_up_finish_kernel adds them in fixed order and applies
// SwiGLU.  P minimises an estimate of the stages the busiest CU runs.  Measured
// (drafter gate/up): T = 1 40.9 -> 25.5 us, T = 2 43.6 -> 33.5, T = 4 43.6 ->
// 33.2, fp8 T = 1 34.0 -> 30.2, narrow layer T = 1 51.4 -> 42.0; calls with at
// least as many tiles as CUs are not split (at T = 224 a split ran slower: the
// partial sums and the second launch cost more than the balance gains).
int split_tile_rows(int64_t rho) { return rho <= 12 ? 16 : rho <= 24 ? 32 : 64; }

template <int FMT>
hipError_t launch_gate_up_split(const ExpertArgs& a, int64_t rho, hipStream_t stream) {
  constexpr SMode M = SMode::GateUp;
  hipError_t e;
  switch (split_tile_rows(rho)) {
    case 16: e = launch_stream<M, 16, 128, 1, fit_fmt<FMT, 16, 128>()>(a, stream); break;
    case 32: e = launch_stream<M, 32, 128, 1, fit_fmt<FMT, 32, 128>()>(a, stream); break;
    default: e = launch_stream<M, 64, 128, 1, fit_fmt<FMT, 64, 128>()>(a, stream); break;
  }
  if (e != hipSuccess) return e;
  const int64_t items = static_cast<int64_t>(a.T) * a.K * (a.I / 4) + static_cast<int64_t>(a.T) * (a.S / 4);
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ceil_div(items, 256), 4096)));
  if (FMT == kDtypeBf16) gate_up_finish_kernel<false><<<grid, 256, 0, stream>>>(a);
  else gate_up_finish_kernel<true><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

template <SMode MODE, int FMT>
hipError_t launch_stream_rho(const ExpertArgs& a, int64_t rho, hipStream_t stream) {
  if constexpr (MODE == SMode::GateUp) {
    if (a.kparts > 1) return launch_gate_up_split<FMT>(a, rho, stream);
  }
  const int64_t slots = static_cast<int64_t>(a.T) * a.K;
  const int64_t touched = std::min<int64_t>(a.E, slots);
  const int64_t n_out = (MODE == SMode::GateUp) ? a.I : a.H;
  const int64_t tiles128 = touched * (MODE == SMode::GateUp ? n_out / 64 : n_out / 128);
  const bool narrow = MODE == SMode::GateUp && tiles128 < 3 * 256;
  // Down tiles of 64 weight rows only where 128-row ones would leave most CUs
  // without a tile (fewer than 256 of them), for bf16 and fp8 weights: the
  // one-token drafter step's down projection ran 17 % (bf16) and 13 % (fp8)
  // faster; from 7 tokens on they were no faster, at 56 and 224 tokens slower
  // (8 %, 13 %), and with MXFP4 weights 3 % slower at one token.
  const bool narrow_down = MODE == SMode::Down && tiles128 < 256 && FMT != kDtypeMxfp4 && FMT != kMxWide;
  // From kStreamTallRows rows per expert: 128 x 128 tiles (MXFP4 in 256-element
  // stages: the 512-element form of this tile does not fit LDS).  For MXFP4 they
  // give 33 % more flops per loaded byte than 64 x 128 in 512-element stages and
  // ran the large layer 16 % faster at T = 8192; for bf16 and fp8 they ran 3-7 %
  // faster than 128-row LDS-tiled kernels between 48 and 160 rows per expert.
  if (rho >= kStreamTallRows) {
    if constexpr (FMT == kDtypeMxfp4 || FMT == kMxWide) {
      // MXFP4: 128 x 256 tiles (256 weight rows) where the output widths allow:
      // 1.5x the flops per loaded byte of 128 x 128.
      const bool wide = (MODE == SMode::GateUp) ? (a.I % 128 == 0 && a.S % 128 == 0) : a.H % 256 == 0;
      if (wide) return launch_stream<MODE, 128, 256, 2, kDtypeMxfp4>(a, stream);
    }
    return launch_stream<MODE, 128, 128, 2, fit_fmt<FMT, 128, 128>()>(a, stream);
  }
  if constexpr (MODE == SMode::Down) {
    if (rho <= 12 && narrow_down) return launch_stream<MODE, 16, 64, 1, fit_fmt<FMT, 16, 64>()>(a, stream);
  }
  if (rho <= 12) return launch_stream<MODE, 16, 128, 1, fit_fmt<FMT, 16, 128>()>(a, stream);
  if (rho <= 24) return narrow ? launch_stream<MODE, 32, 64, 2, fit_fmt<FMT, 32, 64>()>(a, stream)
                               : launch_stream<MODE, 32, 128, 1, fit_fmt<FMT, 32, 128>()>(a, stream);
  return narrow ? launch_stream<MODE, 64, 64, 2, fit_fmt<FMT, 64, 64>()>(a, stream)
                : launch_stream<MODE, 64, 128, 1, fit_fmt<FMT, 64, 128>()>(a, stream);
}

}  // namespace

int gate_up_kparts(int64_t T, int K, int E, int H, int I, int S, int weight_dtype) {
  // bf16 and fp8 weights (MXFP4's one-token gate/up, at 0.25 of the bf16 bytes,
  // measured no faster split).
  if (weight_dtype != kDtypeBf16 && weight_dtype != kDtypeFp8) return 1;
  const int unit = weight_dtype == kDtypeBf16 ? 128 : 512;   // contraction elements per part step
  if (T <= 0 || E <= 0 || H % unit != 0 || I % 64 != 0 || S % 64 != 0) return 1;
  const int64_t rho = T * K / E;
  if (rho >= kStreamTallRows) return 1;
  const int64_t touched = std::min<int64_t>(E, T * K);
  const int64_t tiles = touched * (I / 64) + (S > 0 ? ceil_div(T, split_tile_rows(rho)) * (S / 64) : 0);
  if (tiles >= 256) return 1;
  // Estimated time in 256-byte row steps: rounds of work items over the 256 CUs,
  // each item its share of a weight row's bytes plus ~2 steps of pipeline fill.
  const int q = H / unit;
  const int64_t nk = weight_dtype == kDtypeBf16 ? H / 128 : H / 256;
  auto cost = [&](int p) { return ceil_div(tiles * p, 256) * (nk / p + 2); };
  int best = 1;
  for (int p = 2; p <= 16; ++p)
    if (q % p == 0 && cost(p) < cost(best)) best = p;
  return best;
}

hipError_t launch_router_stream(const ExpertArgs& a, hipStream_t stream) {
  if (a.kparts > 1) {
    // 128 x 128 tiles over 1/kparts of H each (partial logit planes, added in
    // order by the top-k pass): a third fewer bytes through the CUs than 64-row
    // tiles over all of H, with as many work items.
    const int grid = stream_grid(ceil_div(a.T, 128) * ceil_div(a.ncols, 128) * a.kparts);
    using C = StreamCfg<SMode::Router, 128, 128, 2, kDtypeBf16>;
    constexpr int NS = stream_stages(C::kAPasses + C::kBPasses);
    stream_expert_kernel<SMode::Router, 128, 128, 2, kDtypeBf16, NS><<<grid, kStreamThreads, 0, stream>>>(a);
    return hipGetLastError();
  }
  const int grid = stream_grid(ceil_div(a.T, 64) * ceil_div(a.ncols, 128));
  using C = StreamCfg<SMode::Router, 64, 128, 1, kDtypeBf16>;
  constexpr int NS = stream_stages(C::kAPasses + C::kBPasses);
  stream_expert_kernel<SMode::Router, 64, 128, 1, kDtypeBf16, NS><<<grid, kStreamThreads, 0, stream>>>(a);
  return hipGetLastError();
}

// fp8 runs in two-group stages when every contraction (H, I, S) is a multiple of 256;
// gate/up in four-group stages when H is a multiple of 512 and its scale arrays are
// 16-byte aligned (one 16-byte scale load per row and stage: narrow layer 8 %
// faster; the down projection's one-stage tiles ran 3 % slower in them).
static bool fp8_wide(const ExpertArgs& a) { return a.H % 256 == 0 && a.I % 256 == 0 && a.S % 256 == 0; }
static bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }
// The four-group kernels keep the tile walk's cost prefix in 32 bits: bound it by
// the tile count of the smallest tiles (16 rows, 32 columns) times the stages.
static bool quad_costs_fit(const ExpertArgs& a, int64_t n_routed, int64_t n_shared, int64_t kmax) {
  const int64_t rows = static_cast<int64_t>(a.T) * a.K / 16 + std::min<int64_t>(a.E, static_cast<int64_t>(a.T) * a.K);
  const int64_t tiles = rows * ceil_div(n_routed, 32) + ceil_div(a.T, 16) * ceil_div(n_shared, 32);
  return tiles * (kmax / 512) < (int64_t{1} << 31);
}
static bool fp8_quad_gate_up(const ExpertArgs& a) {
  return fp8_wide(a) && a.H % 512 == 0 && aligned16(a.xs) && aligned16(a.s_gate) && aligned16(a.s_up) &&
         aligned16(a.ss_gate) && aligned16(a.ss_up) && quad_costs_fit(a, a.I, a.S, a.H);
}


// MXFP4 runs in 512-element stages (256-byte weight row pieces) when the
// projection's contractions are multiples of 512.
static bool mx_wide_gate_up(const ExpertArgs& a) { return a.H % 512 == 0; }
static bool mx_wide_down(const ExpertArgs& a) { return a.I % 512 == 0 && a.S % 512 == 0; }

hipError_t launch_gate_up_stream(const ExpertArgs& a, int weight_dtype, int64_t rho, hipStream_t stream) {
  if (weight_dtype == kDtypeMxfp4)
    return mx_wide_gate_up(a) ? launch_stream_rho<SMode::GateUp, kMxWide>(a, rho, stream)
                              : launch_stream_rho<SMode::GateUp, kDtypeMxfp4>(a, rho, stream);
  if (weight_dtype == kDtypeFp8)
    return fp8_quad_gate_up(a) ? launch_stream_rho<SMode::GateUp, kFp8Quad>(a, rho, stream)
           : fp8_wide(a)       ? launch_stream_rho<SMode::GateUp, kFp8Wide>(a, rho, stream)
                               : launch_stream_rho<SMode::GateUp, kDtypeFp8>(a, rho, stream);
  return launch_stream_rho<SMode::GateUp, kDtypeBf16>(a, rho, stream);
}

hipError_t launch_down_stream(const ExpertArgs& a, int weight_dtype, int64_t rho, hipStream_t stream) {
  if (weight_dtype == kDtypeMxfp4)
    return mx_wide_down(a) ? launch_stream_rho<SMode::Down, kMxWide>(a, rho, stream)
                           : launch_stream_rho<SMode::Down, kDtypeMxfp4>(a, rho, stream);
  if (weight_dtype == kDtypeFp8)
    return fp8_wide(a) ? launch_stream_rho<SMode::Down, kFp8Wide>(a, rho, stream)
                       : launch_stream_rho<SMode::Down, kDtypeFp8>(a, rho, stream);
  return launch_stream_rho<SMode::Down, kDtypeBf16>(a, rho, stream);
}

}  // namespace moe
