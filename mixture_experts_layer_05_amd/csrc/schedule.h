// Tile schedule shared by the expert kernels (included by each kernel file).
//
// A "group" is a routed expert (rows = its dispatch segment) or the shared expert
// (rows = every token).  Tiles are (group, m-tile of BM rows, n-tile); the
// per-group tile counts come from expert_counts on the device, so no host round
// trip is needed.
#pragma once

#include "kernels.h"

namespace moe {
namespace {

constexpr int kDtypeF32 = 0, kDtypeBf16 = 1, kDtypeFp8 = 2, kDtypeMxfp4 = 3;

// The schedule lives in LDS: prefix[0..G] of per-group tile counts, then each
// group's row count and first dispatch row, so that finding a tile's group reads no
// global memory.  prefix[g+1] - prefix[g] = ceil(rows_g / BM) * ntiles_g for g in
// [0, G), where group E (if has_shared) is the shared expert with T rows.
//
// split divides a call's rows between two kernels by the realised counts (0: all
// rows here).  A group of r rows is "tall" when r >= kSplitRows; its first
// r_t = r rows, or r - r % kTallTile when that tail is shorter than kSplitRows,
// go to the 256-row kernel (split 1; every one of its tiles is then at least half
// full), and the other rows (short groups whole, tall groups' short tails from row
// r_t on) to the streaming kernel (split 2).  Splits 3 and 4 divide split 2's rows
// once more, by group: the groups left with more than kMidRows of them (split 3,
// for 128-row streaming tiles, which read a weight slab once where 64-row tiles
// read it twice) and the others (split 4), provided those groups give at least
// kMidMinTiles tiles of mid_nt n-tiles each; fewer would run as a launch that
// leaves most CUs idle, so then split 4 takes all of split 2's rows and split 3
// none.  Both launches must pass the same mid_nt (the 128-row launch's n-tiles per
// group), whatever their own tile width, so that they divide the rows alike.  The
// shared expert is never cut: its rows are token indices.
constexpr int kSchedStride = kMaxExperts + 2;
constexpr int kSchedInts = 3 * kSchedStride;

constexpr int kSplitRows = 128;
constexpr int kTallTile = 256;
constexpr int kMidRows = 64;
constexpr int kMidMinTiles = 256;

__device__ int build_tile_prefix(int* sched, const int32_t* counts, const int32_t* offsets, int E, int T,
                                 bool has_shared, int BM, int nt_routed, int nt_shared, int split = 0,
                                 int mid_nt = 0) {
  const int G = E + (has_shared ? 1 : 0);
  int* prefix = sched;
  int* rows_of = sched + kSchedStride;
  int* base_of = sched + 2 * kSchedStride;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    // Rows of group g left to the streaming kernel in a row-divided call.
    auto rest_of = [&](int g, int& first) {
      const int r = (g < E) ? counts[g] : T;
      const int tail = r % kTallTile;
      const int rt = r < kSplitRows ? 0 : ((g < E && r >= kTallTile && tail < kSplitRows) ? r - tail : r);
      first = rt;
      return r - rt;
    };
    bool by_size = false;
    if (split >= 3) {
      int mid_tiles = 0;
      for (int base = 0; base < G; base += kWave) {
        const int g = base + lane;
        int first;
        const bool mid = g < G && rest_of(g, first) > kMidRows;
        mid_tiles += __popcll(__ballot(mid));
      }
      by_size = mid_tiles * mid_nt >= kMidMinTiles;
    }
    int carry = 0;
    for (int base = 0; base < G; base += kWave) {
      const int g = base + lane;
      int v = 0;
      if (g < G) {
        const int r = (g < E) ? counts[g] : T;
        int rows = r, first = 0;
        if (split != 0) {
          const int rest = rest_of(g, first);
          if (split == 1) {
            rows = r - rest;
            first = 0;
          } else {
            rows = rest;
            if (split == 3 && (!by_size || rows <= kMidRows)) rows = 0;
            if (split == 4 && by_size && rows > kMidRows) rows = 0;
          }
        }
        rows_of[g] = rows;
        base_of[g] = (g < E) ? offsets[g] + first : 0;
        v = static_cast<int>(ceil_div(rows, BM)) * ((g < E) ? nt_routed : nt_shared);
      }
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int n = __shfl_up(v, o, kWave);
        if (lane >= o) v += n;
      }
      if (g < G) prefix[g + 1] = carry + v;
      carry += __shfl(v, kWave - 1, kWave);
    }
    if (lane == 0) prefix[0] = 0;
  }
  __syncthreads();
  return prefix[G];
}

struct TileInfo {
  int group;   // expert id, or E for the shared expert
  bool shared;
  int rows;    // rows of the group
  int rowbase; // first dispatch row of the group (routed) or 0 (shared)
  int m0;      // first row of the tile inside the group
  int nt;      // n-tile index
};

// Tile order inside a group: bands of `band` m-tiles; within a band the n-tiles are
// walked in order and, for each n-tile, the band's m-tiles are consecutive.  A run
// of consecutive tiles (the ones an XCD works on at once) then covers a few weight
// slabs x a few row blocks, so both operands are reused from that XCD's L2 instead
// of one operand being re-fetched for every tile.  band >= m-tiles gives plain
// m-fastest order.
__device__ __forceinline__ TileInfo tile_in_group(const int* sched, int g, int tile, const ExpertArgs& a,
                                                  int BM, int band = 1 << 30) {
  const int* prefix = sched;
  TileInfo t;
  t.group = g;
  t.shared = g == a.E;
  t.rows = sched[kSchedStride + g];
  t.rowbase = sched[2 * kSchedStride + g];
  const int mt = static_cast<int>(ceil_div(t.rows, BM));
  const int local = tile - prefix[g];
  if (band >= mt) {
    t.nt = local / mt;
    t.m0 = (local % mt) * BM;
    return t;
  }
  const int ntile = (prefix[g + 1] - prefix[g]) / mt;
  const int per_band = band * ntile;
  const int first_m = (local / per_band) * band;
  const int bm = min(mt - first_m, band);
  const int in_band = local - (first_m / band) * per_band;
  t.nt = in_band / bm;
  t.m0 = (first_m + in_band % bm) * BM;
  return t;
}

__device__ __forceinline__ TileInfo find_tile(const int* sched, int G, int tile, const ExpertArgs& a,
                                              int BM, int band = 1 << 30) {
  const int* prefix = sched;
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= tile) lo = mid; else hi = mid;
  }
  return tile_in_group(sched, lo, tile, a, BM, band);
}

// Group of `tile` (the last g < G with prefix[g] <= tile), found by scanning forward
// from group g, which must satisfy prefix[g] <= tile: a persistent walk only moves
// forward.  Each lane of the (whole, converged) wave tests one later group, so one
// LDS read covers 64 groups; prefix is non-decreasing, so the passed groups are the
// first lanes of the ballot.
__device__ __forceinline__ int advance_group(const int* prefix, int G, int tile, int g) {
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  for (;;) {
    const int c = g + 1 + lane;
    const bool passed = c < G && prefix[c] <= tile;
    const int n = __popcll(__ballot(passed));
    g += n;
    if (n < kWave) return g;
  }
}

// Persistent walk over [0, total): the tiles are cut into 8 contiguous ranges, one
// per XCD (workgroup b runs on XCD b % 8), and the workgroups of an XCD stride
// through its range.  Neighbouring tiles share a weight slab, so the m-tiles of a
// slab run at the same time on one XCD and share its L2, and every XCD gets an
// equal share whatever the grid size.  gridDim.x must be a multiple of 8.
struct XcdWalk {
  int tile, end, step;
  __device__ __forceinline__ XcdWalk(int total) {
    const int per = (total + 7) / 8;
    const int xcd = blockIdx.x % 8;
    tile = xcd * per + blockIdx.x / 8;
    end = min(total, xcd * per + per);
    step = gridDim.x / 8;
  }
};

// A dispatch entry clamped into [0, T*K): every slot index the kernels derive an
// address from stays inside its buffer, whatever perm holds (the dispatch leaves
// entries unwritten only for invalid ids, which the header rules out).
__device__ __forceinline__ int slot_clamp(int s, const ExpertArgs& a) {
  return static_cast<int>(min(static_cast<unsigned>(s), static_cast<unsigned>(a.T * a.K - 1)));
}

// Token behind row m of a tile (m clamped into the group by the caller).
__device__ __forceinline__ int row_token(const ExpertArgs& a, const TileInfo& t, int m) {
  return t.shared ? m : slot_clamp(a.perm[t.rowbase + m], a) / a.K;
}

// Destination of row m of a down-projection tile: routed rows go, unweighted, to
// their slot's row of o; shared-expert rows go to y weighted by sigmoid(g).
struct DownDst {
  float* row;
  float w;
};

__device__ __forceinline__ DownDst down_row(const ExpertArgs& a, const TileInfo& t, int m) {
  if (t.shared) return {a.y + static_cast<size_t>(m) * a.H, a.shared_gate[m]};
  return {a.o + static_cast<size_t>(slot_clamp(a.perm[t.rowbase + m], a)) * a.H, 1.0f};
}

}  // namespace
}  // namespace moe
