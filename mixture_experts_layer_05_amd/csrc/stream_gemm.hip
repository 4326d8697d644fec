// Weight-streaming grouped expert GEMMs for decode-sized M (few rows per expert).
//
// At decode sizes every routed expert sees a handful of tokens, so the layer is
// bound by reading each touched expert's weights once from HBM [SpecForge PR
// #943, "Motivation": each draft step streams the touched experts' weights].
// This kernel is organised for that stream:
//
//   * a workgroup (4 waves) owns a tile of BN weight rows of one group (routed
//     expert or shared expert) and BM rows of tokens;
//   * the contraction runs in stages of 256 bytes per row (128 bf16, or one fp8
//     128-group of 128 bytes).  Global loads give each row 256 (bf16) or 128 (fp8)
//     contiguous bytes per wave instruction, the pattern that measured ~7 TB/s on
//     MI355X, whereas loading MFMA fragments straight from HBM (16 rows x 64 bytes
//     per instruction) stays near 4-5 TB/s;
//   * two stages are in flight in registers while the current one is consumed
//     from LDS, so each workgroup keeps ~2 x (BN + BM) x 256 bytes of loads
//     outstanding and a CU holds several workgroups;
//   * each wave computes all BM rows against BN/4 weight rows with 16x16x32 bf16
//     or 16x16x128 fp8 MFMAs (fp8 partial sums rescaled by the row and column
//     group scales in float32);
//   * gate/up tiles fuse SwiGLU and write h; down tiles stage the finished tile in
//     LDS and store whole row segments (512 bytes) of each slot's output row.
#include "kernels.h"
#include "schedule.h"

namespace moe {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kXcdCount = 8;   // the tile walk assumes grids that are multiples of 8

// GateUp: h = SwiGLU(x W_gate^T, x W_up^T); Down: o / y = h W_down^T; Router: the
// router logits z = x [W_r; w_g]^T over all T tokens (one group of T rows).
enum class SMode { GateUp, Down, Router };

template <SMode MODE, int BM, int BN, int WM, bool FP8>
struct StreamCfg {
  static constexpr int kWM = WM;                               // waves along rows
  static constexpr int kWN = 4 / WM;                           // waves along weight rows
  static constexpr int kRowData = FP8 ? 128 : 256;            // bytes per row per stage
  static constexpr int kRowStride = kRowData + 8;             // padded LDS row (8 mod 16)
  static constexpr int kLanesPerRow = kRowData / 16;
  static constexpr int kRowsPerPass = kStreamThreads / kLanesPerRow;
  static constexpr int kAPasses = (BM + kRowsPerPass - 1) / kRowsPerPass;
  static constexpr int kBPasses = BN / kRowsPerPass;
  static constexpr int kRM = BM / WM / 16;                     // row blocks per wave
  static constexpr int kCB = BN / kWN / 16;                    // column blocks per wave
  static constexpr int kElems = FP8 ? 128 : 128;               // contraction elements per stage
  static constexpr int kStage = (BM + BN) * kRowStride;
  static constexpr int kOutBytes = MODE == SMode::Down ? BM * (BN + 4) * 4 : 0;
  static constexpr int kSmem = kStage > kOutBytes ? kStage : kOutBytes;
  static_assert(BN % kRowsPerPass == 0, "BN must be a multiple of the rows per pass");
  static_assert(MODE == SMode::Down || kCB % 2 == 0, "gate/up needs gate and up blocks");
  static_assert(kRM >= 1 && BM % (16 * WM) == 0, "rows per wave must be a multiple of 16");
};

// Weight row of the LDS B tile read by column block j of the wave in weight-row
// column wn of kWN (lane row r).  Gate/up tiles hold BN/2 gate rows then the BN/2
// up rows of the same intermediate columns; wave column wn takes the gate and up
// rows of columns [wn*BN/(2*kWN), (wn+1)*BN/(2*kWN)).
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

template <SMode MODE, int BM, int BN, int WM, bool FP8>
__global__ void __launch_bounds__(kStreamThreads) stream_expert_kernel(ExpertArgs a) {
  using C = StreamCfg<MODE, BM, BN, WM, FP8>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::kSmem];
  __shared__ __attribute__((aligned(16))) float sscale[FP8 ? BM + BN : 4];
  __shared__ int prefix[kSchedInts];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave / C::kWN, wn = wave % C::kWN;
  const int wrow0 = wm * (BM / WM);   // first tile row of this wave

  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int H = a.H;
  const int bn_cols = (MODE == SMode::GateUp) ? BN / 2 : BN;
  int total;
  if constexpr (MODE == SMode::Router) {
    total = static_cast<int>(ceil_div(a.T, BM) * ceil_div(a.ncols, BN));
  } else {
    const int nt_r = (MODE == SMode::GateUp) ? a.I / bn_cols : H / bn_cols;
    const int nt_s = has_shared ? ((MODE == SMode::GateUp) ? a.S / bn_cols : H / bn_cols) : 0;
    total = build_tile_prefix(prefix, a.counts, a.offsets, a.E, a.T, has_shared, BM, nt_r, nt_s);
  }
  const XcdWalk walk(total);
  if (walk.tile >= walk.end) return;   // uniform across the workgroup

  const int lrow = tid / C::kLanesPerRow;            // row inside a load pass
  const int lcol = (tid % C::kLanesPerRow) * 16;     // byte offset inside the stage slice
  const size_t esz = FP8 ? 1 : 2;

  // ---- tile geometry
  struct Tile {
    TileInfo t;
    int kdim, nk, n0;
  };
  auto make_tile = [&](int tile) {
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
      d.t = find_tile(prefix, G, tile, a, BM);
    }
    d.kdim = (MODE != SMode::Down) ? H : (d.t.shared ? a.S : a.I);
    d.nk = d.kdim / C::kElems;
    d.n0 = d.t.nt * bn_cols;
    return d;
  };
  auto hrow = [&](const Tile& d, int m) -> size_t {   // element offset of row m in h / hq
    return d.t.shared ? a.h_shared + static_cast<size_t>(m) * d.kdim
                      : static_cast<size_t>(d.t.rowbase + m) * d.kdim;
  };
  // Rows past the group's end are not loaded: their LDS rows keep stale data, which
  // only reaches output rows that are never written.
  auto a_live = [&](const Tile& d, int q) {
    const int row = lrow + q * C::kRowsPerPass;
    return row < BM && d.t.m0 + row < d.t.rows;
  };

  // ---- sources of this thread's 16-byte pieces for one tile
  struct Src {
    const uint8_t* a[C::kAPasses];
    const uint8_t* b[C::kBPasses];
    const float* s;
  };
  auto make_src = [&](const Tile& d) {
    Src S;
    const TileInfo& t = d.t;
    const int ng = d.kdim / kGroup;
#pragma unroll
    for (int q = 0; q < C::kAPasses; ++q) {
      const int row = lrow + q * C::kRowsPerPass;
      const int m = min(t.m0 + min(row, BM - 1), t.rows - 1);
      if constexpr (MODE != SMode::Down)
        S.a[q] = (FP8 ? a.xq : static_cast<const uint8_t*>(a.x)) +
                 static_cast<size_t>(row_token(a, t, m)) * H * esz;
      else
        S.a[q] = (FP8 ? a.hq : static_cast<const uint8_t*>(a.h)) + hrow(d, m) * esz;
    }
    const uint8_t* w0;
    const uint8_t* w1 = nullptr;
    const float* sw0 = nullptr;
    const float* sw1 = nullptr;
    if constexpr (MODE == SMode::GateUp) {
      w0 = static_cast<const uint8_t*>(t.shared ? a.ws_gate : a.w_gate);
      w1 = static_cast<const uint8_t*>(t.shared ? a.ws_up : a.w_up);
      if (!t.shared) {
        w0 += static_cast<size_t>(t.group) * a.I * H * esz;
        w1 += static_cast<size_t>(t.group) * a.I * H * esz;
      }
      if constexpr (FP8) {
        sw0 = t.shared ? a.ss_gate : a.s_gate + static_cast<size_t>(t.group) * a.I * ng;
        sw1 = t.shared ? a.ss_up : a.s_up + static_cast<size_t>(t.group) * a.I * ng;
      }
    } else if constexpr (MODE == SMode::Router) {
      w0 = static_cast<const uint8_t*>(a.w_router);
    } else {
      w0 = static_cast<const uint8_t*>(t.shared ? a.ws_down : a.w_down);
      if (!t.shared) w0 += static_cast<size_t>(t.group) * H * a.I * esz;
      if constexpr (FP8) sw0 = t.shared ? a.ss_down : a.s_down + static_cast<size_t>(t.group) * H * ng;
    }
#pragma unroll
    for (int q = 0; q < C::kBPasses; ++q) {
      const int br = lrow + q * C::kRowsPerPass;
      if constexpr (MODE == SMode::GateUp) {
        S.b[q] = (br < BN / 2) ? w0 + static_cast<size_t>(d.n0 + br) * d.kdim * esz
                               : w1 + static_cast<size_t>(d.n0 + br - BN / 2) * d.kdim * esz;
      } else if constexpr (MODE == SMode::Router) {
        // Column c < E: router row c; c == E: the shared gate vector; columns past
        // the last one re-read a valid row and are never stored.
        const int c = min(d.n0 + br, a.ncols - 1);
        S.b[q] = (c < a.E) ? w0 + static_cast<size_t>(c) * d.kdim * esz
                           : static_cast<const uint8_t*>(a.w_gcol);
      } else {
        S.b[q] = w0 + static_cast<size_t>(d.n0 + br) * d.kdim * esz;
      }
    }
    S.s = nullptr;
    if constexpr (FP8) {
      // Thread tid < BM stages the scale of tile row tid, BM <= tid < BM+BN that of
      // B row tid-BM.
      if (tid < BM) {
        const int m = min(t.m0 + tid, t.rows - 1);
        if constexpr (MODE == SMode::GateUp) S.s = a.xs + static_cast<size_t>(row_token(a, t, m)) * ng;
        else S.s = a.hs + hrow(d, m) / kGroup;
      } else if (tid < BM + BN) {
        const int br = tid - BM;
        if constexpr (MODE == SMode::GateUp)
          S.s = (br < BN / 2) ? sw0 + static_cast<size_t>(d.n0 + br) * ng
                              : sw1 + static_cast<size_t>(d.n0 + br - BN / 2) * ng;
        else
          S.s = sw0 + static_cast<size_t>(d.n0 + br) * ng;
      }
    }
    return S;
  };

  struct Regs {
    uint4 a[C::kAPasses], b[C::kBPasses];
    float s;
  };
  auto gload = [&](Regs& R, const Tile& d, const Src& S, int ks) {
    const size_t off = static_cast<size_t>(ks) * C::kRowData + lcol;
#pragma unroll
    for (int q = 0; q < C::kBPasses; ++q) R.b[q] = ld16_stream(S.b[q] + off);
#pragma unroll
    for (int q = 0; q < C::kAPasses; ++q)
      if (a_live(d, q)) R.a[q] = ld16(S.a[q] + off);
    if constexpr (FP8) {
      if (S.s) R.s = S.s[ks];
    }
  };
  auto lstore = [&](const Regs& R, const Tile& d) {
#pragma unroll
    for (int q = 0; q < C::kAPasses; ++q)
      if (a_live(d, q))
        lds_st16(smem + (lrow + q * C::kRowsPerPass) * C::kRowStride + lcol, R.a[q]);
#pragma unroll
    for (int q = 0; q < C::kBPasses; ++q)
      lds_st16(smem + (BM + lrow + q * C::kRowsPerPass) * C::kRowStride + lcol, R.b[q]);
    if constexpr (FP8) {
      if (tid < BM + BN) sscale[tid] = R.s;
    }
  };

  f32x4 acc[C::kRM][C::kCB];
  auto clear_acc = [&]() {
#pragma unroll
    for (int i = 0; i < C::kRM; ++i)
#pragma unroll
      for (int j = 0; j < C::kCB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  auto compute = [&]() {
    const uint8_t* As = smem + (wrow0 + r) * C::kRowStride;
    const uint8_t* Bs = smem + BM * C::kRowStride;
    if constexpr (!FP8) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 af[C::kRM], bf[C::kCB];
#pragma unroll
        for (int i = 0; i < C::kRM; ++i) af[i] = lds_ld16(As + 16 * i * C::kRowStride + 64 * s + 16 * g);
#pragma unroll
        for (int j = 0; j < C::kCB; ++j)
          bf[j] = lds_ld16(Bs + stream_b_row<MODE, BN, C::kWN, C::kCB>(wn, j, r) * C::kRowStride + 64 * s +
                           16 * g);
#pragma unroll
        for (int i = 0; i < C::kRM; ++i)
#pragma unroll
          for (int j = 0; j < C::kCB; ++j) acc[i][j] = mfma_bf16_16x16x32(af[i], bf[j], acc[i][j]);
      }
    } else {
      // Lane group g holds bytes [16g, +16) and [64+16g, +16) of its row's 128-byte group.
      i32x8 af[C::kRM], bf[C::kCB];
      f32x4 sa[C::kRM];
      float sb[C::kCB];
#pragma unroll
      for (int i = 0; i < C::kRM; ++i) {
        const uint8_t* p = As + 16 * i * C::kRowStride;
        const uint4 lo = lds_ld16(p + 16 * g);
        const uint4 hi = lds_ld16(p + 64 + 16 * g);
        af[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sa[i] = *reinterpret_cast<const f32x4*>(&sscale[wrow0 + 16 * i + 4 * g]);
      }
#pragma unroll
      for (int j = 0; j < C::kCB; ++j) {
        const int br = stream_b_row<MODE, BN, C::kWN, C::kCB>(wn, j, r);
        const uint8_t* p = Bs + br * C::kRowStride;
        const uint4 lo = lds_ld16(p + 16 * g);
        const uint4 hi = lds_ld16(p + 64 + 16 * g);
        bf[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sb[j] = sscale[BM + br];
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
            if (m < t.rows && col < a.ncols) a.z[static_cast<size_t>(m) * a.ldz + col] = acc[i][j][e];
          }
        }
    } else if constexpr (MODE == SMode::GateUp) {
      const int width = t.shared ? a.S : a.I;
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
      // Stage the BM x BN tile in LDS (all waves are past their last read of the
      // operand tile), then each wave stores whole BN-column row segments.
      __syncthreads();
      float* out = reinterpret_cast<float*>(smem);
      constexpr int ld = BN + 4;
#pragma unroll
      for (int i = 0; i < C::kRM; ++i)
#pragma unroll
        for (int j = 0; j < C::kCB; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            out[(wrow0 + 16 * i + 4 * g + e) * ld + wn * (BN / C::kWN) + 16 * j + r] = acc[i][j][e];
      __syncthreads();
      for (int q = wave; q < BM; q += 4) {
        const int m = t.m0 + q;
        if (m >= t.rows) break;
        const DownDst dst = down_row(a, t, m);
        float* yr = dst.row + d.n0;
#pragma unroll
        for (int c = lane; c < BN; c += kWave) yr[c] = dst.w * out[q * ld + c];
      }
    }
  };

  // ---- the stage stream
  // The workgroup's tiles are consumed as one stream of stages.  Two stages are in
  // flight in registers (R0 / R1 alternate) while one is consumed from LDS; the load
  // cursor runs ahead across tile boundaries, so the next tile's first stages are
  // already in flight while the current tile finishes and writes its results.
  Tile ld = make_tile(walk.tile);
  Src lsrc = make_src(ld);
  int ld_tile = walk.tile, ld_ks = 0;
  auto issue = [&](Regs& R) {
    if (ld_tile >= walk.end) return;
    gload(R, ld, lsrc, ld_ks);
    if (++ld_ks == ld.nk) {
      ld_ks = 0;
      ld_tile += walk.step;
      if (ld_tile < walk.end) {
        ld = make_tile(ld_tile);
        lsrc = make_src(ld);
      }
    }
  };
  Tile cp = ld;
  int cp_tile = walk.tile, cp_ks = 0;
  // Consume one stage; returns false after the workgroup's last tile is written.
  auto consume = [&]() {
    compute();
    if (++cp_ks < cp.nk) return true;
    epilogue(cp);
    clear_acc();
    cp_ks = 0;
    cp_tile += walk.step;
    if (cp_tile >= walk.end) return false;
    cp = make_tile(cp_tile);
    return true;
  };

  Regs R0, R1;
  clear_acc();
  issue(R0);
  issue(R1);
  while (true) {
    __syncthreads();                   // every wave is past its reads of the LDS stage
    lstore(R0, cp);
    __syncthreads();
    issue(R0);
    if (!consume()) break;
    __syncthreads();
    lstore(R1, cp);
    __syncthreads();
    issue(R1);
    if (!consume()) break;
  }
}

int stream_grid(const ExpertArgs& a, int BM, int nt_routed, int nt_shared, int per_cu) {
  const int64_t slots = static_cast<int64_t>(a.T) * a.K;
  int64_t b = (slots / BM + std::min<int64_t>(a.E, slots)) * nt_routed;
  if (a.S > 0) b += ceil_div(a.T, BM) * nt_shared;
  b = std::min<int64_t>(b, 256LL * per_cu);
  return static_cast<int>(std::max<int64_t>(kXcdCount, ceil_div(b, kXcdCount) * kXcdCount));
}

template <SMode MODE, int BM, int BN, int WM, bool FP8>
hipError_t launch_stream(const ExpertArgs& a, hipStream_t stream) {
  const int bn_cols = (MODE == SMode::GateUp) ? BN / 2 : BN;
  const int nt_r = (MODE == SMode::GateUp) ? a.I / bn_cols : a.H / bn_cols;
  const int nt_s = (MODE == SMode::GateUp) ? a.S / bn_cols : a.H / bn_cols;
  const int grid = stream_grid(a, BM, nt_r, nt_s, 2);
  stream_expert_kernel<MODE, BM, BN, WM, FP8><<<grid, kStreamThreads, 0, stream>>>(a);
  return hipGetLastError();
}

// Tile shape from the average rows per expert rho = T*K/E: 16-row tiles up to 12
// rows, 32 up to 24, 64 above.  Tiles of 32 or 64 rows use 64 weight rows split
// over 2 waves (the other 2 waves split the rows) when 128-row tiles would leave
// fewer than ~3 tiles per CU, so that every CU streams from several workgroups.
template <SMode MODE, bool FP8>
hipError_t launch_stream_rho(const ExpertArgs& a, int64_t rho, hipStream_t stream) {
  const int64_t slots = static_cast<int64_t>(a.T) * a.K;
  const int64_t touched = std::min<int64_t>(a.E, slots);
  const int64_t n_out = (MODE == SMode::GateUp) ? a.I : a.H;
  const int64_t tiles128 = touched * (MODE == SMode::GateUp ? n_out / 64 : n_out / 128);
  const bool narrow = tiles128 < 3 * 256;
  if (rho <= 12) return launch_stream<MODE, 16, 128, 1, FP8>(a, stream);
  if (rho <= 24) return narrow ? launch_stream<MODE, 32, 64, 2, FP8>(a, stream)
                               : launch_stream<MODE, 32, 128, 1, FP8>(a, stream);
  return narrow ? launch_stream<MODE, 64, 64, 2, FP8>(a, stream)
                : launch_stream<MODE, 64, 128, 1, FP8>(a, stream);
}

}  // namespace

hipError_t launch_router_stream(const ExpertArgs& a, hipStream_t stream) {
  const int64_t tiles = ceil_div(a.T, 64) * ceil_div(a.ncols, 128);
  const int grid = static_cast<int>(std::max<int64_t>(
      kXcdCount, ceil_div(std::min<int64_t>(tiles, 256LL * 4), kXcdCount) * kXcdCount));
  stream_expert_kernel<SMode::Router, 64, 128, 1, false><<<grid, kStreamThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_gate_up_stream(const ExpertArgs& a, bool fp8, int64_t rho, hipStream_t stream) {
  return fp8 ? launch_stream_rho<SMode::GateUp, true>(a, rho, stream)
             : launch_stream_rho<SMode::GateUp, false>(a, rho, stream);
}

hipError_t launch_down_stream(const ExpertArgs& a, bool fp8, int64_t rho, hipStream_t stream) {
  return fp8 ? launch_stream_rho<SMode::Down, true>(a, rho, stream)
             : launch_stream_rho<SMode::Down, false>(a, rho, stream);
}

}  // namespace moe
