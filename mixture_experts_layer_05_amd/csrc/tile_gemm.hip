// LDS-tiled grouped expert GEMMs for prefill-sized M (many rows per expert).
//
// Same contract as the streaming kernels in stream_gemm.hip (gate/up + SwiGLU
// into h; down into the per-slot output rows), organised for MFMA throughput
// instead of weight streaming:
//
//   * a workgroup of 8 waves owns a BM x BN output tile of one group (routed
//     expert or the shared expert); BM = 256 or 128 rows, BN = 256 columns (for
//     gate/up: 128 gate rows and the 128 up rows of the same intermediate
//     columns, so SwiGLU is fused in registers);
//   * the contraction runs in stages of 128 bytes per row (64 bf16 or one
//     128-element fp8 scale group).  Each stage of A (token rows, gathered
//     through the dispatch permutation) and B (weight rows) is loaded with
//     16-byte coalesced loads into registers one stage ahead, then written to a
//     double-buffered LDS tile whose rows are padded to 136 bytes (8 mod 16:
//     the MFMA fragment reads then run at full LDS rate, see common.h);
//   * each wave computes a 64-row x BN/WGN-column sub-tile with 16x16x32 bf16
//     MFMAs (two per stage and block pair) or 16x16x128 fp8 MFMAs (one per stage,
//     rescaled by the row and column group scales staged in LDS);
//   * tiles are walked persistently; consecutive tiles share a weight slab and
//     are given to workgroups on the same XCD, so the slab is fetched from HBM
//     once per XCD and the other m-tiles hit that XCD's L2.
#include "kernels.h"
#include "schedule.h"

namespace moe {
namespace {

constexpr int kTileThreads = 512;
constexpr int kRowBytes = 136;   // 128 data bytes + 8 padding bytes per LDS row
constexpr int kXcds = 8;
// m-tiles per band of the tile order (see find_tile): 8 row blocks x 4 weight slabs
// per 32 consecutive tiles.
constexpr int kBand = 8;

enum class Mode { GateUp, Down };

template <Mode MODE, int BM, int BN, bool FP8>
struct TileCfg {
  static constexpr int kBK = FP8 ? 128 : 64;        // contraction elements per stage
  static constexpr int kWGM = BM / 64;              // waves along M
  static constexpr int kWGN = 8 / kWGM;             // waves along N
  static constexpr int kWN = BN / kWGN;             // columns per wave
  static constexpr int kNB = kWN / 16;              // 16-column blocks per wave
  static constexpr int kAChunks = BM * 8 / kTileThreads;
  static constexpr int kBChunks = BN * 8 / kTileThreads;
  static constexpr int kStage = (BM + BN) * kRowBytes;
  static_assert(kAChunks >= 1 && kBChunks >= 1, "tile too small for 512 threads");
  static_assert(MODE == Mode::Down || kNB % 2 == 0, "gate/up needs pairs of blocks");
};

// Row of the LDS B tile that feeds column block j of wave wn (lane row r).
template <Mode MODE, int BN, int kWN, int kNB>
__device__ __forceinline__ int b_tile_row(int wn, int j, int r) {
  if constexpr (MODE == Mode::GateUp) {
    // Blocks [0, kNB/2) are gate rows, [kNB/2, kNB) the up rows of the same columns.
    const int jh = (j < kNB / 2) ? j : j - kNB / 2;
    return ((j < kNB / 2) ? 0 : BN / 2) + wn * (kWN / 2) + 16 * jh + r;
  } else {
    return wn * kWN + 16 * j + r;
  }
}

template <Mode MODE, int BM, int BN, bool FP8>
__global__ void __launch_bounds__(kTileThreads) tiled_expert_kernel(ExpertArgs a) {
  using C = TileCfg<MODE, BM, BN, FP8>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::kStage];
  __shared__ __attribute__((aligned(16))) float sscale[2][FP8 ? BM + BN : 4];
  __shared__ int prefix[kSchedInts];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave / C::kWGN, wn = wave % C::kWGN;

  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int H = a.H;
  const int bn_cols = (MODE == Mode::GateUp) ? BN / 2 : BN;   // output columns per tile
  const int nt_r = (MODE == Mode::GateUp) ? a.I / bn_cols : H / bn_cols;
  const int nt_s = has_shared ? ((MODE == Mode::GateUp) ? a.S / bn_cols : H / bn_cols) : 0;
  const int total = build_tile_prefix(prefix, a.counts, a.offsets, a.E, a.T, has_shared, BM, nt_r, nt_s);


  const int crow = tid >> 3;          // first row this thread loads (then +64, +128, ...)
  const int ccol = (tid & 7) * 16;    // byte offset inside the row's 128-byte stage slice

  const XcdWalk walk(total);
  for (int tile = walk.tile; tile < walk.end; tile += walk.step) {
    const TileInfo t = find_tile(prefix, G, tile, a, BM, kBand);
    const int kdim = (MODE == Mode::GateUp) ? H : (t.shared ? a.S : a.I);
    const int nk = kdim / C::kBK;
    const int n0 = t.nt * bn_cols;
    const size_t esz = FP8 ? 1 : 2;
    auto hrow = [&](int m) -> size_t {   // element offset of row m in h / hq
      return t.shared ? a.h_shared + static_cast<size_t>(m) * kdim
                      : static_cast<size_t>(t.rowbase + m) * kdim;
    };

    // ---- global source rows of this thread's 16-byte chunks
    const uint8_t* asrc[C::kAChunks];
#pragma unroll
    for (int q = 0; q < C::kAChunks; ++q) {
      const int m = min(t.m0 + crow + 64 * q, t.rows - 1);
      if constexpr (MODE == Mode::GateUp) {
        const size_t off = static_cast<size_t>(row_token(a, t, m)) * H * esz;
        asrc[q] = (FP8 ? a.xq : static_cast<const uint8_t*>(a.x)) + off;
      } else {
        asrc[q] = (FP8 ? a.hq : static_cast<const uint8_t*>(a.h)) + hrow(m) * esz;
      }
    }
    const uint8_t* wsrc_gate;
    const uint8_t* wsrc_up = nullptr;
    const float* ssrc_gate = nullptr;
    const float* ssrc_up = nullptr;
    const int ng = kdim / kGroup;
    if constexpr (MODE == Mode::GateUp) {
      wsrc_gate = static_cast<const uint8_t*>(t.shared ? a.ws_gate : a.w_gate);
      wsrc_up = static_cast<const uint8_t*>(t.shared ? a.ws_up : a.w_up);
      if (!t.shared) {
        wsrc_gate += static_cast<size_t>(t.group) * a.I * H * esz;
        wsrc_up += static_cast<size_t>(t.group) * a.I * H * esz;
      }
      if constexpr (FP8) {
        ssrc_gate = t.shared ? a.ss_gate : a.s_gate + static_cast<size_t>(t.group) * a.I * ng;
        ssrc_up = t.shared ? a.ss_up : a.s_up + static_cast<size_t>(t.group) * a.I * ng;
      }
    } else {
      wsrc_gate = static_cast<const uint8_t*>(t.shared ? a.ws_down : a.w_down);
      if (!t.shared) wsrc_gate += static_cast<size_t>(t.group) * H * a.I * esz;
      if constexpr (FP8) ssrc_gate = t.shared ? a.ss_down : a.s_down + static_cast<size_t>(t.group) * H * ng;
    }
    const uint8_t* bsrc[C::kBChunks];
#pragma unroll
    for (int q = 0; q < C::kBChunks; ++q) {
      const int br = crow + 64 * q;
      if constexpr (MODE == Mode::GateUp) {
        bsrc[q] = (br < BN / 2) ? wsrc_gate + static_cast<size_t>(n0 + br) * kdim * esz
                                : wsrc_up + static_cast<size_t>(n0 + br - BN / 2) * kdim * esz;
      } else {
        bsrc[q] = wsrc_gate + static_cast<size_t>(n0 + br) * kdim * esz;
      }
    }
    // fp8: thread tid < BM stages the scale of tile row tid, BM <= tid < BM+BN that of B row tid-BM.
    const float* sptr = nullptr;
    if constexpr (FP8) {
      if (tid < BM) {
        const int m = min(t.m0 + tid, t.rows - 1);
        if constexpr (MODE == Mode::GateUp) sptr = a.xs + static_cast<size_t>(row_token(a, t, m)) * ng;
        else sptr = a.hs + hrow(m) / kGroup;
      } else if (tid < BM + BN) {
        const int br = tid - BM;
        if constexpr (MODE == Mode::GateUp)
          sptr = (br < BN / 2) ? ssrc_gate + static_cast<size_t>(n0 + br) * ng
                               : ssrc_up + static_cast<size_t>(n0 + br - BN / 2) * ng;
        else
          sptr = ssrc_gate + static_cast<size_t>(n0 + br) * ng;
      }
    }

    uint4 ra[C::kAChunks], rb[C::kBChunks];
    float rs = 0.f;
    auto gload = [&](int ks) {
      const size_t off = static_cast<size_t>(ks) * 128 + ccol;
#pragma unroll
      for (int q = 0; q < C::kBChunks; ++q) rb[q] = ld16_stream(bsrc[q] + off);
#pragma unroll
      for (int q = 0; q < C::kAChunks; ++q) ra[q] = ld16(asrc[q] + off);
      if constexpr (FP8) {
        if (sptr) rs = sptr[ks];
      }
    };
    auto lstore = [&](int buf) {
      uint8_t* base = smem + buf * C::kStage;
#pragma unroll
      for (int q = 0; q < C::kAChunks; ++q)
        lds_st16(base + (crow + 64 * q) * kRowBytes + ccol, ra[q]);
#pragma unroll
      for (int q = 0; q < C::kBChunks; ++q)
        lds_st16(base + (BM + crow + 64 * q) * kRowBytes + ccol, rb[q]);
      if constexpr (FP8) {
        if (tid < BM + BN) sscale[buf][tid] = rs;
      }
    };

    f32x4 acc[4][C::kNB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < C::kNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    gload(0);
    lstore(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      const int buf = ks & 1;
      if (ks + 1 < nk) gload(ks + 1);
      const uint8_t* As = smem + buf * C::kStage + (wm * 64 + r) * kRowBytes;
      const uint8_t* Bs = smem + buf * C::kStage + BM * kRowBytes;
      if constexpr (!FP8) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          uint4 af[4], bf[C::kNB];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            af[i] = lds_ld16(As + i * 16 * kRowBytes + 64 * s + 16 * g);
#pragma unroll
          for (int j = 0; j < C::kNB; ++j)
            bf[j] = lds_ld16(
                Bs + b_tile_row<MODE, BN, C::kWN, C::kNB>(wn, j, r) * kRowBytes + 64 * s + 16 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < C::kNB; ++j) acc[i][j] = mfma_bf16_16x16x32(af[i], bf[j], acc[i][j]);
        }
      } else {
        i32x8 af[4], bf[C::kNB];
        f32x4 sa[4];
        float sb[C::kNB];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint8_t* p = As + i * 16 * kRowBytes;
          const uint4 lo = lds_ld16(p + 16 * g);
          const uint4 hi = lds_ld16(p + 64 + 16 * g);
          af[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          sa[i] = *reinterpret_cast<const f32x4*>(&sscale[buf][wm * 64 + 16 * i + 4 * g]);
        }
#pragma unroll
        for (int j = 0; j < C::kNB; ++j) {
          const int br = b_tile_row<MODE, BN, C::kWN, C::kNB>(wn, j, r);
          const uint8_t* p = Bs + br * kRowBytes;
          const uint4 lo = lds_ld16(p + 16 * g);
          const uint4 hi = lds_ld16(p + 64 + 16 * g);
          bf[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          sb[j] = sscale[buf][BM + br];
        }
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < C::kNB; ++j) {
            const f32x4 p = mfma_fp8_16x16x128(af[i], bf[j], zero);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(p[e], sa[i][e] * sb[j], acc[i][j][e]);
          }
      }
      if (ks + 1 < nk) lstore(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue
    if constexpr (MODE == Mode::GateUp) {
      const int width = t.shared ? a.S : a.I;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jh = 0; jh < C::kNB / 2; ++jh) {
          const int col = n0 + wn * (C::kWN / 2) + 16 * jh + r;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = t.m0 + wm * 64 + 16 * i + 4 * g + e;
            if (m < t.rows) {
              const float hv = silu_f32(acc[i][jh][e]) * acc[i][jh + C::kNB / 2][e];
              const size_t idx = t.shared ? a.h_shared + static_cast<size_t>(m) * width + col
                                          : static_cast<size_t>(t.rowbase + m) * width + col;
              if constexpr (FP8) static_cast<float*>(a.h)[idx] = hv;
              else static_cast<uint16_t*>(a.h)[idx] = f32_to_bf16_bits(hv);
            }
          }
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = t.m0 + wm * 64 + 16 * i + 4 * g + e;
          if (m >= t.rows) continue;
          const DownDst dst = down_row(a, t, m);
          float* yr = dst.row + n0 + wn * C::kWN + r;
#pragma unroll
          for (int j = 0; j < C::kNB; ++j) yr[16 * j] = dst.w * acc[i][j][e];
        }
    }
  }
}

int tiled_grid(const ExpertArgs& a, int BM, int nt_routed, int nt_shared) {
  const int64_t slots = static_cast<int64_t>(a.T) * a.K;
  int64_t b = (slots / BM + std::min<int64_t>(a.E, slots)) * nt_routed;
  if (a.S > 0) b += ceil_div(a.T, BM) * nt_shared;
  // One resident workgroup per CU (LDS-bound); a multiple of the XCD count.
  b = std::min<int64_t>(b, 256);
  return static_cast<int>(std::max<int64_t>(kXcds, ceil_div(b, kXcds) * kXcds));
}

}  // namespace

// fp8 uses 128-row tiles only: the 256-row fp8 tile does not fit 256 registers per lane.
hipError_t launch_gate_up_tiled(const ExpertArgs& a, bool fp8, bool tall, hipStream_t stream) {
  tall = tall && !fp8;
  const int BM = tall ? 256 : 128;
  const int grid = tiled_grid(a, BM, a.I / 128, a.S / 128);
  if (tall) {
    tiled_expert_kernel<Mode::GateUp, 256, 256, false><<<grid, kTileThreads, 0, stream>>>(a);
  } else {
    if (fp8) tiled_expert_kernel<Mode::GateUp, 128, 256, true><<<grid, kTileThreads, 0, stream>>>(a);
    else tiled_expert_kernel<Mode::GateUp, 128, 256, false><<<grid, kTileThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_down_tiled(const ExpertArgs& a, bool fp8, bool tall, hipStream_t stream) {
  tall = tall && !fp8;
  const int BM = tall ? 256 : 128;
  const int grid = tiled_grid(a, BM, a.H / 256, a.H / 256);
  if (tall) {
    tiled_expert_kernel<Mode::Down, 256, 256, false><<<grid, kTileThreads, 0, stream>>>(a);
  } else {
    if (fp8) tiled_expert_kernel<Mode::Down, 128, 256, true><<<grid, kTileThreads, 0, stream>>>(a);
    else tiled_expert_kernel<Mode::Down, 128, 256, false><<<grid, kTileThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe
