// LDS-tiled grouped expert GEMMs for prefill-sized M (many rows per expert).
//
// Same contract as the streaming kernels in stream_gemm.hip (gate/up + SwiGLU
// into h; down into the per-slot output rows), organised for MFMA throughput
// instead of weight streaming.  A workgroup owns a 256-row output tile of one
// group (routed expert or the shared expert); for gate/up, the tile's B rows are
// gate rows and the up rows of the same intermediate columns, so SwiGLU is fused
// in registers.  The contraction runs in stages of 128 bytes per activation row
// (64 bf16, one 128-element fp8 scale group, or 128 MXFP8 codes).  Tiles are walked persistently; consecutive
// tiles share a weight slab or a row block and are given to workgroups on the
// same XCD, so those operands are fetched from HBM once per XCD and hit that
// XCD's L2 afterwards.  Three kernels, each with two waves per SIMD:
//
//   * tiledpp_expert_kernel (bf16): 256 x 256 tiles, 8 waves of 128 x 64 with
//     32x32x16 MFMAs; see its own description below.
//   * tiled8pp_expert_kernel (fp8): 256 x 256 tiles, 8 waves of 128 x 64 with
//     16x16x128 fp8 MFMAs and all operands loaded by LDS DMA; see below.
//   * tiledmx_expert_kernel (MXFP4 weights x MXFP8 activations): 256 x 256 tiles,
//     8 waves of 64 x 128 on the block-scaled fp8 x fp4 MFMA; see below.
//
// The expert launchers (experts.hip) give these kernels the rows that fill a
// 256-row tile at least half, in calls large enough to fill the GPU with such
// tiles; the streaming kernels serve the rest (their 128 x 128 tiles ran 3-7 %
// faster than 128-row LDS tiles for those, measured).
#include "kernels.h"
#include "schedule.h"

namespace moe {
namespace {

constexpr int kXcds = 8;
// m-tiles per band of the tile order (see find_tile): 8 row blocks x 4 weight slabs
// per 32 consecutive tiles.
constexpr int kBand = 8;

enum class Mode { GateUp, Down };

// ---------------------------------------------------------------- 256-row tiles: shared pieces
//
// A stage of the 256-row kernels is 64 contraction elements of bf16 (or one
// 128-element fp8 group): 128 bytes of each A row and B row, double-buffered in
// LDS.  Full 128-byte row pieces matter: from L2, a CU receives about 2.5x the
// bytes per clock with 128-byte pieces than with 64-byte ones (measured).
//   * A (gathered activation rows, mostly L2 hits) goes memory -> LDS directly,
//     one stage ahead, with buffer loads carrying the LDS flag (each wave
//     instruction writes 64 lanes x 16 bytes = 1 KiB of consecutive LDS);
//   * bf16 B (weight rows, streamed from HBM) is loaded into registers two stages
//     ahead and written to LDS one stage ahead, which keeps two stages of the
//     HBM stream in flight per CU within the LDS budget.
// Rows are stored unpadded with their eight 16-byte pieces permuted by
// (row / 2) mod 8; a fragment read (32 rows x one piece) then touches each
// 16-byte bank group of the 256-byte bank width once per 16 rows.
constexpr int kT4RowBytes = 128;                        // 64 bf16 per row per stage
constexpr int kT4Stage = (256 + 256) * kT4RowBytes;     // 64 KiB

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Buffer resource words for a raw byte buffer.
__device__ __forceinline__ i32x4_t dma_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t r = {static_cast<int>(static_cast<uint32_t>(p)), static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xffff),
               static_cast<int>(bytes), 0x00020000};
  r.x = __builtin_amdgcn_readfirstlane(r.x);
  r.y = __builtin_amdgcn_readfirstlane(r.y);
  r.z = __builtin_amdgcn_readfirstlane(r.z);
  return r;
}

// Wave instructions of buffer loads with the LDS flag.  Instruction q: lane l
// loads 16 bytes at resource offset voff[q] + soff and writes them to LDS at
// lds + 1024 q + 16 l (M0 holds the LDS address; a write of M0 needs one wait
// state before the load that uses it).  Completion is counted by vmcnt like any
// load; the caller waits for it explicitly.  The compiler does not see these
// accesses: it neither waits for them nor moves LDS accesses across them
// ("memory" clobber).
#define MOE_DMA_LINE(V, S) "s_nop 0\n\tbuffer_load_dwordx4 " V ", %[rs], " S " offen lds\n\t"
#define MOE_DMA_NEXT "s_add_u32 m0, m0, 0x400\n\t"

// Four instructions (voff[0..3]).
__device__ __forceinline__ void dma4_rows(i32x4_t rsrc, const uint32_t (&voff)[4], uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %[lds]\n\t"
               MOE_DMA_LINE("%[v0]", "%[so]") MOE_DMA_NEXT MOE_DMA_LINE("%[v1]", "%[so]") MOE_DMA_NEXT
               MOE_DMA_LINE("%[v2]", "%[so]") MOE_DMA_NEXT MOE_DMA_LINE("%[v3]", "%[so]")
               :
               : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [v2] "v"(voff[2]), [v3] "v"(voff[3]),
                 [rs] "s"(rsrc), [so] "s"(__builtin_amdgcn_readfirstlane(soff)),
                 [lds] "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "scc");
}

// Two 16-byte instructions over rows `step` bytes apart (voff[0], then voff[1] at
// soff + step), writing LDS at lds and lds + 1024.
__device__ __forceinline__ void dma2_step(i32x4_t rsrc, const uint32_t (&voff)[2], uint32_t soff, uint32_t step,
                                          uint32_t lds) {
  uint32_t so;
  asm volatile("s_mov_b32 m0, %[lds]\n\ts_mov_b32 %[so], %[s0]\n\t"
               MOE_DMA_LINE("%[va]", "%[so]") MOE_DMA_NEXT "s_add_u32 %[so], %[so], %[st]\n\t"
               MOE_DMA_LINE("%[vb]", "%[so]")
               : [so] "=&s"(so)
               : [va] "v"(voff[0]), [vb] "v"(voff[1]), [rs] "s"(rsrc),
                 [s0] "s"(__builtin_amdgcn_readfirstlane(soff)), [st] "s"(__builtin_amdgcn_readfirstlane(step)),
                 [lds] "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "scc");
}

// One 4-byte instruction: lane l loads the dword at voff + soff into LDS at lds + 4 l.
__device__ __forceinline__ void dma1_dword(i32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %[lds]\n\ts_nop 0\n\tbuffer_load_dword %[v], %[rs], %[so] offen lds"
               :
               : [v] "v"(voff), [rs] "s"(rsrc), [so] "s"(__builtin_amdgcn_readfirstlane(soff)),
                 [lds] "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

#undef MOE_DMA_LINE
#undef MOE_DMA_NEXT

// Wait until at most N vector-memory instructions of this wave are outstanding
// (they complete in issue order).  vmcnt sits in bits 3:0 and 15:14; expcnt and
// lgkmcnt are left at "no wait".
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xf00);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- 256 x 256, 8 waves (bf16)
//
// The bf16 prefill tile: 256 x 256 outputs per workgroup of 8 waves, two per
// SIMD.  Wave w computes rows [128 (w / 4), +128) x one quarter of the tile's
// columns as 4 x 2 blocks of 32x32 (32x32x16 MFMAs, 128 accumulator registers),
// so that one wave's fragment reads and waits overlap the other's MFMAs.  With
// one wave per SIMD (4 waves of 128 x 128, 256 accumulators each) the same tile
// ran 9.5 % slower on the large layer's gate/up (measured); the 32x32x16 MFMA
// sustains close to the chip's peak where the 16x16x32 one reaches about half.
// Per stage each wave issues 4 DMA instructions of activation rows, then 4
// register loads of weight rows.
constexpr int kPPThreads = 512;

template <Mode MODE>
__global__ void __launch_bounds__(kPPThreads) tiledpp_expert_kernel(ExpertArgs a) {
  constexpr int BM = 256, BN = 256;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kT4Stage];
  __shared__ int prefix[kSchedInts];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int wm = wave >> 2, wn = wave & 3;

  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int H = a.H;
  const int bn_cols = (MODE == Mode::GateUp) ? BN / 2 : BN;
  const int nt_r = (MODE == Mode::GateUp) ? a.I / bn_cols : H / bn_cols;
  const int nt_s = has_shared ? ((MODE == Mode::GateUp) ? a.S / bn_cols : H / bn_cols) : 0;
  const int total = build_tile_prefix(prefix, a.counts, a.offsets, a.E, a.T, has_shared, BM, nt_r, nt_s,
                                      a.split);

  // DMA lane mapping: instruction q of this wave covers tile rows
  // 8 (4 wave + q) + lane / 8; LDS piece lane % 8 holds global piece
  // (lane % 8) ^ ((row / 2) mod 8), which depends only on q's parity.
  const int drow = lane >> 3;
  uint32_t dpiece[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) dpiece[h] = static_cast<uint32_t>(((lane & 7) ^ ((4 * h + (drow >> 1)) & 7)) * 16);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(smem));
  const int r32 = lane & 31, hi = lane >> 5;
  const uint32_t fswz = static_cast<uint32_t>(hi ^ ((r32 >> 1) & 7));
  // B register rows t / 8 + 64 q: the piece permutation depends on t / 8 only.
  const uint32_t bldsoff = static_cast<uint32_t>((tid >> 3) * kT4RowBytes + (((tid & 7) ^ ((tid >> 4) & 7)) * 16));

  const XcdWalk walk(total);
  for (int tile = walk.tile; tile < walk.end; tile += walk.step) {
    TileInfo t = find_tile(prefix, G, tile, a, BM, kBand);
    t.group = __builtin_amdgcn_readfirstlane(t.group);
    t.shared = __builtin_amdgcn_readfirstlane(static_cast<int>(t.shared)) != 0;
    t.rows = __builtin_amdgcn_readfirstlane(t.rows);
    t.rowbase = __builtin_amdgcn_readfirstlane(t.rowbase);
    t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
    t.nt = __builtin_amdgcn_readfirstlane(t.nt);
    const int kdim = (MODE == Mode::GateUp) ? H : (t.shared ? a.S : a.I);
    const int nk = kdim / 64;
    const int n0 = t.nt * bn_cols;
    const uint32_t krow = static_cast<uint32_t>(kdim) * 2;   // bytes per operand row

    i32x4_t ra;
    const uint8_t* b0p;   // B rows [0, 128) of the tile
    const uint8_t* b1p;   // B rows [128, 256)
    uint32_t aoff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = min(t.m0 + 8 * (4 * wave + q) + drow, t.rows - 1);
      if constexpr (MODE == Mode::GateUp)
        aoff[q] = static_cast<uint32_t>(row_token(a, t, m)) * krow + dpiece[q & 1];
      else
        aoff[q] = static_cast<uint32_t>(m) * krow + dpiece[q & 1];
    }
    if constexpr (MODE == Mode::GateUp) {
      ra = dma_rsrc(a.x, static_cast<uint32_t>(a.T) * krow);
      const uint8_t* wg = static_cast<const uint8_t*>(t.shared ? a.ws_gate : a.w_gate);
      const uint8_t* wu = static_cast<const uint8_t*>(t.shared ? a.ws_up : a.w_up);
      const size_t eoff = (t.shared ? 0 : static_cast<size_t>(t.group) * a.I * krow) +
                          static_cast<size_t>(n0) * krow;
      b0p = wg + eoff;
      b1p = wu + eoff;
    } else {
      const size_t hrow = t.shared ? static_cast<size_t>(a.h_shared) : static_cast<size_t>(t.rowbase) * kdim;
      ra = dma_rsrc(static_cast<const uint8_t*>(a.h) + hrow * 2, static_cast<uint32_t>(t.rows) * krow);
      const uint8_t* wd = static_cast<const uint8_t*>(t.shared ? a.ws_down : a.w_down);
      const size_t eoff = (t.shared ? 0 : static_cast<size_t>(t.group) * H * krow) +
                          static_cast<size_t>(n0) * krow;
      b0p = wd + eoff;
      b1p = wd + eoff + 128 * static_cast<size_t>(krow);
    }
    const __amdgpu_buffer_rsrc_t rb0v = buf_rsrc(b0p, 128 * krow);
    const __amdgpu_buffer_rsrc_t rb1v = buf_rsrc(b1p, 128 * krow);
    const uint32_t bvoff = static_cast<uint32_t>(tid >> 3) * krow + (tid & 7) * 16;
    // Down: the destinations of the 32 rows this wave stores in the epilogue (lane
    // l < 32: round l / 8, row 8 wave + l % 8 of it), loaded here and not touched
    // before the epilogue.  A load issued between the epilogue's stores would make
    // the wave wait for those stores (one counter covers loads and stores).
    int pre_slot = 0;
    float pre_w = 1.0f;
    if constexpr (MODE == Mode::Down) {
      const int l = lane & 31, R = 8 * wave + (l & 7), ri = l >> 3;
      const int m = min(t.m0 + (R < 32 ? 32 * ri + R : 128 + 32 * ri + (R - 32)), t.rows - 1);
      pre_slot = a.perm[t.rowbase + m];
      if (t.shared) pre_w = a.shared_gate[m];
    }

    auto issue_a = [&](int ks) {
      const uint32_t buf = lds0 + static_cast<uint32_t>(ks & 1) * kT4Stage + 4 * wave * 1024;
      dma4_rows(ra, aoff, static_cast<uint32_t>(ks) * kT4RowBytes, buf);
    };
    struct BRegs {
      uint4 v[4];
    };
    // Thread t holds B rows t / 8 + 64 q (q < 2 from rb0, the rest from rb1), piece t % 8.
    auto load_b = [&](BRegs& R, int ks) {
      const uint32_t kb = static_cast<uint32_t>(ks) * kT4RowBytes;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        R.v[q] = buf_ld16(q < 2 ? rb0v : rb1v, bvoff, kb + 64 * (q & 1) * krow);
    };
    auto store_b = [&](const BRegs& R, int ks) {
      uint8_t* dst = smem + (ks & 1) * kT4Stage + BM * kT4RowBytes + bldsoff;
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(dst + 64 * q * kT4RowBytes) = R.v[q];
    };

    constexpr int NI = 4;                      // 32-row blocks per wave
    constexpr int NJ = 2;                      // 32-column blocks per wave
    const int arow0 = wm * 128;

    // LDS row of B feeding 32-column block j.  Gate/up: block 0 is the gate rows,
    // block 1 the up rows of the wave's 32 intermediate columns.
    auto brow = [&](int j) -> int {
      if constexpr (MODE == Mode::GateUp) return (j == 0 ? 0 : BN / 2) + wn * 32 + r32;
      else return wn * 64 + 32 * j + r32;
    };

    f32x16 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    auto compute = [&](int ks) {
      const uint8_t* base = smem + (ks & 1) * kT4Stage;
      const uint8_t* As = base + (arow0 + r32) * kT4RowBytes;
      const uint8_t* Bs = base + BM * kT4RowBytes;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t piece = ((2 * kk) ^ fswz) * 16;
        uint4 af[NI], bf[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) bf[j] = *reinterpret_cast<const uint4*>(Bs + brow(j) * kT4RowBytes + piece);
#pragma unroll
        for (int i = 0; i < NI; ++i) af[i] = *reinterpret_cast<const uint4*>(As + i * 32 * kT4RowBytes + piece);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_bf16_32x32x16(af[i], bf[j], acc[i][j]);
      }
    };

    // nk is even (contractions are multiples of 128).  Iteration ks: wait for
    // A(ks); barrier; write B(ks + 1) from registers and start A(ks + 1) into
    // the other buffer; refill those registers with B(ks + 3); multiply stage
    // ks.  Each wait leaves only the newest 4 register loads in flight.  The
    // register loads are issued unconditionally (past the end they re-read the
    // last stage, an L2 hit), so every iteration has the same number of loads
    // in flight and the compiler's waits for the registers stay exact.
    BRegs R0, R1;
    load_b(R0, 0);
    load_b(R1, 1);
    __syncthreads();                 // the previous tile is done with both buffers
    store_b(R0, 0);
    issue_a(0);
    load_b(R0, min(2, nk - 1));
    for (int ks = 0; ks < nk; ks += 2) {
      wait_vm<4>();
      __syncthreads();
      store_b(R1, ks + 1);
      issue_a(ks + 1);
      load_b(R1, min(ks + 3, nk - 1));
      compute(ks);
      wait_vm<4>();
      __syncthreads();
      if (ks + 2 < nk) {
        store_b(R0, ks + 2);
        issue_a(ks + 2);
      }
      load_b(R0, min(ks + 4, nk - 1));
      compute(ks + 1);
    }
    wait_vm<0>();                    // no load may still be writing registers or LDS
    __syncthreads();                 // every wave is done reading the stage buffers

    // The tile leaves through LDS so that every global store is a whole row
    // segment: 16 bytes per lane, 256 contiguous bytes (h) or 1 KiB (down) per row
    // [the row-staged output of DeepGEMM fork PR #5, "What changed - large M", L2
    // scatter].  32x32 output placement: lane l, element v -> row 8 (v / 4) +
    // 4 (l / 32) + v % 4, column l % 32.
    if constexpr (MODE == Mode::GateUp) {
      // The whole 256 x 128 bf16 h tile, rows padded to 136 elements (272 bytes:
      // the two row halves a 32x32 store touches fall on disjoint banks).  Each
      // lane writes its own 2-byte element (a pairing of neighbouring columns
      // through a lane exchange made every write wait for that exchange).
      constexpr int kHs = 136;
      uint16_t* stg = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float hv = silu_f32(acc[i][0][v]) * acc[i][1][v];
          const int row = arow0 + 32 * i + 8 * (v >> 2) + 4 * hi + (v & 3);
          stg[row * kHs + wn * 32 + r32] = f32_to_bf16_bits(hv);
        }
      __syncthreads();
      const int width = t.shared ? a.S : a.I;
      uint16_t* hbase = static_cast<uint16_t*>(a.h) +
                        (t.shared ? static_cast<size_t>(a.h_shared) : static_cast<size_t>(t.rowbase) * width);
      const int piece = lane & 15;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = 32 * wave + 4 * k + (lane >> 4);
        const int m = t.m0 + row;
        const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(smem) + row * kHs * 2 +
                                                        piece * 16);
        if (m < t.rows) *reinterpret_cast<uint4*>(hbase + static_cast<size_t>(m) * width + n0 + 8 * piece) = v;
      }
      __syncthreads();               // the next tile's first loads overwrite the staging rows
    } else {
      // Four rounds of 64 tile rows (32 from each row half) x 256 float32 columns,
      // rows padded to 264 floats (the two row halves of a 32x32 store fall on
      // disjoint banks).  In each round wave w stores 8 whole rows, one 1 KiB
      // row segment per instruction.
      constexpr int kOs = 264;
      float* stg = reinterpret_cast<float*>(smem);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            stg[(wm * 32 + 8 * (v >> 2) + 4 * hi + (v & 3)) * kOs + wn * 64 + 32 * j + r32] = acc[i][j][v];
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int R = 8 * wave + k;
          const int m = t.m0 + (R < 32 ? 32 * i + R : 128 + 32 * i + (R - 32));
          const int slot = __shfl(pre_slot, 8 * i + k, kWave);
          const float w = __shfl(pre_w, 8 * i + k, kWave);
          if (m < t.rows) {          // uniform across the wave
            float* row = t.shared ? a.y + static_cast<size_t>(m) * a.H
                                  : a.o + static_cast<size_t>(slot_clamp(slot, a)) * a.H;
            float4 v = *reinterpret_cast<const float4*>(stg + R * kOs + 4 * lane);
            v.x *= w; v.y *= w; v.z *= w; v.w *= w;
            *reinterpret_cast<float4*>(row + n0 + 4 * lane) = v;
          }
        }
        __syncthreads();
      }
    }
  }
}

// ---------------------------------------------------------------- 256 x 256 (fp8): shared pieces
//
// The fp8 prefill tile: 256 x 256 outputs per workgroup, from 16x16x128 fp8
// MFMAs.  A stage is one 128-element scale group (128 bytes per row).  Every
// product is rescaled by its row and column group scales on the VALU, which
// cannot reach the accumulation registers; the accumulators therefore live in
// ordinary registers.
//
// Everything a stage needs goes memory -> LDS by DMA: the 256 activation rows,
// the 256 weight rows and both sets of group scales (64 KiB + 2 KiB).  Two stage
// buffers: the next stage is in flight while one is multiplied out.  The waits
// are explicit (every wave issues the same instructions per stage and they
// complete in order).  Same unpadded, piece-permuted row layout as the bf16 tile.
// Every kernel here receives its operands at a similar rate per CU, whatever
// their source (L2 or HBM), so the tile is as large as the registers allow: a
// 256 x 128 tile with two stages in flight (48 KiB per 8.4 MFLOP stage) ran the
// large fp8 layer slower than this one (66 KiB per 16.8 MFLOP stage).
constexpr int kF8Bufs = 2;
constexpr int kF8Stage = (256 + 256) * kT4RowBytes;   // 64 KiB

// ---------------------------------------------------------------- 256 x 256, 8 waves (fp8)
//
// 8 waves, two per SIMD: wave w computes rows [128 (w / 4), +128) x the column
// quarter w % 4 (gate/up: 32 gate and the 32 up rows of the same h columns;
// down: 64 output columns) as 8 x 4 blocks of 16x16 (128 accumulator registers),
// so that one wave's VALU rescale, fragment reads and waits overlap the other's
// MFMAs.  Per stage every wave issues the same 9 DMA instructions: 4 of
// activation rows (32 rows), 4 of weight rows (32 rows), and 1 of scales (waves
// 0-3: 64 activation rows each; waves 4-7: 64 weight rows each).
constexpr int kF8PPThreads = 512;

template <Mode MODE>
__global__ void __launch_bounds__(kF8PPThreads) tiled8pp_expert_kernel(ExpertArgs a) {
  constexpr int BM = 256, BN = 256;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kF8Bufs * kF8Stage];
  __shared__ __attribute__((aligned(16))) float sscale[kF8Bufs][BM + BN];
  __shared__ int prefix[kSchedInts];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int wm = wave >> 2, wn = wave & 3;

  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int H = a.H;
  const int bn_cols = (MODE == Mode::GateUp) ? BN / 2 : BN;
  const int nt_r = (MODE == Mode::GateUp) ? a.I / bn_cols : H / bn_cols;
  const int nt_s = has_shared ? ((MODE == Mode::GateUp) ? a.S / bn_cols : H / bn_cols) : 0;
  const int total = build_tile_prefix(prefix, a.counts, a.offsets, a.E, a.T, has_shared, BM, nt_r, nt_s,
                                      a.split);

  // DMA lane mapping: instruction q covers 8 rows (row 8 q' + lane / 8); LDS piece
  // lane % 8 holds global piece (lane % 8) ^ ((row / 2) mod 8), which depends on
  // q's parity only.
  const int drow = lane >> 3;
  uint32_t dpiece[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) dpiece[h] = static_cast<uint32_t>(((lane & 7) ^ ((4 * h + (drow >> 1)) & 7)) * 16);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(smem));
  const uint32_t sc0 = __builtin_amdgcn_readfirstlane(lds_address(&sscale[0][0]));
  const int r16 = lane & 15, g = lane >> 4;
  const uint32_t fsw = static_cast<uint32_t>((r16 >> 1) & 7);
  const uint32_t pc0 = (static_cast<uint32_t>(g) ^ fsw) * 16, pc1 = (static_cast<uint32_t>(4 + g) ^ fsw) * 16;

  const XcdWalk walk(total);
  for (int tile = walk.tile; tile < walk.end; tile += walk.step) {
    TileInfo t = find_tile(prefix, G, tile, a, BM, kBand);
    t.group = __builtin_amdgcn_readfirstlane(t.group);
    t.shared = __builtin_amdgcn_readfirstlane(static_cast<int>(t.shared)) != 0;
    t.rows = __builtin_amdgcn_readfirstlane(t.rows);
    t.rowbase = __builtin_amdgcn_readfirstlane(t.rowbase);
    t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
    t.nt = __builtin_amdgcn_readfirstlane(t.nt);
    const int kdim = (MODE == Mode::GateUp) ? H : (t.shared ? a.S : a.I);
    const int nk = kdim / kGroup;               // one scale group per stage
    const int ng = nk;
    const int n0 = t.nt * bn_cols;
    const uint32_t krow = static_cast<uint32_t>(kdim);          // bytes per fp8 row
    const size_t hrow0 = t.shared ? static_cast<size_t>(a.h_shared) : static_cast<size_t>(t.rowbase) * kdim;

    // A rows of this wave: 32 wave + 8 q + lane / 8 (q < 4).
    i32x4_t ra, rsa;
    uint32_t aoff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = min(t.m0 + 32 * wave + 8 * q + drow, t.rows - 1);
      if constexpr (MODE == Mode::GateUp)
        aoff[q] = static_cast<uint32_t>(row_token(a, t, m)) * krow + dpiece[q & 1];
      else
        aoff[q] = static_cast<uint32_t>(m) * krow + dpiece[q & 1];
    }
    if constexpr (MODE == Mode::GateUp) {
      ra = dma_rsrc(a.xq, static_cast<uint32_t>(a.T) * krow);
      rsa = dma_rsrc(a.xs, static_cast<uint32_t>(a.T) * ng * 4);
    } else {
      ra = dma_rsrc(a.hq + hrow0, static_cast<uint32_t>(t.rows) * krow);
      rsa = dma_rsrc(a.hs + hrow0 / kGroup, static_cast<uint32_t>(t.rows) * ng * 4);
    }
    // B rows of this wave: tile rows [32 wave, +32).  Gate/up: waves 0-3 the gate
    // rows n0 + 32 wave ..., waves 4-7 the up rows of the same h columns; down:
    // output rows n0 + 32 wave ...
    i32x4_t rb;
    uint32_t boff[4];
    {
      const uint8_t* wsrc;
      size_t erow;
      if constexpr (MODE == Mode::GateUp) {
        const bool up = wave >= 4;
        wsrc = static_cast<const uint8_t*>(t.shared ? (up ? a.ws_up : a.ws_gate) : (up ? a.w_up : a.w_gate));
        erow = (t.shared ? 0 : static_cast<size_t>(t.group) * a.I) + n0 + 32 * (wave & 3);
      } else {
        wsrc = static_cast<const uint8_t*>(t.shared ? a.ws_down : a.w_down);
        erow = (t.shared ? 0 : static_cast<size_t>(t.group) * H) + n0 + 32 * wave;
      }
      rb = dma_rsrc(wsrc + erow * krow, 32 * krow);
#pragma unroll
      for (int q = 0; q < 4; ++q) boff[q] = static_cast<uint32_t>(8 * q + drow) * krow + dpiece[q & 1];
    }
    // Down: the destinations of the wave's 128 output rows (lane l: rows
    // 128 wm + l and 128 wm + 64 + l), loaded here and not touched before the
    // epilogue (a load issued between the epilogue's stores would make the wave
    // wait for them).
    int pre_slot[2] = {0, 0};
    float pre_w[2] = {1.0f, 1.0f};
    if constexpr (MODE == Mode::Down) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = min(t.m0 + wm * 128 + 64 * h + lane, t.rows - 1);
        pre_slot[h] = a.perm[t.rowbase + m];
        if (t.shared) pre_w[h] = a.shared_gate[m];
      }
    }

    // The scale vector this wave stages: waves 0-3 the activation rows
    // [64 wave, +64); waves 4-7 the weight rows [64 (wave - 4), +64) (gate/up:
    // waves 4-5 gate rows, 6-7 up rows).
    i32x4_t rss;
    uint32_t ssoff, ssdst;
    if (wave < 4) {
      const int ms = min(t.m0 + 64 * wave + lane, t.rows - 1);
      rss = rsa;
      if constexpr (MODE == Mode::GateUp) ssoff = static_cast<uint32_t>(row_token(a, t, ms)) * ng * 4;
      else ssoff = static_cast<uint32_t>(ms) * ng * 4;
      ssdst = 64 * wave * 4;
    } else {
      const int bw = wave - 4;
      const float* ssrc;
      size_t erow;
      if constexpr (MODE == Mode::GateUp) {
        const bool up = bw >= 2;
        ssrc = t.shared ? (up ? a.ss_up : a.ss_gate) : (up ? a.s_up : a.s_gate);
        erow = (t.shared ? 0 : static_cast<size_t>(t.group) * a.I) + n0 + 64 * (bw & 1);
      } else {
        ssrc = t.shared ? a.ss_down : a.s_down;
        erow = (t.shared ? 0 : static_cast<size_t>(t.group) * H) + n0 + 64 * bw;
      }
      rss = dma_rsrc(ssrc + erow * ng, 64 * ng * 4);
      ssoff = static_cast<uint32_t>(lane) * ng * 4;
      ssdst = (BM + 64 * bw) * 4;
    }

    // Stage ks -> buffer ks % 2: A rows at [0, 32 KiB), B rows after; scales in sscale.
    auto issue = [&](int ks) {
      const int b = ks & 1;
      const uint32_t buf = lds0 + static_cast<uint32_t>(b) * kF8Stage;
      const uint32_t kb = static_cast<uint32_t>(ks) * kT4RowBytes;
      dma4_rows(ra, aoff, kb, buf + 4 * wave * 1024);
      dma4_rows(rb, boff, kb, buf + BM * kT4RowBytes + 4 * wave * 1024);
      const uint32_t sbuf = sc0 + static_cast<uint32_t>(b) * (BM + BN) * 4;
      dma1_dword(rss, ssoff, static_cast<uint32_t>(ks) * 4, sbuf + ssdst);
    };

    auto brow = [&](int j) -> int {
      if constexpr (MODE == Mode::GateUp) return ((j < 2) ? 0 : BN / 2) + wn * 32 + 16 * (j & 1) + r16;
      else return wn * 64 + 16 * j + r16;
    };
    auto frag = [&](const uint8_t* row) -> i32x8 {
      const uint4 lo = *reinterpret_cast<const uint4*>(row + pc0);
      const uint4 hi = *reinterpret_cast<const uint4*>(row + pc1);
      return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    constexpr int NI = 8;
    f32x4 acc[NI][4];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int ks) {
      const int b = ks & 1;
      const uint8_t* base = smem + b * kF8Stage;
      const uint8_t* As = base + (wm * 128 + r16) * kT4RowBytes;
      const uint8_t* Bs = base + BM * kT4RowBytes;
      const float* sA = &sscale[b][wm * 128 + 4 * g];
      const float* sB = &sscale[b][BM];
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      i32x8 bf[4];
      float sb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf[j] = frag(Bs + brow(j) * kT4RowBytes);
        sb[j] = sB[brow(j)];
      }
      // Products one row block ahead of their rescale (independent MFMA work
      // while the VALU waits for results).
      f32x4 pc[4], pn[4];
      {
        const i32x8 af = frag(As);
#pragma unroll
        for (int j = 0; j < 4; ++j) pc[j] = mfma_fp8_16x16x128(af, bf[j], zero);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (i + 1 < NI) {
          const i32x8 af = frag(As + (i + 1) * 16 * kT4RowBytes);
#pragma unroll
          for (int j = 0; j < 4; ++j) pn[j] = mfma_fp8_16x16x128(af, bf[j], zero);
        }
        const f32x4 sa = *reinterpret_cast<const f32x4*>(sA + 16 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(pc[j][e], sa[e] * sb[j], acc[i][j][e]);
#pragma unroll
        for (int j = 0; j < 4; ++j) pc[j] = pn[j];
      }
    };

    // Stage ks: wait for this wave's part of it; barrier (every wave's part has
    // landed and every wave is done with stage ks - 1); start stage ks + 1 into the
    // buffer stage ks - 1 used; multiply stage ks.
    __syncthreads();                   // the previous tile is done with both buffers
    issue(0);
    for (int ks = 0; ks < nk; ++ks) {
      wait_vm<0>();
      __syncthreads();
      if (ks + 1 < nk) issue(ks + 1);
      compute(ks);
    }

    // 16x16 output placement: lane l, element e -> row 4 (l / 16) + e, column l % 16.
    if constexpr (MODE == Mode::GateUp) {
      const int width = t.shared ? a.S : a.I;
      float* hbase = static_cast<float*>(a.h) +
                     (t.shared ? static_cast<size_t>(a.h_shared) : static_cast<size_t>(t.rowbase) * width);
      const int col0 = n0 + wn * 32 + r16;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = t.m0 + wm * 128 + 16 * i + 4 * g + e;
          if (m < t.rows) {
            float* hr = hbase + static_cast<size_t>(m) * width + col0;
#pragma unroll
            for (int jh = 0; jh < 2; ++jh) hr[16 * jh] = silu_f32(acc[i][jh][e]) * acc[i][jh + 2][e];
          }
        }
    } else {
      const int col0 = n0 + wn * 64 + r16;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + 4 * g + e;           // wave row; half i / 4 of pre_slot
          const int m = t.m0 + wm * 128 + r;
          const int slot = __shfl(pre_slot[i >> 2], r & 63, kWave);
          const float w = __shfl(pre_w[i >> 2], r & 63, kWave);
          if (m < t.rows) {
            float* yr = (t.shared ? a.y + static_cast<size_t>(m) * a.H
                                  : a.o + static_cast<size_t>(slot_clamp(slot, a)) * a.H) + col0;
#pragma unroll
            for (int j = 0; j < 4; ++j) yr[16 * j] = w * acc[i][j][e];
          }
        }
    }
  }
}

// ---------------------------------------------------------------- 256 x 256 (MXFP4)
//
// The MXFP4 prefill tile: MXFP8 activation rows x MXFP4 weight rows, 256 x 256
// outputs per workgroup, on the block-scaled 16x16x128 fp8 x fp4 MFMA, which
// applies both operands' E8M0 scales itself (no VALU rescale: the accumulators
// stay in the MFMA chain).  A stage is 128 contraction
// elements: 128 bytes of each activation row, 64 bytes of each weight row and one
// 4-byte scale word per row (the E8M0 bytes of its four 32-element blocks), 50 KiB
// per stage, all by LDS DMA into three stage buffers (two stages in flight).  Wave
// w computes rows [64 (w / 2), +64) x the column half w % 2 as 4 x 8 blocks of
// 16x16: a weight fragment is half an activation one, so this reads 16 KiB of
// fragments per wave and stage where the fp8 tile's 128 x 64 layout would read 20
// (measured ~1 % faster).
//
// Weight rows of 64 bytes (four 16-byte pieces) keep piece p at slot
// p ^ ((row / 4) mod 4): a fragment read (16 consecutive rows x one piece) then
// touches 16 distinct 16-byte bank groups.  A DMA instruction writes 16 such rows
// (1 KiB): lane l fills row l / 4, slot l % 4, so it loads global piece
// (l % 4) ^ ((l / 16) mod 4) of its row.
constexpr int kMxBufs = 3;
constexpr int kMxRowB = 64;                                  // weight bytes per row per stage
constexpr int kMxStage = 256 * kT4RowBytes + 256 * kMxRowB;   // 48 KiB of codes

template <Mode MODE>
__global__ void __launch_bounds__(kF8PPThreads) tiledmx_expert_kernel(ExpertArgs a) {
  constexpr int BM = 256, BN = 256;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kMxBufs * kMxStage];
  __shared__ __attribute__((aligned(16))) uint32_t sscale[kMxBufs][BM + BN];
  __shared__ int prefix[kSchedInts];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int wm = wave >> 1, wn = wave & 1;   // 64 rows x 128 columns per wave

  const bool has_shared = a.S > 0;
  const int G = a.E + (has_shared ? 1 : 0);
  const int H = a.H;
  const int bn_cols = (MODE == Mode::GateUp) ? BN / 2 : BN;
  const int nt_r = (MODE == Mode::GateUp) ? a.I / bn_cols : H / bn_cols;
  const int nt_s = has_shared ? ((MODE == Mode::GateUp) ? a.S / bn_cols : H / bn_cols) : 0;
  const int total = build_tile_prefix(prefix, a.counts, a.offsets, a.E, a.T, has_shared, BM, nt_r, nt_s,
                                      a.split);

  // Activation rows: as in the fp8 tile (instruction q covers 8 rows of 128 bytes).
  const int drow = lane >> 3;
  uint32_t dpiece[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) dpiece[h] = static_cast<uint32_t>(((lane & 7) ^ ((4 * h + (drow >> 1)) & 7)) * 16);
  // Weight rows: instruction q covers 16 rows of 64 bytes.
  const uint32_t wpiece = static_cast<uint32_t>(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(smem));
  const uint32_t sc0 = __builtin_amdgcn_readfirstlane(lds_address(&sscale[0][0]));
  const int r16 = lane & 15, g = lane >> 4;
  const uint32_t fsw = static_cast<uint32_t>((r16 >> 1) & 7);
  const uint32_t pc0 = (static_cast<uint32_t>(g) ^ fsw) * 16, pc1 = (static_cast<uint32_t>(4 + g) ^ fsw) * 16;
  const uint32_t pb = (static_cast<uint32_t>(g) ^ ((r16 >> 2) & 3)) * 16;

  const XcdWalk walk(total);
  for (int tile = walk.tile; tile < walk.end; tile += walk.step) {
    TileInfo t = find_tile(prefix, G, tile, a, BM, kBand);
    t.group = __builtin_amdgcn_readfirstlane(t.group);
    t.shared = __builtin_amdgcn_readfirstlane(static_cast<int>(t.shared)) != 0;
    t.rows = __builtin_amdgcn_readfirstlane(t.rows);
    t.rowbase = __builtin_amdgcn_readfirstlane(t.rowbase);
    t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
    t.nt = __builtin_amdgcn_readfirstlane(t.nt);
    const int kdim = (MODE == Mode::GateUp) ? H : (t.shared ? a.S : a.I);
    const int nk = kdim / kGroup;               // 128 elements per stage
    const int n0 = t.nt * bn_cols;
    const uint32_t krow = static_cast<uint32_t>(kdim);          // bytes per MXFP8 row
    const uint32_t wrow = static_cast<uint32_t>(kdim / 2);      // bytes per MXFP4 row
    const uint32_t srow = static_cast<uint32_t>(kdim / kMxBlock);   // E8M0 bytes per row
    const size_t hrow0 = t.shared ? static_cast<size_t>(a.h_shared) : static_cast<size_t>(t.rowbase) * kdim;

    // A rows of this wave: 32 wave + 8 q + lane / 8 (q < 4).
    i32x4_t ra, rsa;
    uint32_t aoff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = min(t.m0 + 32 * wave + 8 * q + drow, t.rows - 1);
      if constexpr (MODE == Mode::GateUp)
        aoff[q] = static_cast<uint32_t>(row_token(a, t, m)) * krow + dpiece[q & 1];
      else
        aoff[q] = static_cast<uint32_t>(m) * krow + dpiece[q & 1];
    }
    if constexpr (MODE == Mode::GateUp) {
      ra = dma_rsrc(a.xq, static_cast<uint32_t>(a.T) * krow);
      rsa = dma_rsrc(a.xe8, static_cast<uint32_t>(a.T) * srow);
    } else {
      ra = dma_rsrc(a.hq + hrow0, static_cast<uint32_t>(t.rows) * krow);
      rsa = dma_rsrc(a.he8 + hrow0 / kMxBlock, static_cast<uint32_t>(t.rows) * srow);
    }
    // B rows of this wave: tile rows [32 wave, +32) (gate/up: waves 0-3 gate rows,
    // 4-7 the up rows of the same h columns; down: output rows n0 + 32 wave ...).
    i32x4_t rb;
    uint32_t boff[2];
    {
      const uint8_t* wsrc;
      size_t erow;
      if constexpr (MODE == Mode::GateUp) {
        const bool up = wave >= 4;
        wsrc = static_cast<const uint8_t*>(t.shared ? (up ? a.ws_up : a.ws_gate) : (up ? a.w_up : a.w_gate));
        erow = (t.shared ? 0 : static_cast<size_t>(t.group) * a.I) + n0 + 32 * (wave & 3);
      } else {
        wsrc = static_cast<const uint8_t*>(t.shared ? a.ws_down : a.w_down);
        erow = (t.shared ? 0 : static_cast<size_t>(t.group) * H) + n0 + 32 * wave;
      }
      rb = dma_rsrc(wsrc + erow * wrow, 32 * wrow);
#pragma unroll
      for (int q = 0; q < 2; ++q) boff[q] = static_cast<uint32_t>(16 * q + (lane >> 2)) * wrow + wpiece;
    }
    // Down: the destinations of the wave's 64 output rows (lane l: row 64 wm + l),
    // loaded here and not touched before the epilogue (see the fp8 tile).
    int pre_slot = 0;
    float pre_w = 1.0f;
    if constexpr (MODE == Mode::Down) {
      const int m = min(t.m0 + wm * 64 + lane, t.rows - 1);
      pre_slot = a.perm[t.rowbase + m];
      if (t.shared) pre_w = a.shared_gate[m];
    }

    // Scale words this wave stages: waves 0-3 the activation rows [64 wave, +64);
    // waves 4-7 the weight rows [64 (wave - 4), +64) (gate/up: 4-5 gate, 6-7 up).
    i32x4_t rss;
    uint32_t ssoff, ssdst;
    if (wave < 4) {
      const int ms = min(t.m0 + 64 * wave + lane, t.rows - 1);
      rss = rsa;
      if constexpr (MODE == Mode::GateUp) ssoff = static_cast<uint32_t>(row_token(a, t, ms)) * srow;
      else ssoff = static_cast<uint32_t>(ms) * srow;
      ssdst = 64 * wave * 4;
    } else {
      const int bw = wave - 4;
      const uint8_t* ssrc;
      size_t erow;
      if constexpr (MODE == Mode::GateUp) {
        const bool up = bw >= 2;
        ssrc = t.shared ? (up ? a.e8s_up : a.e8s_gate) : (up ? a.e8_up : a.e8_gate);
        erow = (t.shared ? 0 : static_cast<size_t>(t.group) * a.I) + n0 + 64 * (bw & 1);
      } else {
        ssrc = t.shared ? a.e8s_down : a.e8_down;
        erow = (t.shared ? 0 : static_cast<size_t>(t.group) * H) + n0 + 64 * bw;
      }
      rss = dma_rsrc(ssrc + erow * srow, 64 * srow);
      ssoff = static_cast<uint32_t>(lane) * srow;
      ssdst = (BM + 64 * bw) * 4;
    }

    // Stage ks -> buffer ks % 3: A rows at [0, 32 KiB), B rows after; scales in sscale.
    auto issue = [&](int ks) {
      const int b = ks % kMxBufs;
      const uint32_t buf = lds0 + static_cast<uint32_t>(b) * kMxStage;
      dma4_rows(ra, aoff, static_cast<uint32_t>(ks) * kT4RowBytes, buf + 4 * wave * 1024);
      const uint32_t bbuf = buf + BM * kT4RowBytes + 32 * wave * kMxRowB;
      dma2_step(rb, boff, static_cast<uint32_t>(ks) * kMxRowB, 0, bbuf);   // rows 16 q + lane / 4
      const uint32_t sbuf = sc0 + static_cast<uint32_t>(b) * (BM + BN) * 4;
      dma1_dword(rss, ssoff, static_cast<uint32_t>(ks) * 4, sbuf + ssdst);
    };

    // Weight-row fragments are half the activation ones (64-byte rows), so each
    // wave takes more columns than rows: 4 row blocks x 8 column blocks (gate/up:
    // the gate rows of 64 h columns, then their up rows).
    auto brow = [&](int j) -> int {
      if constexpr (MODE == Mode::GateUp) return ((j < 4) ? 0 : BN / 2) + wn * 64 + 16 * (j & 3) + r16;
      else return wn * 128 + 16 * j + r16;
    };
    constexpr int NI = 4, NJ = 8;
    f32x4 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int ks) {
      const int b = ks % kMxBufs;
      const uint8_t* base = smem + b * kMxStage;
      const uint8_t* As = base + (wm * 64 + r16) * kT4RowBytes;
      const uint8_t* Bs = base + BM * kT4RowBytes;
      const uint32_t* sA = &sscale[b][wm * 64 + r16];
      const uint32_t* sB = &sscale[b][BM];
      i32x8 bf[NJ];
      int sb[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(Bs + brow(j) * kMxRowB + pb);
        bf[j] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        sb[j] = static_cast<int>((sB[brow(j)] >> (8 * g)) & 0xffu);
      }
      // Every scale word of the stage first (a word read just before its MFMAs
      // would stall them for the LDS latency), then the A fragments one row block
      // ahead of their MFMAs.
      uint32_t saw[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) saw[i] = sA[16 * i];
      auto afrag = [&](int i) {
        const uint8_t* row = As + i * 16 * kT4RowBytes;
        const uint4 lo = *reinterpret_cast<const uint4*>(row + pc0);
        const uint4 hi = *reinterpret_cast<const uint4*>(row + pc1);
        return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
      i32x8 af[2];
      af[0] = afrag(0);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (i + 1 < NI) af[(i + 1) & 1] = afrag(i + 1);
        const int sa = static_cast<int>((saw[i] >> (8 * g)) & 0xffu);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_mxfp8_mxfp4_16x16x128(af[i & 1], bf[j], acc[i][j], sa, sb[j]);
      }
    };

    // Stage ks: wait for this wave's part of it (stage ks + 1's instructions may
    // still be pending); barrier (every wave's part has landed and every wave is
    // done with stage ks - 1); start stage ks + 2 into the buffer stage ks - 1 used;
    // multiply stage ks.
    constexpr int kDmaPerStage = 4 + 2 + 1;
    __syncthreads();                   // the previous tile is done with every buffer
    issue(0);
    if (nk > 1) issue(1);
    for (int ks = 0; ks < nk; ++ks) {
      if (ks + 1 < nk) wait_vm<kDmaPerStage>();
      else wait_vm<0>();
      __syncthreads();
      if (ks + 2 < nk) issue(ks + 2);
      compute(ks);
    }

    // 16x16 output placement: lane l, element e -> row 4 (l / 16) + e, column l % 16.
    if constexpr (MODE == Mode::GateUp) {
      const int width = t.shared ? a.S : a.I;
      float* hbase = static_cast<float*>(a.h) +
                     (t.shared ? static_cast<size_t>(a.h_shared) : static_cast<size_t>(t.rowbase) * width);
      const int col0 = n0 + wn * 64 + r16;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = t.m0 + wm * 64 + 16 * i + 4 * g + e;
          if (m < t.rows) {
            float* hr = hbase + static_cast<size_t>(m) * width + col0;
#pragma unroll
            for (int jh = 0; jh < 4; ++jh) hr[16 * jh] = silu_f32(acc[i][jh][e]) * acc[i][jh + 4][e];
          }
        }
    } else {
      const int col0 = n0 + wn * 128 + r16;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + 4 * g + e;           // wave row
          const int m = t.m0 + wm * 64 + r;
          const int slot = __shfl(pre_slot, r, kWave);
          const float w = __shfl(pre_w, r, kWave);
          if (m < t.rows) {
            float* yr = (t.shared ? a.y + static_cast<size_t>(m) * a.H
                                  : a.o + static_cast<size_t>(slot_clamp(slot, a)) * a.H) + col0;
#pragma unroll
            for (int j = 0; j < NJ; ++j) yr[16 * j] = w * acc[i][j][e];
          }
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

// The 256-row kernels address operands with 32-bit buffer offsets: every
// activation matrix they read (x, or one group's rows of h) must stay below 4 GiB.
bool dma_offsets_fit(const ExpertArgs& a) {
  const int64_t widest = std::max<int64_t>(a.H, std::max(a.I, a.S));
  return static_cast<int64_t>(a.T) * widest * 2 < (int64_t{1} << 32);
}

}  // namespace

bool tall_tiles_fit(const ExpertArgs& a) { return dma_offsets_fit(a); }

hipError_t launch_gate_up_tall(const ExpertArgs& a, int weight_dtype, hipStream_t stream) {
  const int hcols = 128;              // h columns per tile (every weight format)
  const int grid = tiled_grid(a, 256, a.I / hcols, a.S / hcols);
  if (weight_dtype == kDtypeFp8) tiled8pp_expert_kernel<Mode::GateUp><<<grid, kF8PPThreads, 0, stream>>>(a);
  else if (weight_dtype == kDtypeMxfp4) tiledmx_expert_kernel<Mode::GateUp><<<grid, kF8PPThreads, 0, stream>>>(a);
  else tiledpp_expert_kernel<Mode::GateUp><<<grid, kPPThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_tall(const ExpertArgs& a, int weight_dtype, hipStream_t stream) {
  const int ycols = 256;              // output columns per tile (every weight format)
  const int grid = tiled_grid(a, 256, a.H / ycols, a.H / ycols);
  if (weight_dtype == kDtypeFp8) tiled8pp_expert_kernel<Mode::Down><<<grid, kF8PPThreads, 0, stream>>>(a);
  else if (weight_dtype == kDtypeMxfp4) tiledmx_expert_kernel<Mode::Down><<<grid, kF8PPThreads, 0, stream>>>(a);
  else tiledpp_expert_kernel<Mode::Down><<<grid, kPPThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace moe
