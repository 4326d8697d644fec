// Kernel declarations and the argument block shared by the expert kernels.
#pragma once

#include "common.h"

namespace moe {

// Everything an expert kernel may need.  Unused fields are null / zero.
//
// Down-projection outputs: a routed row (token t, slot k) is written, unweighted,
// to row t*K+k of o; shared-expert rows go straight to y, weighted by
// sigmoid(g_t).  A combine pass then adds the weighted slots of each token in
// slot order, so y is bit-reproducible and no atomics are needed.
//
// Intermediate activations h: routed rows first, in dispatch (perm) order,
// [T*K, I]; then the shared expert's rows [T, S] starting at element h_shared.
// With fp8 or MXFP4 weights h is kept in float32 and then quantised to hq with
// the same layout, its scales in hs (fp8: one float per 128 elements) or he8
// (MXFP8: one E8M0 byte per 32 elements).
struct ExpertArgs {
  const void* x;                 // [T, H] act dtype
  const int32_t* counts;         // [E]
  const int32_t* offsets;        // [E+1]
  const int32_t* perm;           // [T*K]
  const float* topk_w;           // [T, K]
  const float* shared_gate;      // [T]
  const void *w_gate, *w_up, *w_down;
  const float *s_gate, *s_up, *s_down;
  const void *ws_gate, *ws_up, *ws_down;
  const float *ss_gate, *ss_up, *ss_down;
  void* h;
  size_t h_shared;               // element offset of the shared rows in h / hq
  const uint8_t* xq;             // fp8: quantised x [T, H]
  const float* xs;               // fp8: scales [T, H/128]
  const uint8_t* hq;             // fp8: quantised h
  const float* hs;               // fp8: scales of h
  // MXFP4 weights (w_* / ws_* hold the packed E2M1 codes): E8M0 scale bytes, one
  // per 32 contraction elements; x and h quantised to MXFP8 codes in xq / hq with
  // E8M0 scales in xe8 [T, H/32] / he8 (one per 32 elements of h).
  const uint8_t *e8_gate, *e8_up, *e8_down, *e8s_gate, *e8s_up, *e8s_down;
  const uint8_t* xe8;
  const uint8_t* he8;
  float* o;                      // [T*K, H] unweighted routed outputs, row = slot t*K+k
  float* y;                      // [T, H]
  // Which of a call's rows this launch serves when the expert launchers divide
  // them between two kernels by the realised counts (0: all; see schedule.h).
  int split;
  // Tile override (host side only, from MOE_FORCE_TILE): 0 = the per-call choice;
  // 16, 32, 64 or 128 = the streaming kernel alone with tiles of that many rows;
  // kForceSplit = rows divided between the 256-row and the streaming kernels.
  int force_tile;
  // Contraction split of a gate/up streaming launch (1: none).  Each tile then
  // covers 1/kparts of the contraction and writes its raw gate and up sums,
  // float32, to part p of gpart (layout: gate_up_part_floats); a finishing pass
  // adds the parts in order p = 0, 1, ... and applies SwiGLU.
  int kparts;
  float* gpart;
  size_t gpart_floats;           // capacity of gpart: the launcher never splits beyond it
  void* y_act;                   // [T, H] act dtype or null: the cast of y
  int act_bf16;                  // y_act is bf16 (else float32)
  // Router logits (router mode of the streaming kernel): z[t, c] = x_t . col_c with
  // col_c = w_router[c] for c < E and col_E = w_gcol (the shared gate) if present.
  const void* w_router;          // [E, H]
  const void* w_gcol;            // [H] or null
  float* z;                      // [T, ldz]
  int ldz, ncols;
  size_t zplane;                 // floats between the logit planes of a split router launch
  int T, H, I, S, E, K;
};

constexpr int kForceSplit = -1;

// route.hip
__global__ void router_logits_bf16_kernel(const uint16_t*, const uint16_t*, const uint16_t*, int, int,
                                          int, int, float*, int, size_t);
__global__ void router_logits_f32_kernel(const float*, const float*, const float*, int, int, int, int,
                                         float*, int);
__global__ void topk_kernel(const float*, int, int, size_t, const float*, int, int, int, int, float, int,
                            int32_t*, float*, float*, unsigned long long*, int32_t*);
constexpr int kBudgetChunkTokens = 256;   // tokens (and threads) per workgroup of the budget passes
__global__ void budget_aggregate_kernel(const int32_t*, const float*, int, int, int, unsigned long long*, int32_t*,
                                        int32_t*);
__global__ void budget_apply_kernel(int32_t*, float*, int, int, int, int, int, const unsigned long long*,
                                    const int32_t*, int32_t*);

// dispatch.hip
__global__ void dispatch_kernel(const int32_t*, int, int, int, int32_t*, int32_t*, int32_t*);
__global__ void dispatch_chunk_kernel(const int32_t*, int, int, int, int32_t*, int32_t*);
__global__ void dispatch_scan_kernel(int, int, int32_t*, int32_t*, int32_t*);
__global__ void dispatch_scatter_kernel(const int32_t*, int, int, int, const int32_t*, const int32_t*,
                                        int32_t*);

// experts.hip: host-side launchers (they pick tile shapes and grid sizes).
hipError_t launch_gate_up(const ExpertArgs& a, int weight_dtype, hipStream_t stream);
// Whether the rows of a call may be divided between the 256-row LDS-tiled kernels
// and the streaming kernel (BF16 / FP8 weights whose operands the 256-row kernels
// can address).
bool split_allowed(const ExpertArgs& a, int weight_dtype);
hipError_t launch_down(const ExpertArgs& a, int weight_dtype, hipStream_t stream);
// 256-row LDS-tiled kernels (tile_gemm.hip); tall_tiles_fit: their 32-bit
// operand offsets cover the call's activation matrices.
bool tall_tiles_fit(const ExpertArgs& a);
hipError_t launch_gate_up_tall(const ExpertArgs& a, int weight_dtype, hipStream_t stream);
hipError_t launch_down_tall(const ExpertArgs& a, int weight_dtype, hipStream_t stream);
hipError_t launch_gate_up_stream(const ExpertArgs& a, int weight_dtype, int64_t rho, hipStream_t stream);
// Contraction parts of a call's gate/up streaming launch (1: unsplit; see
// stream_gemm.hip).
int gate_up_kparts(int64_t T, int K, int E, int H, int I, int S, int weight_dtype);
// Floats of one contraction part's partial sums: per routed dispatch row (T*K
// rows) 2*I values, the I gate sums then the I up sums; then per shared-expert row
// (T rows) 2*S values.
__host__ __device__ inline size_t gate_up_part_floats(int64_t T, int K, int I, int S) {
  return static_cast<size_t>(T) * K * 2 * I + static_cast<size_t>(T) * 2 * S;
}
hipError_t launch_down_stream(const ExpertArgs& a, int weight_dtype, int64_t rho, hipStream_t stream);
hipError_t launch_combine(const ExpertArgs& a, hipStream_t stream);
hipError_t launch_router_stream(const ExpertArgs& a, hipStream_t stream);
hipError_t launch_quant_x(const ExpertArgs& a, uint8_t* xq, float* xs, hipStream_t stream);
hipError_t launch_quant_h(const ExpertArgs& a, uint8_t* hq, float* hs, hipStream_t stream);
hipError_t launch_quant_x_mx(const ExpertArgs& a, uint8_t* xq, uint8_t* xe8, hipStream_t stream);
hipError_t launch_quant_h_mx(const ExpertArgs& a, uint8_t* hq, uint8_t* he8, hipStream_t stream);

}  // namespace moe
