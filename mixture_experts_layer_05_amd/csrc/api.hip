// C ABI: argument validation, workspace layout, and the launches of each call.
// Everything is enqueued on the caller's stream; nothing is allocated, nothing is
// read back to the host.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "moe_mi355x.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
// From this many tokens the router logits run on the LDS-staged streaming kernel
// (64-token x 128-column tiles); below it, on 16-token x 32-column tiles whose
// waves split H, which spreads the router weights over more workgroups.
constexpr int32_t kRouterTiledTokens = 4096;
// Router contraction split for decode-sized batches (see moe_route).
constexpr int32_t kRouterPlaneTokens = 1024;
constexpr int kRouterParts = 8;
// Contraction parts of the LDS-staged router (T >= kRouterTiledTokens) when its
// columns fill whole 128-column tiles.
constexpr int kRouterStreamParts = 2;
// Upper bound (exclusive) on the byte size of x and of h; see check_forward.
constexpr int64_t kMaxActivationBytes = 3LL << 30;

bool valid_dtype(int d) {
  return d == MOE_DTYPE_F32 || d == MOE_DTYPE_BF16 || d == MOE_DTYPE_FP8_E4M3_G128 || d == MOE_DTYPE_MXFP4;
}
bool quantised_weights(int d) { return d == MOE_DTYPE_FP8_E4M3_G128 || d == MOE_DTYPE_MXFP4; }

// Shape and dtype checks shared by every entry point.
int check_config(const moe_config* c) {
  if (!c) return MOE_ERR_NULL_PTR;
  if (!valid_dtype(c->weight_dtype) || !valid_dtype(c->act_dtype)) return MOE_ERR_BAD_DTYPE;
  const bool combo = (c->weight_dtype == MOE_DTYPE_F32 && c->act_dtype == MOE_DTYPE_F32) ||
                     (c->weight_dtype == MOE_DTYPE_BF16 && c->act_dtype == MOE_DTYPE_BF16) ||
                     (c->weight_dtype == MOE_DTYPE_FP8_E4M3_G128 && c->act_dtype == MOE_DTYPE_BF16) ||
                     (c->weight_dtype == MOE_DTYPE_MXFP4 && c->act_dtype == MOE_DTYPE_BF16);
  if (!combo) return MOE_ERR_BAD_DTYPE;
  if (c->hidden_size <= 0 || c->moe_intermediate_size <= 0 || c->n_routed_experts <= 0 ||
      c->num_experts_per_tok <= 0 || c->shared_expert_intermediate_size < 0 || c->expert_budget < 0 ||
      (c->norm_topk_prob != 0 && c->norm_topk_prob != 1))
    return MOE_ERR_BAD_SHAPE;
  if (c->num_experts_per_tok > c->n_routed_experts) return MOE_ERR_BAD_SHAPE;
  if (!(c->top_p >= 0.f && c->top_p <= 1.f)) return MOE_ERR_BAD_SHAPE;   // also rejects NaN
  if (c->n_routed_experts > kMaxExperts || c->num_experts_per_tok > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (c->weight_dtype != MOE_DTYPE_F32) {
    // The expert kernels contract in whole stages: 128 elements, 256 with MXFP4.
    const int q = c->weight_dtype == MOE_DTYPE_MXFP4 ? 256 : 128;
    if (c->hidden_size % q || c->moe_intermediate_size % q || c->shared_expert_intermediate_size % q)
      return MOE_ERR_UNSUPPORTED;
  }
  // Index arithmetic is 32-bit inside the kernels for rows and slots.
  if (static_cast<int64_t>(c->hidden_size) * c->moe_intermediate_size > (1LL << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_tokens(const moe_config* c, int32_t T) {
  if (T < 0) return MOE_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(T) * c->num_experts_per_tok >= (1LL << 31) / 2) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct Layout {
  size_t z, h, o, xq, xs, hq, hs, chunks, ranks, bpart, bcount, gpart, gpart_bytes, total;
  int ldz;
  int64_t zrows;   // rows of z: T per logit plane
  size_t h_shared;  // element offset of the shared expert's rows in h
};

// Bytes of the partial gate/up sums that any call of at most T tokens needs (the
// largest contraction-split count times one part's floats over T' <= T, so the size
// is monotone in T).  A split needs fewer 64-column tiles than CUs, so beyond
// t_hi = 256 * 64 / (I K) tokens only a layer whose experts alone give fewer than
// 256 tiles can split; for those the bound 16 parts of the largest call is taken.
size_t gate_up_part_bytes(const moe_config& c, int64_t T) {
  const int K = std::max(c.num_experts_per_tok, 1), E = c.n_routed_experts;
  const int I = c.moe_intermediate_size, S = c.shared_expert_intermediate_size;
  const int64_t t_rho = int64_t{48} * E / K + 1;                   // rows per expert below 48
  const int64_t t_hi = ceil_div(int64_t{256} * 64, static_cast<int64_t>(std::max(I, 1)) * K);
  const bool few_tiles = static_cast<int64_t>(E) * (I / 64) < 256;
  const int64_t scan = std::min<int64_t>(T, few_tiles ? std::min<int64_t>(t_rho, 512) : std::min(t_rho, t_hi));
  size_t need = 0;
  for (int64_t t = 1; t <= scan; ++t) {
    const int p = gate_up_kparts(t, K, E, c.hidden_size, I, S, c.weight_dtype);
    if (p > 1) need = std::max(need, p * gate_up_part_floats(t, K, I, S));
  }
  if (few_tiles && std::min(T, t_rho) > scan) need = std::max(need, 16 * gate_up_part_floats(std::min(T, t_rho), K, I, S));
  return need * sizeof(float);
}

Layout layout(const moe_config& c, int64_t T) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = align_up(off + n, kAlign);
    return o;
  };
  const int E = c.n_routed_experts;
  L.ldz = static_cast<int>(align_up(E + 1, 16));
  // Logit planes: decode-sized batches (T <= kRouterPlaneTokens) split the router's
  // contraction over up to kRouterParts workgroups, each writing a partial plane.
  // From kRouterTiledTokens the LDS-staged router may write kRouterStreamParts
  // planes.  max(T or 2 T, kRouterParts * min(T, kRouterPlaneTokens)) rows keeps
  // the size monotone in T, so a workspace sized for max_tokens fits every
  // smaller call.
  const int64_t tplanes = T >= kRouterTiledTokens ? kRouterStreamParts : 1;
  L.zrows = std::max<int64_t>(tplanes * T,
                              static_cast<int64_t>(kRouterParts) * std::min<int64_t>(T, kRouterPlaneTokens));
  L.z = take(static_cast<size_t>(L.zrows) * L.ldz * sizeof(float));
  L.chunks = take(static_cast<size_t>(ceil_div(T, 1024)) * E * sizeof(int32_t));
  L.ranks = take(static_cast<size_t>(T) * c.num_experts_per_tok * sizeof(int32_t));
  // Expert budget: fixed-point aggregates and presence flags.
  L.bpart = take(static_cast<size_t>(E) * sizeof(unsigned long long));
  L.bcount = take(static_cast<size_t>(E) * sizeof(int32_t));
  const size_t routed = static_cast<size_t>(T) * c.num_experts_per_tok * c.moe_intermediate_size;
  const size_t elems = routed + static_cast<size_t>(T) * c.shared_expert_intermediate_size;
  L.h_shared = routed;
  const size_t hsize = (c.weight_dtype == MOE_DTYPE_BF16) ? 2 : 4;
  L.h = take(elems * hsize);
  L.o = take(static_cast<size_t>(T) * c.num_experts_per_tok * c.hidden_size * sizeof(float));
  L.gpart_bytes = gate_up_part_bytes(c, T);
  L.gpart = take(L.gpart_bytes);               // decode-sized calls' contraction split
  if (c.weight_dtype == MOE_DTYPE_FP8_E4M3_G128) {
    L.xq = take(static_cast<size_t>(T) * c.hidden_size);
    L.xs = take(static_cast<size_t>(T) * (c.hidden_size / kGroup) * sizeof(float));
    L.hq = take(elems);
    L.hs = take(elems / kGroup * sizeof(float));
  } else if (c.weight_dtype == MOE_DTYPE_MXFP4) {
    L.xq = take(static_cast<size_t>(T) * c.hidden_size);
    L.xs = take(static_cast<size_t>(T) * (c.hidden_size / kMxBlock));
    L.hq = take(elems);
    L.hs = take(elems / kMxBlock);
  }
  L.total = std::max<size_t>(off, kAlign);
  return L;
}

int check_workspace(const moe_config& c, int32_t T, const void* ws, size_t ws_bytes, Layout* L) {
  *L = layout(c, T);
  if (!ws) return MOE_ERR_NULL_PTR;
  if (ws_bytes < L->total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

int launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH_FAILED; }

// Returns MOE_OK for T = 0 without looking at any pointer (nothing is read or written).
// The optional activation-dtype output must be aligned to its element size.
int check_act_output(const moe_config& c, const void* y_act) {
  const uintptr_t size = c.act_dtype == MOE_DTYPE_BF16 ? 2 : 4;
  return (y_act && reinterpret_cast<uintptr_t>(y_act) % size != 0) ? MOE_ERR_UNSUPPORTED : MOE_OK;
}

// The tile override of the header's conventions: MOE_FORCE_TILE, read on every
// call.  Writes the kernels' setting (ExpertArgs::force_tile) or returns
// MOE_ERR_BAD_SHAPE for a value this configuration cannot use.
int tile_override(const moe_config& c, int* force) {
  *force = 0;
  const char* v = std::getenv("MOE_FORCE_TILE");
  if (!v || !*v || std::strcmp(v, "auto") == 0) return MOE_OK;
  if (c.weight_dtype == MOE_DTYPE_F32) return MOE_ERR_BAD_SHAPE;
  static const struct { const char* name; int rows; } kStream[] = {
      {"stream16", 16}, {"stream32", 32}, {"stream64", 64}, {"stream128", 128}};
  for (const auto& s : kStream)
    if (std::strcmp(v, s.name) == 0) {
      *force = s.rows;
      return MOE_OK;
    }
  if (std::strcmp(v, "split") == 0) {   // bf16, fp8 and MXFP4 (f32 returned above)
    *force = kForceSplit;
    return MOE_OK;
  }
  return MOE_ERR_BAD_SHAPE;
}

int check_forward(const moe_config* cfg, int32_t T, const void* x, const float* topk_w,
                  const float* shared_gate, const int32_t* counts, const int32_t* offsets,
                  const int32_t* perm, const moe_expert_weights* w, float* y) {
  int st = check_config(cfg);
  if (st) return st;
  if ((st = check_tokens(cfg, T))) return st;
  int force = 0;
  if ((st = tile_override(*cfg, &force))) return st;
  if (T == 0) return MOE_OK;
  // The expert kernels address x and h (per-slot activations) with 32-bit byte
  // offsets, and keep offsets from 3 GiB up free to mark rows that load zeros.
  const int64_t xbytes = static_cast<int64_t>(T) * cfg->hidden_size * (cfg->act_dtype == MOE_DTYPE_F32 ? 4 : 2);
  const int64_t hbytes = (static_cast<int64_t>(T) * cfg->num_experts_per_tok * cfg->moe_intermediate_size +
                          static_cast<int64_t>(T) * cfg->shared_expert_intermediate_size) *
                         (cfg->weight_dtype == MOE_DTYPE_BF16 ? 2 : 4);
  if (xbytes >= kMaxActivationBytes || hbytes >= kMaxActivationBytes) return MOE_ERR_UNSUPPORTED;
  if (!x || !topk_w || !counts || !offsets || !perm || !w || !y) return MOE_ERR_NULL_PTR;
  if (!w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_NULL_PTR;
  const bool fp8 = quantised_weights(cfg->weight_dtype);   // scales required
  if (fp8 && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_NULL_PTR;
  if (cfg->shared_expert_intermediate_size > 0) {
    if (!shared_gate || !w->ws_gate || !w->ws_up || !w->ws_down) return MOE_ERR_NULL_PTR;
    if (fp8 && (!w->ss_gate || !w->ss_up || !w->ss_down)) return MOE_ERR_NULL_PTR;
  }
  if (reinterpret_cast<uintptr_t>(y) % 16) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

ExpertArgs expert_args(const moe_config& c, int32_t T, const void* x, const float* topk_w,
                       const float* shared_gate, const int32_t* counts, const int32_t* offsets,
                       const int32_t* perm, const moe_expert_weights& w, float* y, void* ws,
                       const Layout& L) {
  ExpertArgs a{};
  a.x = x;
  a.counts = counts;
  a.offsets = offsets;
  a.perm = perm;
  a.topk_w = topk_w;
  a.shared_gate = shared_gate;
  a.w_gate = w.w_gate; a.w_up = w.w_up; a.w_down = w.w_down;
  a.ws_gate = w.ws_gate; a.ws_up = w.ws_up; a.ws_down = w.ws_down;
  a.h = at<void>(ws, L.h);
  a.h_shared = L.h_shared;
  if (c.weight_dtype == MOE_DTYPE_FP8_E4M3_G128) {
    a.s_gate = static_cast<const float*>(w.s_gate);
    a.s_up = static_cast<const float*>(w.s_up);
    a.s_down = static_cast<const float*>(w.s_down);
    a.ss_gate = static_cast<const float*>(w.ss_gate);
    a.ss_up = static_cast<const float*>(w.ss_up);
    a.ss_down = static_cast<const float*>(w.ss_down);
    a.xq = at<uint8_t>(ws, L.xq);
    a.xs = at<float>(ws, L.xs);
    a.hq = at<uint8_t>(ws, L.hq);
    a.hs = at<float>(ws, L.hs);
  } else if (c.weight_dtype == MOE_DTYPE_MXFP4) {
    a.e8_gate = static_cast<const uint8_t*>(w.s_gate);
    a.e8_up = static_cast<const uint8_t*>(w.s_up);
    a.e8_down = static_cast<const uint8_t*>(w.s_down);
    a.e8s_gate = static_cast<const uint8_t*>(w.ss_gate);
    a.e8s_up = static_cast<const uint8_t*>(w.ss_up);
    a.e8s_down = static_cast<const uint8_t*>(w.ss_down);
    a.xq = at<uint8_t>(ws, L.xq);
    a.xe8 = at<uint8_t>(ws, L.xs);
    a.hq = at<uint8_t>(ws, L.hq);
    a.he8 = at<uint8_t>(ws, L.hs);
  }
  a.o = at<float>(ws, L.o);
  a.split = 0;
  a.kparts = 1;   // the gate/up launcher sets the contraction split
  a.gpart = at<float>(ws, L.gpart);
  a.gpart_floats = L.gpart_bytes / sizeof(float);
  tile_override(c, &a.force_tile);   // validated by check_forward
  a.y = y;
  a.T = T;
  a.H = c.hidden_size;
  a.I = c.moe_intermediate_size;
  a.S = c.shared_expert_intermediate_size;
  a.E = c.n_routed_experts;
  a.K = c.num_experts_per_tok;
  return a;
}

// ---------------------------------------------------------------- static scratch
//
// The scratch of moe_forward_noalloc: a file-scope device array that every GPU the
// library runs on holds from module load until the process ends.  Its host-side
// name is not a device address; the address comes from hipGetSymbolAddress, once
// per device, with that device current.
constexpr size_t kScratchBytes = size_t{64} << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> scratch_ptr[kMaxDevices];

// The current device's scratch address, or nullptr with *status set on failure.
void* device_scratch(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = MOE_ERR_LAUNCH_FAILED;
    return nullptr;
  }
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    // Two threads may both look the address up; they store the same value.
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *status = MOE_ERR_LAUNCH_FAILED;
      return nullptr;
    }
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *status = MOE_OK;
  return p;
}

}  // namespace

extern "C" {

int moe_version(void) { return 0x000100; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_PTR: return "a required pointer is NULL";
    case MOE_ERR_BAD_SHAPE: return "a size is out of range";
    case MOE_ERR_BAD_DTYPE: return "unknown dtype or unsupported dtype combination";
    case MOE_ERR_UNSUPPORTED: return "configuration not supported (alignment or limits)";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than moe_workspace_size()";
    case MOE_ERR_LAUNCH_FAILED: return "a HIP kernel launch failed";
    case MOE_ERR_SCRATCH_TOO_SMALL:
      return "the call needs more workspace than the static scratch of moe_forward_noalloc holds";
    default: return "unknown status";
  }
}

int moe_workspace_size(const moe_config* cfg, int32_t max_tokens, size_t* bytes) {
  int st = check_config(cfg);
  if (st) return st;
  if (!bytes) return MOE_ERR_NULL_PTR;
  if ((st = check_tokens(cfg, max_tokens))) return st;
  *bytes = layout(*cfg, max_tokens).total;
  return MOE_OK;
}

int moe_route(const moe_config* cfg, int32_t T, const void* x, const void* w_router,
              const void* w_shared_gate, const float* logit_bias, int32_t* topk_ids, float* topk_w,
              float* shared_gate, int32_t* route_stats, void* ws, size_t ws_bytes, void* stream) {
  int st = check_config(cfg);
  if (st) return st;
  if ((st = check_tokens(cfg, T))) return st;
  const bool has_shared = cfg->shared_expert_intermediate_size > 0;
  if (T == 0) return MOE_OK;  // nothing is read or written
  if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_NULL_PTR;
  if (has_shared && (!w_shared_gate || !shared_gate)) return MOE_ERR_NULL_PTR;
  Layout L;
  if ((st = check_workspace(*cfg, T, ws, ws_bytes, &L))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = cfg->n_routed_experts, H = cfg->hidden_size, K = cfg->num_experts_per_tok;
  const int ncols = E + (has_shared ? 1 : 0);
  float* z = at<float>(ws, L.z);
  int parts = 1;                                            // logit planes written
  const size_t plane = static_cast<size_t>(T) * L.ldz;      // floats between planes
  // The LDS-staged router addresses x with 32-bit offsets (below 3 GiB).
  const bool x_fits = static_cast<int64_t>(T) * H * 2 < kMaxActivationBytes;
  if (cfg->act_dtype == MOE_DTYPE_BF16 && T >= kRouterTiledTokens && x_fits) {
    ExpertArgs r{};
    r.x = x;
    r.w_router = w_router;
    r.w_gcol = has_shared ? w_shared_gate : nullptr;
    r.z = z;
    r.ldz = L.ldz;
    r.ncols = ncols;
    r.T = T;
    r.H = H;
    r.E = E;
    // Split in two when the columns fill whole 128-column tiles and each part
    // keeps whole 128-element stages.
    if (ncols % 128 == 0 && H % (128 * kRouterStreamParts) == 0) parts = kRouterStreamParts;
    r.kparts = parts;
    r.zplane = plane;
    if ((st = launched(launch_router_stream(r, s)))) return st;
  } else if (cfg->act_dtype == MOE_DTYPE_BF16) {
    // Enough workgroups for ~256 CUs: split the hidden dimension into parts when
    // the token x column tiles alone are too few (at least 4 chunks of 128 per part).
    const int64_t tiles = ceil_div(T, 16) * ceil_div(ncols, 32);
    if (T <= kRouterPlaneTokens)
      parts = static_cast<int>(std::max<int64_t>(
          1, std::min<int64_t>({kRouterParts, ceil_div(256, tiles), (H / 128) / 4})));
    dim3 grid(static_cast<unsigned>(ceil_div(T, 16)), static_cast<unsigned>(ceil_div(ncols, 32)),
              static_cast<unsigned>(parts));
    router_logits_bf16_kernel<<<grid, 256, 0, s>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
        static_cast<const uint16_t*>(has_shared ? w_shared_gate : w_router), T, H, E, ncols, z, L.ldz,
        plane);
  } else {
    const int64_t items = static_cast<int64_t>(T) * ncols;
    router_logits_f32_kernel<<<static_cast<unsigned>(ceil_div(items, 4)), 256, 0, s>>>(
        static_cast<const float*>(x), static_cast<const float*>(w_router),
        static_cast<const float*>(has_shared ? w_shared_gate : w_router), T, H, E, ncols, z, L.ldz);
  }
  if ((st = launched(hipGetLastError()))) return st;
  const bool budget_pass = cfg->expert_budget > 0 || route_stats;
  unsigned long long* bagg = at<unsigned long long>(ws, L.bpart);
  int32_t* bpresent = at<int32_t>(ws, L.bcount);
  topk_kernel<<<static_cast<unsigned>(ceil_div(T, 4)), 256, 0, s>>>(
      z, L.ldz, parts, plane, logit_bias, T, E, K, cfg->norm_topk_prob,
      (cfg->top_p > 0.f && cfg->top_p < 1.f) ? cfg->top_p : 0.f, has_shared ? 1 : 0, topk_ids, topk_w,
      shared_gate, budget_pass ? bagg : nullptr, bpresent);
  if ((st = launched(hipGetLastError()))) return st;
  if (budget_pass) {
    const unsigned nchunks = static_cast<unsigned>(ceil_div(T, kBudgetChunkTokens));
    budget_aggregate_kernel<<<nchunks, kBudgetChunkTokens, 0, s>>>(topk_ids, topk_w, T, E, K, bagg, bpresent,
                                                                   route_stats);
    if ((st = launched(hipGetLastError()))) return st;
    // Without a budget only workgroup 0 runs (it writes the statistics).
    budget_apply_kernel<<<cfg->expert_budget > 0 ? nchunks : 1u, kBudgetChunkTokens, 0, s>>>(
        topk_ids, topk_w, T, E, K, cfg->expert_budget, cfg->norm_topk_prob, bagg, bpresent, route_stats);
    if ((st = launched(hipGetLastError()))) return st;
  }
  return MOE_OK;
}

int moe_dispatch(const moe_config* cfg, int32_t T, const int32_t* topk_ids, int32_t* counts,
                 int32_t* offsets, int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  int st = check_config(cfg);
  if (st) return st;
  if ((st = check_tokens(cfg, T))) return st;
  if (!counts || !offsets) return MOE_ERR_NULL_PTR;
  if (T > 0 && (!topk_ids || !perm)) return MOE_ERR_NULL_PTR;
  Layout L;
  if ((st = check_workspace(*cfg, T, ws, ws_bytes, &L))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = cfg->n_routed_experts, K = cfg->num_experts_per_tok;
  if (T <= 1024) {
    dispatch_kernel<<<1, 1024, 0, s>>>(topk_ids, T, E, K, counts, offsets, perm);
    return launched(hipGetLastError());
  }
  const int nchunks = static_cast<int>(ceil_div(T, 1024));
  int32_t* chunk = at<int32_t>(ws, L.chunks);
  int32_t* ranks = at<int32_t>(ws, L.ranks);
  dispatch_chunk_kernel<<<nchunks, 1024, 0, s>>>(topk_ids, T, E, K, chunk, ranks);
  if ((st = launched(hipGetLastError()))) return st;
  dispatch_scan_kernel<<<1, 1024, 0, s>>>(nchunks, E, chunk, counts, offsets);
  if ((st = launched(hipGetLastError()))) return st;
  const int64_t slots = static_cast<int64_t>(T) * K;
  dispatch_scatter_kernel<<<static_cast<unsigned>(std::min<int64_t>(ceil_div(slots, 256), 4096)), 256, 0, s>>>(
      topk_ids, T, E, K, chunk, ranks, perm);
  return launched(hipGetLastError());
}

int moe_forward_gate_up(const moe_config* cfg, int32_t T, const void* x, const float* topk_w,
                        const float* shared_gate, const int32_t* counts, const int32_t* offsets,
                        const int32_t* perm, const moe_expert_weights* w, float* y, void* y_act, void* ws,
                        size_t ws_bytes, void* stream) {
  (void)y_act;   // written by the down half only
  int st = check_forward(cfg, T, x, topk_w, shared_gate, counts, offsets, perm, w, y);
  if (st || T == 0) return st;
  Layout L;
  if ((st = check_workspace(*cfg, T, ws, ws_bytes, &L))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ExpertArgs a = expert_args(*cfg, T, x, topk_w, shared_gate, counts, offsets, perm, *w, y, ws, L);
  if (cfg->weight_dtype == MOE_DTYPE_FP8_E4M3_G128) {
    if ((st = launched(launch_quant_x(a, at<uint8_t>(ws, L.xq), at<float>(ws, L.xs), s)))) return st;
  } else if (cfg->weight_dtype == MOE_DTYPE_MXFP4) {
    if ((st = launched(launch_quant_x_mx(a, at<uint8_t>(ws, L.xq), at<uint8_t>(ws, L.xs), s)))) return st;
  }
  if ((st = launched(launch_gate_up(a, cfg->weight_dtype, s)))) return st;
  if (cfg->weight_dtype == MOE_DTYPE_FP8_E4M3_G128) {
    if ((st = launched(launch_quant_h(a, at<uint8_t>(ws, L.hq), at<float>(ws, L.hs), s)))) return st;
  } else if (cfg->weight_dtype == MOE_DTYPE_MXFP4) {
    if ((st = launched(launch_quant_h_mx(a, at<uint8_t>(ws, L.hq), at<uint8_t>(ws, L.hs), s)))) return st;
  }
  return MOE_OK;
}

int moe_forward_down(const moe_config* cfg, int32_t T, const void* x, const float* topk_w,
                     const float* shared_gate, const int32_t* counts, const int32_t* offsets,
                     const int32_t* perm, const moe_expert_weights* w, float* y, void* y_act, void* ws,
                     size_t ws_bytes, void* stream) {
  int st = check_forward(cfg, T, x, topk_w, shared_gate, counts, offsets, perm, w, y);
  if (st || T == 0) return st;
  if ((st = check_act_output(*cfg, y_act))) return st;
  Layout L;
  if ((st = check_workspace(*cfg, T, ws, ws_bytes, &L))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ExpertArgs a = expert_args(*cfg, T, x, topk_w, shared_gate, counts, offsets, perm, *w, y, ws, L);
  a.y_act = y_act;
  a.act_bf16 = cfg->act_dtype == MOE_DTYPE_BF16 ? 1 : 0;
  if ((st = launched(launch_down(a, cfg->weight_dtype, s)))) return st;
  return launched(launch_combine(a, s));
}

int moe_forward(const moe_config* cfg, int32_t T, const void* x, const float* topk_w,
                const float* shared_gate, const int32_t* counts, const int32_t* offsets,
                const int32_t* perm, const moe_expert_weights* w, float* y, void* y_act, void* ws,
                size_t ws_bytes, void* stream) {
  // Everything the down half checks is checked before the gate/up half launches.
  int st = check_forward(cfg, T, x, topk_w, shared_gate, counts, offsets, perm, w, y);
  if (st || T == 0) return st;
  if ((st = check_act_output(*cfg, y_act))) return st;
  st = moe_forward_gate_up(cfg, T, x, topk_w, shared_gate, counts, offsets, perm, w, y, y_act, ws,
                               ws_bytes, stream);
  if (st) return st;
  return moe_forward_down(cfg, T, x, topk_w, shared_gate, counts, offsets, perm, w, y, y_act, ws,
                          ws_bytes, stream);
}

int moe_forward_noalloc(const moe_config* cfg, int32_t T, const void* x, const float* topk_w,
                        const float* shared_gate, const int32_t* counts, const int32_t* offsets,
                        const int32_t* perm, const moe_expert_weights* w, float* y, void* y_act,
                        void* stream) {
  // Every check moe_forward makes, with the workspace checked against the static
  // scratch's size, before the scratch address is looked up or anything launched.
  int st = check_forward(cfg, T, x, topk_w, shared_gate, counts, offsets, perm, w, y);
  if (st || T == 0) return st;
  if ((st = check_act_output(*cfg, y_act))) return st;
  if (layout(*cfg, T).total > kScratchBytes) return MOE_ERR_SCRATCH_TOO_SMALL;
  void* ws = device_scratch(&st);
  if (!ws) return st;
  return moe_forward(cfg, T, x, topk_w, shared_gate, counts, offsets, perm, w, y, y_act, ws, kScratchBytes,
                     stream);
}

}  // extern "C"
