/*
 * moe_mi355x.h -- C ABI of the routed Mixture-of-Experts FFN forward for AMD
 * MI355X (gfx950).
 *
 * The layer (one call sequence per batch of T tokens):
 *   moe_route     router logits, softmax top-k with renormalisation, optional
 *                 cross-token expert budget, sigmoid shared-expert gate;
 *   moe_dispatch  per-expert counts, exclusive offsets, and the slot
 *                 permutation sorted by (expert, token);
 *   moe_forward   routed SwiGLU experts (grouped gate/up with fused SwiGLU, then
 *                 down with the gate-weighted combine) plus the shared expert.
 *
 * The problem statement is the pages' config keys: hidden size,
 * n_routed_experts, moe_intermediate_size, num_experts_per_tok, a shared
 * expert width [SpecForge PR #943, "Modifications"], the weight dtype, and an
 * expert budget [colibri issue_budget.md, "TL;DR" and "How it works"].
 *
 * Conventions shared by every entry point:
 *   - Pointers marked (device) are device pointers; (host) are host pointers.
 *     The caller owns every buffer.  The library allocates nothing, keeps no
 *     mutable global state and caches nothing between calls, except the static
 *     scratch of moe_forward_noalloc (one array per GPU, held from module load to
 *     process exit) and that array's device address, looked up once per GPU.
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  Nothing synchronises with the host and nothing is copied
 *     device-to-host, so the calls may be captured into a HIP graph.
 *   - Row-major layouts; "[A, B]" means A rows of B contiguous elements.
 *   - Every argument is validated on the host before anything is launched.  The
 *     return value is MOE_OK (0) or a negative moe_status; on error nothing has
 *     been enqueued and no output has been touched.  No exception or abort
 *     crosses this boundary.  MOE_ERR_LAUNCH_FAILED reports a HIP launch error
 *     (earlier launches of the same call may already be enqueued).
 *   - T = 0 is valid: moe_route and moe_forward* then return MOE_OK without
 *     reading any pointer but cfg and enqueue nothing; moe_dispatch writes zero
 *     counts and offsets (topk_ids and perm may be NULL).
 *   - Tile override, for benchmarks and tests only: the environment variable
 *     MOE_FORCE_TILE, read on every moe_forward / moe_forward_gate_up /
 *     moe_forward_down call (nothing is cached), forces the expert kernels' tile
 *     family.  Unset, empty or "auto": the per-call choice from the rows per expert
 *     (the small-M / large-M family choice of [DeepGEMM fork PR #5, "Dynamic
 *     family selection"]).  "stream16", "stream32", "stream64", "stream128": the
 *     weight-streaming kernel alone with tiles of that many token rows.  "split":
 *     the rows divided by the realised counts between the 256-row LDS-tiled kernel
 *     and the streaming kernel.  Any other value, or a value the configuration
 *     cannot use (F32 weights), returns MOE_ERR_BAD_SHAPE before anything is
 *     launched, as invalid
 *     overrides fail loudly in [DeepGEMM PR #381, "Forced-wave calibration"].
 *     Every setting computes the same y up to float32 summation order.
 *   - Supported dtype combinations (weight_dtype / act_dtype):
 *       F32 / F32, BF16 / BF16, FP8_E4M3_G128 / BF16, MXFP4 / BF16.
 *     With BF16 or FP8 weights, hidden_size, moe_intermediate_size and
 *     shared_expert_intermediate_size must be multiples of 128, with MXFP4
 *     weights multiples of 256 (MOE_ERR_UNSUPPORTED otherwise).  1 <= n_routed_experts <= 512,
 *     1 <= num_experts_per_tok <= min(n_routed_experts, 16).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL_PTR = -1,            /* a required pointer is NULL                  */
  MOE_ERR_BAD_SHAPE = -2,           /* a size is out of range                      */
  MOE_ERR_BAD_DTYPE = -3,           /* unknown dtype or unsupported combination    */
  MOE_ERR_UNSUPPORTED = -4,         /* valid but not implemented (alignment, E>512) */
  MOE_ERR_WORKSPACE_TOO_SMALL = -5, /* ws_bytes < moe_workspace_size(...)          */
  MOE_ERR_LAUNCH_FAILED = -6,       /* a HIP launch reported an error              */
  MOE_ERR_SCRATCH_TOO_SMALL = -7    /* moe_forward_noalloc: the call needs more
                                       workspace than its static scratch holds    */
} moe_status;

typedef enum moe_dtype {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1,
  /* OCP FP8 E4M3 ("e4m3fn": bias 7, max 448, no inf) codes, one byte each, with a
   * float32 scale per output row and per group of 128 consecutive elements of the
   * contraction dimension: w = decode(q) * s.  Activations that meet these
   * weights in a contraction are quantised the same way inside the kernels,
   * per token row and 128-group: s = amax/448 (s = 1 if amax = 0),
   * q = RNE(clamp(v/s, +-448)).  Group-128 scaling follows [colibri
   * issue_budget.md, header notes on issue_grouped_quant.md]; the fp8 x fp8
   * expert contraction follows the W8A8 MoE path that [DeepGEMM fork PR #5,
   * "Performance"] compares against. */
  MOE_DTYPE_FP8_E4M3_G128 = 2,
  /* OCP MX (microscaling v1.0) MXFP4 weights: E2M1 codes (sign, 2 exponent bits
   * with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte along
   * the contraction dimension (element 2i in the low nibble), and one E8M0 scale
   * byte (2^(e-127)) per 32 consecutive contraction elements: w = decode(q) * 2^(e-127).
   * Activations (BF16 x) that meet these weights in a contraction are quantised
   * inside the kernels to MXFP8, per token row and 32-element block: shared
   * exponent s = floor(log2(amax)) - 8 clamped to [-127, 127] (s = 0 if amax =
   * 0), element = RNE(clamp(v / 2^s, +-448)) as E4M3; the contraction applies both
   * block scales in the matrix cores.  The 4-bit group-scaled weights are what
   * the pages point to for the decode-bound layers (NVFP4 and FP8 x FP4 in
   * [DeepGEMM fork PR #5] and [DeepGEMM PR #381]). */
  MOE_DTYPE_MXFP4 = 3
} moe_dtype;

typedef struct moe_config {
  int32_t hidden_size;                     /* H                                             */
  int32_t n_routed_experts;                /* E, 1..512                                     */
  int32_t moe_intermediate_size;           /* I, width of each routed expert                */
  int32_t num_experts_per_tok;             /* K, 1..min(E,16)                               */
  int32_t shared_expert_intermediate_size; /* S, 0 = no shared expert                        */
  int32_t weight_dtype;                    /* moe_dtype of routed and shared expert weights  */
  int32_t act_dtype;                       /* moe_dtype of x, w_router, w_shared_gate        */
  int32_t norm_topk_prob;                  /* 1: renormalise the kept top-k weights to sum 1 */
  int32_t expert_budget;                   /* B >= 0, 0 = off: cap on distinct routed experts
                                              over the whole batch [colibri issue_budget.md] */
  float top_p;                             /* 0 <= p <= 1, 0 or 1 = off: per-token trim of the
                                              top-k to its top-p mass before the budget
                                              [colibri issue_budget.md, "Relationship to
                                              existing features"] */
} moe_config;

/* Expert weights, all (device).  The contraction dimension is contiguous.
 *   w_gate, w_up   [E, I, H]      w_down [E, H, I]
 *   s_gate, s_up   [E, I, H/128]  s_down [E, H, I/128]   (FP8 only, else NULL)
 *   ws_gate, ws_up [S, H]         ws_down [H, S]         (S > 0 only, else NULL)
 *   ss_gate, ss_up [S, H/128]     ss_down [H, S/128]     (FP8 and S > 0 only)
 * Element type is weight_dtype (one byte per element for FP8, half a byte for
 * MXFP4: the last dimension of w_* holds K/2 bytes).  Scales: float32 for FP8;
 * for MXFP4 uint8 E8M0 codes with K/32 per row in place of K/128
 * (s_gate [E, I, H/32], s_down [E, H, I/32], ss_* likewise). */
typedef struct moe_expert_weights {
  const void *w_gate, *w_up, *w_down;
  const void *s_gate, *s_up, *s_down;
  const void *ws_gate, *ws_up, *ws_down;
  const void *ss_gate, *ss_up, *ss_down;
} moe_expert_weights;

/* Bytes of device workspace needed by moe_route / moe_dispatch / moe_forward for
 * any T <= max_tokens.  One workspace may be reused by consecutive calls on one
 * stream; moe_forward_gate_up and moe_forward_down must see the same workspace
 * (the intermediate activations live there).  bytes: (host) out. */
int moe_workspace_size(const moe_config* cfg, int32_t max_tokens, size_t* bytes);

/* Router: logits z[t,e] = x_t . w_router[e] (+ logit_bias[t,e]) accumulated in
 * float32; softmax over the E experts, keep the K largest (ties: lower expert
 * id), renormalise them to sum 1 if norm_topk_prob [SpecForge PR #943,
 * "Modifications": softmax, renormalised top-k]; then, if 0 < top_p < 1, trim
 * each token to the shortest prefix of its picks (by descending probability)
 * whose summed probability reaches top_p times the summed probability of all K
 * picks, and renormalise the kept ones if norm_topk_prob [colibri
 * issue_budget.md, "Relationship to existing features": the per-position trim
 * runs before the budget]; then, if expert_budget > 0 and
 * the batch uses more than B distinct experts, keep the B experts with the
 * largest summed weight (ties: lower id), drop the other slots and renormalise
 * each token's kept weights [colibri issue_budget.md, "How it works" steps 1-5].
 *   x            (device) [T, H] act_dtype
 *   w_router     (device) [E, H] act_dtype
 *   w_shared_gate(device) [H] act_dtype; required iff S > 0, else ignored
 *   logit_bias   (device) [T, E] float32 or NULL (added to the logits).  An entry
 *                may be -inf to mask an expert for a token; a NaN logit counts as
 *                -inf.  Masked experts are still picked (after every finite one,
 *                lower id first) when fewer than K are finite, each at most once,
 *                with weight 0; a token whose logits are all -inf gets NaN weights.
 *                +inf is not allowed (its weights would be NaN).
 *   topk_ids     (device) out [T, K] int32, by descending weight; dropped slots
 *                are moved to the end of their row as id -1
 *   topk_weights (device) out [T, K] float32; 0 for dropped slots
 *   shared_gate  (device) out [T] float32 sigmoid(x_t . w_shared_gate); required
 *                iff S > 0, else ignored
 *   route_stats  (device) out int32[4] or NULL: {distinct experts before the
 *                budget, after, dropped slots, tokens left with no expert}
 * A token that loses every expert to the budget keeps ids -1 / weights 0.  The
 * top-p trim always keeps the first pick; its dropped slots are id -1 / weight 0
 * at the end of the row and are not counted in route_stats. */
int moe_route(const moe_config* cfg, int32_t num_tokens, const void* x, const void* w_router,
              const void* w_shared_gate, const float* logit_bias, int32_t* topk_ids,
              float* topk_weights, float* shared_gate, int32_t* route_stats, void* workspace,
              size_t workspace_bytes, void* stream);

/* Dispatch: the token-to-expert grouping that a grouped GEMM over
 * expert-contiguous rows consumes ([SpecForge PR #943, "Modifications": grouped_mm
 * dispatch]; the per-expert counts are the received-token counters of [DeepGEMM
 * PR #381, description]).  expert_counts[e] = number of slots with id e;
 * expert_offsets = exclusive prefix sum of counts (E+1 entries, last = kept
 * slots); perm[offsets[e] + j] = t*K + k for the j-th token (ascending t) routed
 * to e.  Slots whose id lies outside [0, E) (-1: dropped) are skipped.  The ids of
 * one token must be distinct (moe_route guarantees it); with a repeated id some
 * entries of perm below offsets[E] stay unwritten.  Entries of perm past
 * offsets[E] are left untouched.
 *   topk_ids (device) [T, K] int32
 *   expert_counts (device) out [E], expert_offsets (device) out [E+1],
 *   perm (device) out [T*K] int32 */
int moe_dispatch(const moe_config* cfg, int32_t num_tokens, const int32_t* topk_ids,
                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Experts and combine: the routed SwiGLU experts weighted by the renormalised
 * top-k gates, plus the sigmoid-gated shared expert [SpecForge PR #943,
 * "Modifications": shared expert (2048, sigmoid-gated), softmax renormalised
 * top-k; the expert FFN shape of its parameter counts, 3 * H * I per expert]:
 *   y[t,:] = sum_k topk_weights[t,k] * down_e(silu(gate_e x_t) * up_e x_t)
 *          + shared_gate[t] * down_s(silu(gate_s x_t) * up_s x_t)
 * with e = topk_ids[t,k], taken through the dispatch outputs.  A slot that the
 * dispatch skipped (id -1, or outside [0, E)) must have topk_weights 0, as
 * moe_route writes it: its row of the per-slot outputs is never computed, and a
 * non-zero weight would add that row's stale contents to y.  y (device) out
 * [T, H] float32, 16-byte aligned, overwritten.  The intermediate activations
 * are stored in the workspace as bf16 (BF16 weights), float32 (F32), e4m3 +
 * group-128 scales (FP8) or MXFP8 codes + E8M0 block-32 scales (MXFP4; x is
 * quantised the same way).  Accumulation is float32.  Each routed slot's
 * down-projection row is kept in the workspace and the slots of a token are
 * added to y in slot order after the shared term, so y is bit-reproducible
 * (no atomics).  Slots with weight 0 (dropped by the budget) are skipped.
 * y_act (device) out [T, H] or NULL: the optional cast of y to the activation
 * dtype, for a caller whose next layer takes activations in that dtype.  BF16
 * activations: y rounded to bfloat16 to nearest, ties to even (NaN stays NaN);
 * F32 activations: a copy of y.  Written from the same float32 values as y, in
 * the same pass; y itself stays float32 (the layer's result is defined before
 * any rounding).  y_act must be aligned to its element size
 * (MOE_ERR_UNSUPPORTED otherwise).  Size limit: x (T * H activations) and the
 * intermediate activations ((T * K * I + T * S) elements, 2 bytes each with BF16
 * weights, else 4) must each stay below 3 GiB (MOE_ERR_UNSUPPORTED otherwise);
 * the kernels address them with 32-bit offsets. */
int moe_forward(const moe_config* cfg, int32_t num_tokens, const void* x,
                const float* topk_weights, const float* shared_gate,
                const int32_t* expert_counts, const int32_t* expert_offsets, const int32_t* perm,
                const moe_expert_weights* weights /* (host) struct of (device) pointers */,
                float* y, void* y_act, void* workspace, size_t workspace_bytes, void* stream);

/* The two halves of moe_forward, same arguments, for callers that time or
 * overlap them: gate_up writes the intermediate activations to the workspace
 * (y and y_act are not touched); down reads them, writes the per-slot outputs to
 * the workspace and then y (and y_act if not NULL).  Calling gate_up then down
 * on one stream with one workspace equals moe_forward. */
int moe_forward_gate_up(const moe_config* cfg, int32_t num_tokens, const void* x,
                        const float* topk_weights, const float* shared_gate,
                        const int32_t* expert_counts, const int32_t* expert_offsets,
                        const int32_t* perm, const moe_expert_weights* weights, float* y,
                        void* y_act, void* workspace, size_t workspace_bytes, void* stream);
int moe_forward_down(const moe_config* cfg, int32_t num_tokens, const void* x,
                     const float* topk_weights, const float* shared_gate,
                     const int32_t* expert_counts, const int32_t* expert_offsets,
                     const int32_t* perm, const moe_expert_weights* weights, float* y,
                     void* y_act, void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, checks, kernels and result as moe_forward,
 * which it calls with a static scratch in place of the workspace: a file-scope
 * device array of 64 MiB that each GPU the library runs on holds from module load
 * until the process ends.  Its device address is looked up with
 * hipGetSymbolAddress on the first call on each GPU (with that GPU current) and
 * kept; nothing is allocated and nothing is freed, ever.  A call whose
 * moe_workspace_size(cfg, T) exceeds 64 MiB returns MOE_ERR_SCRATCH_TOO_SMALL
 * before anything is launched (the drafter layer at T = 224 needs ~12 MiB, the
 * 512 x 512 top-10 layer ~50 MiB).  Every call on one GPU shares that GPU's
 * scratch, which keeps the last call's contents; no kernel needs it zeroed.
 * Calls that overlap on one GPU (on different streams, or from different host
 * threads without ordering) race on it: serialise them. */
int moe_forward_noalloc(const moe_config* cfg, int32_t num_tokens, const void* x,
                        const float* topk_weights, const float* shared_gate,
                        const int32_t* expert_counts, const int32_t* expert_offsets,
                        const int32_t* perm, const moe_expert_weights* weights, float* y,
                        void* y_act, void* stream);

/* Static description of a status code (never NULL). */
const char* moe_status_string(int status);

/* Library version, e.g. 0x000100 = 0.1.0. */
int moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
