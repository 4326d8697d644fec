"""Seeded synthetic inputs for the routed MoE FFN forward.

This module only draws random numbers and lays them out. It holds none of the
layer's arithmetic (no logits, no top-k, no dispatch, no expert math), so both
the CPU oracle (through the tests) and the HIP path can be fed from it without
sharing any of the method.

Workloads follow the shapes the pages measure:
  * tiny fp32 layer (hidden 256, 8 experts x 512, top-2), the oracle's quick case;
  * the 16 x 1024 top-2 drafter with a 2048-wide sigmoid-gated shared expert
    [SpecForge PR #943, "Modifications" and "End-to-end serving speed"], at
    7-token speculative blocks x concurrency 1/8/32;
  * the 512 x 512 top-10 drafter with the same shared expert, uniformly routed
    ("routing is uniform = worst case for expert bytes", same page, "Modifications");
  * the 256-expert top-8 hidden-7168 / intermediate-2048 layer with a Zipf
    router skew [DeepGEMM PR #381, "Validation" and the block_m note];
  * the same layer with fp8 e4m3 weights, group-128 scales and an expert budget of
    64 [colibri issue_budget.md, "How it works"].

Every tensor is produced on the CPU by ``torch.Generator`` seeded from
(base seed, tensor sub-seed), so any single expert can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

GROUP = 128  # quantisation group along the contraction dimension

DT_F32, DT_BF16, DT_FP8, DT_MXFP4 = "f32", "bf16", "fp8_e4m3_g128", "mxfp4"
MX_BLOCK = 32
# MXFP4 test weights: E8M0 scale codes drawn from [lo, hi] (2^-8 .. 2^-6); with
# uniform E2M1 codes the element standard deviation is ~0.02, like the others.
MX_SCALE_CODES = (119, 121)

_TORCH_ACT = {DT_F32: torch.float32, DT_BF16: torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Problem statement of one MoE FFN layer, named as the pages' config keys."""
    name: str
    hidden_size: int                  # H
    n_routed_experts: int             # E
    moe_intermediate_size: int        # I
    num_experts_per_tok: int          # K
    shared_expert_intermediate_size: int  # S, 0 = no shared expert
    weight_dtype: str                 # f32 / bf16 / fp8_e4m3_g128
    act_dtype: str                    # f32 / bf16
    norm_topk_prob: int = 1
    expert_budget: int = 0            # B, 0 = off
    top_p: float = 0.0                # per-token top-p trim of the top-k, 0 = off
    block_bias: bool = False          # router bias shared per 7-token block (the drafter family)
    weight_std: float = 0.02
    x_std: float = 1.0
    router_std: Optional[float] = None  # default 1/sqrt(H)

    @property
    def r_std(self) -> float:
        return self.router_std if self.router_std is not None else 1.0 / math.sqrt(self.hidden_size)

    def with_(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


# The five workloads (index order matters: the fp8 + budget case reuses index 3's shape).
TINY = LayerShape("tiny_fp32", 256, 8, 512, 2, 0, DT_F32, DT_F32,
                  weight_std=0.02, x_std=0.02, router_std=0.02)
DRAFTER = LayerShape("drafter_16x1024_top2_shared2048", 5120, 16, 1024, 2, 2048, DT_BF16, DT_BF16,
                     block_bias=True)
NARROW = LayerShape("narrow_512x512_top10_shared2048", 5120, 512, 512, 10, 2048, DT_BF16, DT_BF16)
LARGE = LayerShape("large_256x2048_top8_h7168", 7168, 256, 2048, 8, 0, DT_BF16, DT_BF16)
LARGE_FP8 = LARGE.with_(name="large_fp8_budget64", weight_dtype=DT_FP8, expert_budget=64)
# 4-bit (MXFP4) expert weights on the decode-bound layers [the 4-bit group-scaled
# weights the pages point to for decode]: same shapes, synthetic MXFP4 codes.
DRAFTER_MX4 = DRAFTER.with_(name="drafter_mxfp4", weight_dtype=DT_MXFP4)
# The decode layers with fp8 e4m3 group-128 weights (no budget).
DRAFTER_FP8 = DRAFTER.with_(name="drafter_fp8", weight_dtype=DT_FP8)
NARROW_FP8 = NARROW.with_(name="narrow_fp8", weight_dtype=DT_FP8)
NARROW_MX4 = NARROW.with_(name="narrow_mxfp4", weight_dtype=DT_MXFP4)
LARGE_MX4 = LARGE.with_(name="large_mxfp4", weight_dtype=DT_MXFP4)

# One GPU's share of the large layer sharded over 8 GPUs by experts: rank r
# holds experts [32r, 32r + 32) of the 256 (H 7168, I 2048) and receives, for a
# 4096-token batch (512 tokens per rank x 8 ranks), every (token, slot) of the
# global top-8 routing whose expert is one of its own.  Its problem is this
# 32-expert layer with K = 8 slots per token, local id = global id - 32r, the
# non-local slots marked -1 (weight 0).  The ids come from routing the global
# layer (LARGE inputs); the caller picks the rank that receives the most slots,
# which sets the step time of an expert-parallel layer.
EP_RANK_LOCAL = 32
EP_RANKS = 8
EP_RANK = LARGE.with_(name="ep_rank_32of256x2048_top8_h7168", n_routed_experts=EP_RANK_LOCAL)

SHAPES = [TINY, DRAFTER, NARROW, LARGE, LARGE_FP8, EP_RANK]

TOKENS = {
    TINY.name: (64,),
    DRAFTER.name: (7, 56, 224),       # 7-token block x concurrency 1 / 8 / 32
    NARROW.name: (7, 56, 224),
    LARGE.name: (512, 2048, 8192),
    LARGE_FP8.name: (8192,),
    EP_RANK.name: (4096,),
}
ALPHAS = {LARGE.name: (0.0, 1.0, 1.5), LARGE_FP8.name: (1.5,), EP_RANK.name: (1.5,)}

DRAFT_BLOCK = 7                        # speculative block size
DRAFTER_BIAS_SCALES = (0.0, 1.0, 2.0, 4.0, 8.0)  # per-block bias scale choices

# Sub-seeds per tensor family.
_SUB_X, _SUB_ROUTER, _SUB_SHARED_GATE, _SUB_SHARED, _SUB_BIAS, _SUB_EXPERT = 1, 2, 3, 5, 6, 10


def base_seed(shape_index: int, T: int) -> int:
    return 1000 * shape_index + T


def _gen(*key: int, device="cpu") -> torch.Generator:
    # Fold an integer tuple into one 63-bit seed (hash-combine of the parts).
    h = 0x9E3779B97F4A7C15
    for k in key:
        h ^= (int(k) + 0x9E3779B97F4A7C15 + ((h << 6) & 0xFFFFFFFFFFFFFFFF) + (h >> 2)) & 0xFFFFFFFFFFFFFFFF
        h &= 0xFFFFFFFFFFFFFFFF
    return torch.Generator(device=device).manual_seed(h & 0x7FFFFFFFFFFFFFFF)


def _normal(shape, std: float, g: torch.Generator) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=g.device) * std


def act_torch_dtype(shape: LayerShape) -> torch.dtype:
    return _TORCH_ACT[shape.act_dtype]


# ----------------------------------------------------------------------------- activations

def tokens(shape: LayerShape, seed: int, T: int) -> torch.Tensor:
    """x [T, H] in the activation dtype."""
    x = _normal((T, shape.hidden_size), shape.x_std, _gen(seed, _SUB_X))
    return x.to(act_torch_dtype(shape))


def token_row(shape: LayerShape, seed: int, t: int, attempt: int) -> torch.Tensor:
    """A fresh draw for row t of x (used to re-draw rows whose routing is too close to a tie)."""
    x = _normal((shape.hidden_size,), shape.x_std, _gen(seed, _SUB_X, t, attempt))
    return x.to(act_torch_dtype(shape))


def router_weight(shape: LayerShape, seed: int) -> torch.Tensor:
    """W_r [E, H] in the activation dtype."""
    w = _normal((shape.n_routed_experts, shape.hidden_size), shape.r_std, _gen(seed, _SUB_ROUTER))
    return w.to(act_torch_dtype(shape))


def shared_gate_weight(shape: LayerShape, seed: int) -> Optional[torch.Tensor]:
    """w_g [H] in the activation dtype (None without a shared expert)."""
    if shape.shared_expert_intermediate_size == 0:
        return None
    w = _normal((shape.hidden_size,), 1.0 / math.sqrt(shape.hidden_size), _gen(seed, _SUB_SHARED_GATE))
    return w.to(act_torch_dtype(shape))


# ----------------------------------------------------------------------------- router biases

def drafter_block_bias(shape: LayerShape, seed: int, T: int) -> torch.Tensor:
    """Per-token logit bias shared inside each 7-token block: b[t,e] = s_blk * g[blk, e].

    g ~ N(0,1) per block and expert; s_blk is drawn per block from
    DRAFTER_BIAS_SCALES, so blocks range from nearly uniform routing to strongly
    concentrated routing (2..14 distinct experts of 16 under top-2).
    """
    g = _gen(seed, _SUB_BIAS)
    nblk = (T + DRAFT_BLOCK - 1) // DRAFT_BLOCK
    gb = torch.randn(nblk, shape.n_routed_experts, generator=g, dtype=torch.float32)
    pick = torch.randint(0, len(DRAFTER_BIAS_SCALES), (nblk,), generator=g)
    s = torch.tensor(DRAFTER_BIAS_SCALES, dtype=torch.float32)[pick]
    b = (gb * s[:, None]).repeat_interleave(DRAFT_BLOCK, dim=0)[:T]
    return b.contiguous()


def zipf_rank_bias(shape: LayerShape, seed: int, T: int, alpha: float, attempt: int = 0) -> torch.Tensor:
    """b[t,e] = alpha * log(Zipf pmf at rank_e) up to a constant = -alpha * ln(rank_e).

    rank is a seeded permutation of 1..E (the hot expert is not always expert 0).
    The Zipf normaliser is a per-token constant and is left out.
    """
    g = _gen(seed, _SUB_BIAS, attempt)
    rank = torch.randperm(shape.n_routed_experts, generator=g).to(torch.float64) + 1.0
    b = (-alpha * torch.log(rank)).to(torch.float32)
    return b[None, :].expand(T, shape.n_routed_experts).contiguous()


# ----------------------------------------------------------------------------- expert weights

def _quantise_rows_g128(w: torch.Tensor):
    """fp32 [N, Kc] -> (e4m3fn codes [N, Kc] as uint8, fp32 scales [N, Kc/128]).

    Used only to *make* fp8 test weights: scale = amax/448 per (row, 128-group),
    codes from torch's own float8_e4m3fn conversion.  The layer consumes these as
    given inputs.
    """
    n, kc = w.shape
    wg = w.reshape(n, kc // GROUP, GROUP)
    amax = wg.abs().amax(dim=2)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (wg / s[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.reshape(n, kc).view(torch.uint8), s.to(torch.float32).contiguous()


def expert_weights(shape: LayerShape, seed: int, e: int, device="cpu") -> Dict[str, torch.Tensor]:
    """Weights of routed expert e.

    gate, up: [I, H]; down: [H, I] (contraction dim contiguous).  For fp8 also
    the group-128 scales gate_s/up_s [I, H/128], down_s [H, I/128].  The numbers
    depend on the device's generator (CPU and GPU draws differ), never on anything else.
    """
    H, I = shape.hidden_size, shape.moe_intermediate_size
    g = _gen(seed, _SUB_EXPERT, e, device=device)
    if shape.weight_dtype == DT_MXFP4:
        return _mx_random((I, H), (I, H), (H, I), g)
    wg = _normal((I, H), shape.weight_std, g)
    wu = _normal((I, H), shape.weight_std, g)
    wd = _normal((H, I), shape.weight_std, g)
    return _pack(shape, wg, wu, wd)


def shared_expert_weights(shape: LayerShape, seed: int, device="cpu") -> Optional[Dict[str, torch.Tensor]]:
    """Shared expert: gate, up [S, H]; down [H, S] (+ scales for fp8)."""
    S, H = shape.shared_expert_intermediate_size, shape.hidden_size
    if S == 0:
        return None
    g = _gen(seed, _SUB_SHARED, device=device)
    if shape.weight_dtype == DT_MXFP4:
        return _mx_random((S, H), (S, H), (H, S), g)
    wg = _normal((S, H), shape.weight_std, g)
    wu = _normal((S, H), shape.weight_std, g)
    wd = _normal((H, S), shape.weight_std, g)
    return _pack(shape, wg, wu, wd)


def stacked_expert_weights(shape: LayerShape, seed: int, device="cpu") -> Dict[str, torch.Tensor]:
    """Routed weights stacked over experts ([E, I, H], [E, I, H], [E, H, I] (+ scales)),
    filled expert by expert so that only one expert's float32 draw is live at a time."""
    out = None
    for e in range(shape.n_routed_experts):
        w = expert_weights(shape, seed, e, device)
        if out is None:
            out = {k: torch.empty((shape.n_routed_experts, *v.shape), dtype=v.dtype, device=v.device)
                   for k, v in w.items()}
        for k, v in w.items():
            out[k][e].copy_(v)
    return out


def _mx_random(gate_shape, up_shape, down_shape, g) -> Dict[str, torch.Tensor]:
    """MXFP4 weights drawn directly as codes: uniform random bytes (two E2M1 codes
    each, element 2i in the low nibble) and E8M0 scale codes from MX_SCALE_CODES,
    one per 32 contraction elements.  No quantisation step is involved."""
    out = {}
    for name, (rows, k) in (("gate", gate_shape), ("up", up_shape), ("down", down_shape)):
        out[name] = torch.randint(0, 256, (rows, k // 2), generator=g, dtype=torch.uint8, device=g.device)
        out[name + "_s"] = torch.randint(MX_SCALE_CODES[0], MX_SCALE_CODES[1] + 1, (rows, k // MX_BLOCK),
                                         generator=g, dtype=torch.uint8, device=g.device)
    return out


def _pack(shape: LayerShape, wg, wu, wd) -> Dict[str, torch.Tensor]:
    if shape.weight_dtype == DT_FP8:
        out = {}
        for name, w in (("gate", wg), ("up", wu), ("down", wd)):
            q, s = _quantise_rows_g128(w)
            out[name] = q
            out[name + "_s"] = s
        return out
    dt = _TORCH_ACT[shape.weight_dtype]
    return {"gate": wg.to(dt), "up": wu.to(dt), "down": wd.to(dt)}


# ----------------------------------------------------------------------------- whole layer

@dataclasses.dataclass
class LayerInputs:
    shape: LayerShape
    T: int
    seed: int
    x: torch.Tensor
    w_router: torch.Tensor
    w_shared_gate: Optional[torch.Tensor]
    logit_bias: Optional[torch.Tensor]
    alpha: Optional[float] = None


def layer_inputs(shape: LayerShape, T: int, seed: int, alpha: Optional[float] = None,
                 bias_attempt: int = 0) -> LayerInputs:
    """Activations and router inputs for one call (expert weights come separately)."""
    bias = None
    if shape.block_bias:
        bias = drafter_block_bias(shape, seed, T)
    elif alpha is not None and alpha != 0.0:
        bias = zipf_rank_bias(shape, seed, T, alpha, bias_attempt)
    return LayerInputs(shape, T, seed, tokens(shape, seed, T), router_weight(shape, seed),
                       shared_gate_weight(shape, seed), bias, alpha)


