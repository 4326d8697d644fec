"""Test-side harness: seeded inputs, conditioned by the oracle so that every
routing decision has a margin, run through the HIP library and compared with the
CPU oracle.

TEST INFRASTRUCTURE (imports the oracle).  Used by tests/ and the smoke check.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import workloads as W
from oracle import moe as O

# Top-k margin: the sorted logits of every token differ by more than this between
# neighbours 1..K+1, so the float32 GPU logits pick the same ids in the same order.
TOPK_MARGIN = 1e-3
# Top-p margin: every prefix sum of a token's top-k probabilities differs from
# top_p times their total by more than this fraction of the total, so the GPU
# (float32 logits and sums) and the oracle trim at the same pick.
TOPP_MARGIN = 1e-3
# Budget margin: the B-th and (B+1)-th aggregate weights differ by more than this.
BUDGET_MARGIN = 1e-4

TOL = {"f32": 1e-5, "bf16": 2e-3, "fp8_e4m3_g128": 1e-2, "mxfp4": 1e-2}   # relative L2 of y

# Kernel-bug checks, tighter than the parity bars above, against the oracle variant
# that sees what the kernels see:
#   bf16 weights: the bf16-h diagnostic (h rounded to bf16 before down).  What is
#   left is float32 summation order, plus the rare element of h whose float32
#   value rounds to the other bf16 neighbour than the exact value does: a
#   relative difference d ~ 1e-6 moves about d / 2^-8 of the elements by one bf16
#   step (2^-8 relative), ~1e-4 relative L2 in all.
#   fp8 / MXFP4 weights: the oracle that models the activation quantisation; a
#   code that lands on the other side of a rounding boundary moves that element
#   by one 3-bit-mantissa step, ~1e-3 relative L2 in all.
#   f32 weights: the plain oracle, float32 summation order only.
BUG_TOL = {"f32": 1e-5, "bf16": 2e-4, "fp8_e4m3_g128": 3e-3, "mxfp4": 3e-3}
# The same per token (relative L2 of each checked token's row of y): every token
# within TOKEN_TOL, and the median token within BUG_TOL.  With fp8 / MXFP4 weights a
# single code of h landing on the other side of a rounding boundary moves that
# element of h by one 3-bit-mantissa step (up to 2^-3 of it); if it is the largest
# element of a short row (I = 256: |h_max| / ||h|| up to ~0.3) the token's output
# moves by up to ~4 %, so the per-token bound is 5e-2 there and the median carries
# the check.
TOKEN_TOL = {"f32": 1e-4, "bf16": 1e-3, "fp8_e4m3_g128": 5e-2, "mxfp4": 5e-2}
# Oracle variant each bug check compares with (see oracle.moe.VARIANTS).
BUG_REF = {"f32": "model", "bf16": "bf16_h", "fp8_e4m3_g128": "model", "mxfp4": "model"}
# Routing weights, absolute.  The pages fix no tolerance here; the bound comes from
# the arithmetic: the logits are float32 sums of H <= 7168 bf16 products with
# |z| = O(1), whose rounding (random-walk ~ sqrt(H) * 2^-24 * |partial sums|) is a
# few 1e-6, and a renormalised softmax weight moves by at most about that much.
W_TOL = 1e-5


@dataclasses.dataclass
class Case:
    shape: W.LayerShape
    T: int
    seed: int
    alpha: Optional[float]
    inp: W.LayerInputs
    weights: Dict[str, torch.Tensor]            # stacked routed weights (device)
    shared: Optional[Dict[str, torch.Tensor]]   # shared expert weights (device)
    redrawn_rows: int = 0
    bias_attempts: int = 0

    def expert_cpu(self, e: int) -> Dict[str, torch.Tensor]:
        return {k: v[e].cpu() for k, v in self.weights.items()}

    def shared_cpu(self):
        return None if self.shared is None else {k: v.cpu() for k, v in self.shared.items()}


def _topk_gaps_ok(z: np.ndarray, K: int, top_p: float = 0.0) -> np.ndarray:
    """Per token: the K+1 largest logits are separated by more than TOPK_MARGIN, and
    (top-p on) no prefix of the top-k probabilities sits within TOPP_MARGIN of the cut."""
    E = z.shape[1]
    top = -np.sort(-z, axis=1)[:, :min(K + 1, E)]
    gaps = top[:, :-1] - top[:, 1:]
    ok = (gaps > TOPK_MARGIN).all(axis=1) if gaps.shape[1] else np.ones(z.shape[0], bool)
    if 0.0 < top_p < 1.0:
        p = np.exp(top[:, :K] - top[:, :1])
        total = p.sum(axis=1, keepdims=True)
        prefix = np.cumsum(p, axis=1)[:, :-1]
        ok &= (np.abs(prefix - top_p * total) > TOPP_MARGIN * total).all(axis=1)
    return ok


def condition_topk(shape: W.LayerShape, inp: W.LayerInputs, max_attempts: int = 200) -> int:
    """Re-draw rows of x (seeded by token and attempt) until every token's top-k has margins."""
    redrawn = 0
    for attempt in range(1, max_attempts + 1):
        z = O.router_logits(inp.x, inp.w_router, inp.logit_bias)
        bad = np.nonzero(~_topk_gaps_ok(z, shape.num_experts_per_tok, shape.top_p))[0]
        if len(bad) == 0:
            return redrawn
        for t in bad:
            inp.x[t] = W.token_row(shape, inp.seed, int(t), attempt)
        redrawn += len(bad)
    raise RuntimeError("could not condition the top-k margins")


def _budget_gap(shape: W.LayerShape, inp: W.LayerInputs) -> float:
    r = O.route(inp.x, inp.w_router, inp.w_shared_gate, inp.logit_bias, shape.num_experts_per_tok,
                bool(shape.norm_topk_prob), 0, shape.top_p)
    ids, w = r["ids"], r["w"]
    agg = sorted((float(w[ids == e].sum()) for e in set(ids.ravel().tolist())), reverse=True)
    B = shape.expert_budget
    if B <= 0 or len(agg) <= B:
        return float("inf")
    return agg[B - 1] - agg[B]


def make_case(shape: W.LayerShape, T: int, seed: int, alpha: Optional[float] = None,
              device: str = "cuda", condition: bool = True) -> Case:
    inp = W.layer_inputs(shape, T, seed, alpha)
    redrawn = attempts = 0
    if condition and T > 0:
        redrawn = condition_topk(shape, inp)
        while shape.expert_budget > 0 and _budget_gap(shape, inp) <= BUDGET_MARGIN:
            attempts += 1
            if attempts > 50:
                raise RuntimeError("could not condition the budget margin")
            if alpha:   # re-permute the Zipf ranks
                inp.logit_bias = W.zipf_rank_bias(shape, seed, T, alpha, attempts)
            else:       # re-draw the first token
                inp.x[0] = W.token_row(shape, seed, 0, 10_000 + attempts)
            redrawn += condition_topk(shape, inp)
    weights = W.stacked_expert_weights(shape, seed, device)
    shared = W.shared_expert_weights(shape, seed, device)
    return Case(shape, T, seed, alpha, inp, weights, shared, redrawn, attempts)


def config(shape: W.LayerShape):
    import mixture_experts_layer_05_amd as moe
    return moe.MoEConfig(shape.hidden_size, shape.n_routed_experts, shape.moe_intermediate_size,
                         shape.num_experts_per_tok, shape.shared_expert_intermediate_size,
                         shape.weight_dtype, shape.act_dtype, shape.norm_topk_prob, shape.expert_budget,
                         shape.top_p)


def run_gpu(case: Case, layer=None) -> Dict[str, np.ndarray]:
    """route -> dispatch -> forward through the C ABI; returns host copies of every output."""
    import mixture_experts_layer_05_amd as moe
    shape, T = case.shape, case.T
    if layer is None:
        layer = moe.MoELayer(config(shape), case.weights, case.inp.w_router.cuda(),
                             None if case.inp.w_shared_gate is None else case.inp.w_shared_gate.cuda(),
                             case.shared, max_tokens=max(T, 1), stats=True)
    x = case.inp.x.cuda()
    bias = None if case.inp.logit_bias is None else case.inp.logit_bias.cuda()
    if layer.route_stats is not None:
        layer.route_stats.fill_(-7)
    y = layer(x, bias)
    torch.cuda.synchronize()
    v = layer.views(T)
    nkept = int(layer.offsets[-1].item())
    return {
        "ids": v["topk_ids"].cpu().numpy(), "w": v["topk_weights"].cpu().numpy(),
        "shared_gate": v["shared_gate"].cpu().numpy(),
        "stats": None if layer.route_stats is None else layer.route_stats.cpu().numpy(),
        "counts": layer.counts.cpu().numpy(), "offsets": layer.offsets.cpu().numpy(),
        "perm": v["perm"][:nkept].cpu().numpy(), "y": y.cpu().numpy().astype(np.float64),
    }


def cover_tokens(ids: np.ndarray, offsets: np.ndarray, perm: np.ndarray, K: int, n: int,
                 seed: int = 0) -> np.ndarray:
    """About n tokens whose rows reach every kind of tile the kernels form: the first
    and last token; up to 16 tokens left with no expert; for every touched expert
    its first and last dispatch row; for
    the busiest experts also the rows on both sides of every 128-row boundary (the
    streaming kernel's tallest tiles and the 256-row kernel's tiles and their short
    tails); the rest a seeded sample."""
    T = ids.shape[0]
    E = len(offsets) - 1
    counts = np.diff(offsets)
    must, extra = {0, T - 1}, set()
    # Tokens that lost every slot (their y must be exactly the shared term, or 0).
    must |= set(np.nonzero((ids < 0).all(axis=1))[0][:16].tolist())
    busiest = np.argsort(-counts, kind="stable")[:8]
    for e in range(E):
        c = int(counts[e])
        if c == 0:
            continue
        rows = {0, c - 1}
        if e in busiest:
            rows |= {r for b in range(128, c, 128) for r in (b - 1, b)}
            rows |= {c - c % 256 - 1, c - c % 256} if c > 256 else set()
        toks = {int(perm[offsets[e] + r]) // K for r in rows if 0 <= r < c}
        (must if e in busiest else extra).update(toks)
    rng = np.random.default_rng(seed)
    pick = sorted(must)
    if len(pick) > n:
        pick = sorted(rng.choice(pick, size=n, replace=False).tolist())
    rest = sorted(extra - set(pick))
    if len(pick) + len(rest) > n:
        rest = rng.choice(rest, size=n - len(pick), replace=False).tolist() if n > len(pick) else []
    pick = sorted(set(pick) | set(rest))
    if len(pick) < n:
        free = np.setdiff1d(np.arange(T), pick)
        pick = sorted(set(pick) | set(rng.choice(free, size=min(n - len(pick), len(free)),
                                                 replace=False).tolist()))
    return np.asarray(pick, dtype=np.int64)


def run_oracle(case: Case, tokens=None) -> Dict[str, np.ndarray]:
    """The oracle on the case: routing and dispatch of every token, y (the parity
    reference) and the bug-check / report variants for `tokens` (all by default;
    an int n picks n covering tokens, see cover_tokens).  ora["tokens"] holds the
    tokens y was computed for (None: all)."""
    shape = case.shape
    K, E = shape.num_experts_per_tok, shape.n_routed_experts
    r = O.route(case.inp.x, case.inp.w_router, case.inp.w_shared_gate, case.inp.logit_bias, K,
                bool(shape.norm_topk_prob), shape.expert_budget, shape.top_p)
    counts, offsets, perm = O.dispatch(r["ids"], E)
    if isinstance(tokens, (int, np.integer)):
        tokens = cover_tokens(r["ids"], offsets, perm, K, int(tokens), case.seed)
    variants = ["model", BUG_REF[shape.weight_dtype]]
    if shape.weight_dtype in ("fp8_e4m3_g128", "mxfp4"):
        variants.append("plain")
    variants = list(dict.fromkeys(variants))
    ys = O.moe_combine(case.inp.x, r["ids"], r["w"], r["shared_gate"], case.expert_cpu, case.shared_cpu(),
                       shape.weight_dtype, tokens, variants)
    r.update(counts=counts, offsets=offsets, perm=perm, y=ys["model"], tokens=tokens)
    for n in variants[1:]:
        r["y_" + n] = ys[n]
    return r


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a))


def token_rel_l2(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Relative L2 of each row (rows whose reference is all zero are left out)."""
    den = np.linalg.norm(b, axis=1)
    num = np.linalg.norm(a - b, axis=1)
    return num[den > 0] / den[den > 0]


def compare(case: Case, gpu: Dict, ora: Dict, tokens: Optional[Sequence[int]] = None) -> Dict[str, float]:
    """Assert parity and the kernel-bug checks; return the measured errors."""
    shape = case.shape
    if tokens is None:
        tokens = ora.get("tokens")
    K = shape.num_experts_per_tok
    assert np.array_equal(gpu["ids"], ora["ids"]), "expert ids differ"
    werr = float(np.abs(gpu["w"] - ora["w"]).max()) if gpu["w"].size else 0.0
    assert werr <= W_TOL, f"routing weights differ by {werr}"
    if shape.expert_budget > 0:
        assert np.array_equal(gpu["stats"], ora["stats"]), (gpu["stats"], ora["stats"])
    else:
        nu = len(set(ora["ids"].ravel().tolist()) - {-1})
        assert gpu["stats"].tolist() == [nu, nu, 0, 0]
    assert np.array_equal(gpu["counts"], ora["counts"]), "expert counts differ"
    assert np.array_equal(gpu["offsets"], ora["offsets"]), "expert offsets differ"
    assert np.array_equal(gpu["perm"], ora["perm"]), "dispatch permutation differs"
    # Dispatch as a pure function of the GPU's own ids, too.
    c2, o2, p2 = O.dispatch(gpu["ids"], shape.n_routed_experts)
    assert np.array_equal(gpu["perm"], p2) and np.array_equal(gpu["counts"], c2)
    sg_err = 0.0
    if shape.shared_expert_intermediate_size > 0:
        sg_err = float(np.abs(gpu["shared_gate"] - ora["shared_gate"]).max())
        assert sg_err <= 1e-5, f"shared gate differs by {sg_err}"
    y_gpu = gpu["y"] if tokens is None else gpu["y"][np.asarray(tokens)]
    dt = shape.weight_dtype
    err = rel_l2(y_gpu, ora["y"])
    tol = TOL[dt]
    assert err <= tol, f"y relative L2 {err:.3e} > {tol:.0e}"
    # Kernel-bug checks against the oracle variant that sees what the kernels see.
    ref = ora["y"] if BUG_REF[dt] == "model" else ora["y_" + BUG_REF[dt]]
    bug = rel_l2(y_gpu, ref)
    assert bug <= BUG_TOL[dt], f"y relative L2 vs the {BUG_REF[dt]} oracle {bug:.3e} > {BUG_TOL[dt]:.0e}"
    per_tok = token_rel_l2(y_gpu, ref)
    tok_max = float(per_tok.max()) if per_tok.size else 0.0
    tok_med = float(np.median(per_tok)) if per_tok.size else 0.0
    assert tok_max <= TOKEN_TOL[dt], f"a token's relative L2 vs the {BUG_REF[dt]} oracle is {tok_max:.3e}"
    assert tok_med <= BUG_TOL[dt], f"median token relative L2 vs the {BUG_REF[dt]} oracle is {tok_med:.3e}"
    out = {"y_rel_l2": err, "y_bug_rel_l2": bug, "y_token_max": tok_max, "y_token_median": tok_med,
           "y_token_max_vs_plain": float(token_rel_l2(y_gpu, ora["y"]).max()) if y_gpu.size else 0.0,
           "w_max_abs": werr, "shared_gate_max_abs": sg_err}
    if "y_plain" in ora:
        # fp8 / MXFP4: the format's own error against the unquantised layer, reported, not gated.
        out["quant_err_vs_plain"] = rel_l2(y_gpu, ora["y_plain"])
    # Tokens with no kept expert and no shared expert must be exactly zero.
    if shape.shared_expert_intermediate_size == 0:
        toks = np.arange(case.T) if tokens is None else np.asarray(tokens)
        empty = (ora["ids"][toks] < 0).all(axis=1)
        assert (y_gpu[empty] == 0).all()
        out["empty_tokens_checked"] = int(empty.sum())
    return out


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    """n tokens spread over [0, T): first, last and a seeded sample in between."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid]))
