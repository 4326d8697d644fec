"""Plain CPU oracle of the routed Mixture-of-Experts FFN forward (float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only tests/, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes, step by step, each from the page that defines it:

1. Router logits z[t,e] = x_t . W_r[e] (+ an optional per-token bias, which is
   how the Zipf router skew of [DeepGEMM PR #381, block_m note on the
   "--skew-alpha" router bias] enters), and the shared-expert gate logit
   g[t] = x_t . w_g.
2. Softmax over all experts, top-k, renormalise over the k kept
   [SpecForge PR #943, "Modifications": softmax, renormalised top-k preset].
2b. Optional per-token top-p trim of the top-k, which runs before the budget
   [colibri issue_budget.md, "Relationship to existing features": TOPP trims
   within one position's top-K; TOPP then EXPERT_BUDGET compose in that order].
3. Optional expert budget across the batch union [colibri issue_budget.md,
   "How it works"]: aggregate gate weight per distinct expert, keep the B
   heaviest, remove the others from every token's list, renormalise if
   norm_topk.
4. Dispatch: per-expert counts, exclusive offsets, and the slot permutation
   sorted by (expert, token).
5. Routed experts: y_t += w_{t,k} * W_down[e] (silu(W_gate[e] x_t) * (W_up[e] x_t)).
6. Shared expert, sigmoid-gated [SpecForge PR #943, "Modifications": shared
   expert (2048, sigmoid-gated)]: y_t += sigmoid(g[t]) * SwiGLU_shared(x_t).
7. fp8 weights (e4m3, group-128 fp32 scales) are used as decode(q) * s; the
   activations that enter an fp8 contraction (x before gate/up, h before down)
   are quantised per row per 128-group exactly as the kernels do, in float32
   (see oracle.e4m3.quantise_group128).
7b. MXFP4 weights (E2M1 codes, one E8M0 scale per 32 elements) are used as
   decoded code * 2^(e - 127); the activations entering their contractions are
   quantised per row and 32-block to MXFP8 (see oracle.mx.quantise_mxfp8).

8. Diagnostic variant (not the parity reference): h rounded to bfloat16
   (nearest, ties to even, straight from float64) before the down contraction,
   which is what a kernel that stores h in bf16 consumes.  It separates kernel
   errors from the bf16 rounding of h, which alone moves y by ~1.7e-3 relative L2.
   For fp8 / MXFP4 weights a "plain" variant leaves the activations unquantised
   (dequantised weights only), to report the format's own error apart.

Readings where the pages are silent (all listed in the design notes):
  * top-k selection is decided on float32 logits, ties to the lower expert id;
    a NaN logit counts as -inf; the k ids are stored by descending weight;
  * the budget ranks experts by (aggregate weight desc, id asc), triggers only
    when the union exceeds B (B = 0 is off), compacts kept slots to the front
    and marks dropped slots id -1 / weight 0; a token that loses every slot is
    not renormalised and gets no routed contribution;
  * SwiGLU is down(silu(gate x) * (up x)) with no biases; silu(a) = a / (1 + e^-a);
  * the shared expert is not counted against the budget;
  * top-p (0 < p < 1; 0 and 1 are off): the picks are taken by descending
    probability and pick k survives iff the picks before it hold less than p of
    the K picks' summed probability, so the survivors are the shortest prefix
    reaching p of the top-k mass and pick 0 always survives; the survivors are
    renormalised if norm_topk; the survive/drop decision is taken in float32,
    as the kernel takes it (probabilities exp(z - z_max) of the float32 logits,
    summed in pick order); dropped slots are id -1 / weight 0 at the row's end
    and are not counted in the budget statistics.
"""
from __future__ import annotations

from typing import Callable, Dict, Optional, Sequence

import numpy as np

from . import e4m3
from . import mx

# ----------------------------------------------------------------------------- helpers


def as_f64(a) -> np.ndarray:
    """Any numeric array (numpy or a CPU torch tensor, incl. bfloat16) -> float64."""
    if hasattr(a, "detach"):  # torch tensor; bf16 / fp16 / fp32 -> float64 is exact
        import torch
        return a.detach().cpu().to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def round_bf16(v) -> np.ndarray:
    """float64 -> nearest bfloat16 value (8 significant bits, ties to even), as float64.

    Rounds straight from float64 (no intermediate float32 step, which could round
    twice).  bf16 shares float32's exponent range: below 2^-126 the spacing is
    2^-133 (subnormals); results of magnitude 2^128 or more are infinite.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                                   # v = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)                          # exponent of one unit in the last place
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)           # np.rint rounds half to even
    with np.errstate(invalid="ignore"):
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
    return np.where(np.isfinite(v), r, v)


def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def sigmoid(a: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-a))


# ----------------------------------------------------------------------------- 1. router


def router_logits(x, w_router, logit_bias=None) -> np.ndarray:
    """z [T, E] = x W_r^T (+ bias), float64."""
    z = as_f64(x) @ as_f64(w_router).T
    if logit_bias is not None:
        z = z + as_f64(logit_bias)
    return z


def shared_gate_logit(x, w_shared_gate) -> np.ndarray:
    """g [T] = x . w_g, float64."""
    return as_f64(x) @ as_f64(w_shared_gate)


# ----------------------------------------------------------------------------- 2. softmax / top-k


def topk_softmax(z: np.ndarray, K: int, norm_topk: bool = True):
    """Softmax over all experts, keep the K largest, renormalise if norm_topk.

    The selection is decided on float32 logits with ties going to the lower
    expert id; ids are listed by descending logit.  Returns ids int32 [T, K],
    weights float64 [T, K].
    """
    z = np.where(np.isnan(z), -np.inf, np.asarray(z, dtype=np.float64))
    T, E = z.shape
    z32 = z.astype(np.float32)
    ids = np.empty((T, K), dtype=np.int32)
    for t in range(T):
        # Stable sort on (-z32, e): lexsort's last key is primary.
        order = np.lexsort((np.arange(E), -z32[t].astype(np.float64)))
        ids[t] = order[:K]
    # Softmax over all E in float64 (max-subtracted), then pick and renormalise.
    zmax = z.max(axis=1, keepdims=True)
    p = np.exp(z - zmax)
    p = p / p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if norm_topk:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w


# ----------------------------------------------------------------------------- 2b. top-p trim


def top_p_trim(z: np.ndarray, ids: np.ndarray, w: np.ndarray, top_p: float, norm_topk: bool = True):
    """Trim each token's top-k picks to its top-p mass [colibri issue_budget.md,
    "Relationship to existing features"].

    Pick k (ids are by descending probability) survives iff the probability of
    the picks before it is below top_p times that of all K picks.  The test runs
    in float32 on exp(z - z_max) of the float32 logits, summed in pick order.
    Survivors keep their float64 weight, renormalised over the survivors if
    norm_topk; the other slots become id -1 / weight 0.  top_p outside (0, 1)
    leaves the picks unchanged.
    """
    ids = np.array(ids, dtype=np.int32, copy=True)
    w = np.array(w, dtype=np.float64, copy=True)
    if not (0.0 < top_p < 1.0):
        return ids, w
    z32 = np.asarray(z, dtype=np.float64).astype(np.float32)
    p_cut = np.float32(top_p)
    T, K = ids.shape
    for t in range(T):
        zk = z32[t, ids[t].astype(np.int64)]
        p = np.exp(zk - zk[0])                  # float32, pick 0 is the largest logit
        total = np.float32(0.0)
        for k in range(K):
            total = np.float32(total + p[k])
        before = np.float32(0.0)
        n = 0
        for k in range(K):
            if k > 0 and not (before < p_cut * total):
                break
            n += 1
            before = np.float32(before + p[k])
        if n == K:
            continue
        kept = w[t, :n].copy()
        ids[t, n:] = -1
        w[t, n:] = 0.0
        w[t, :n] = kept / kept.sum() if norm_topk else kept
    return ids, w


# ----------------------------------------------------------------------------- 3. expert budget


def expert_budget(ids: np.ndarray, w: np.ndarray, budget: int, norm_topk: bool = True):
    """Cap the number of distinct experts over the whole batch [colibri issue_budget.md,
    "How it works", steps 1-5].

    Returns (ids, w, stats) with stats = [union size before, union size after,
    dropped slots, tokens left with no expert].
    """
    ids = np.array(ids, dtype=np.int32, copy=True)
    w = np.array(w, dtype=np.float64, copy=True)
    T, K = ids.shape
    union = sorted({int(e) for e in ids.ravel() if e >= 0})
    nu = len(union)
    if budget <= 0 or nu <= budget:
        return ids, w, np.array([nu, nu, 0, 0], dtype=np.int64)
    # Step 1: aggregate gate weight per distinct expert, summed in slot order.
    agg = {e: 0.0 for e in union}
    for t in range(T):
        for k in range(K):
            if ids[t, k] >= 0:
                agg[int(ids[t, k])] += w[t, k]
    # Steps 2-3: order by descending aggregate (ties: lower id) and keep the first `budget`.
    ranked = sorted(union, key=lambda e: (-agg[e], e))
    keep = set(ranked[:budget])
    # Step 4: remove dropped experts from every token's list; renormalise if norm_topk.
    dropped = 0
    empty = 0
    for t in range(T):
        kept = [(int(ids[t, k]), w[t, k]) for k in range(K) if ids[t, k] >= 0 and int(ids[t, k]) in keep]
        dropped += sum(1 for k in range(K) if ids[t, k] >= 0) - len(kept)
        if not kept:
            empty += 1
        total = sum(v for _, v in kept)
        ids[t, :] = -1
        w[t, :] = 0.0
        for k, (e, v) in enumerate(kept):
            ids[t, k] = e
            w[t, k] = v / total if norm_topk else v
    # Step 5 (compacting the union) is implicit: the union is now the kept set.
    return ids, w, np.array([nu, budget, dropped, empty], dtype=np.int64)


# ----------------------------------------------------------------------------- 4. dispatch


def dispatch(ids: np.ndarray, E: int):
    """counts [E], offsets [E+1] (exclusive scan) and perm: the kept slot indices
    s = t*K + k sorted by (expert, token)."""
    ids = np.asarray(ids)
    T, K = ids.shape
    slots = [s for s in range(T * K) if ids.flat[s] >= 0]
    perm = np.array(sorted(slots, key=lambda s: (int(ids.flat[s]), s // K)), dtype=np.int32)
    counts = np.zeros(E, dtype=np.int32)
    for s in slots:
        counts[ids.flat[s]] += 1
    offsets = np.zeros(E + 1, dtype=np.int32)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    return counts, offsets, perm


# ----------------------------------------------------------------------------- 5-7. experts


def _np(a) -> np.ndarray:
    return a.detach().cpu().numpy() if hasattr(a, "detach") else np.asarray(a)


def _weights_f64(wdict: Dict, weight_dtype: str):
    """Expert weight dict -> float64 (gate [N,H], up [N,H], down [H,N])."""
    if weight_dtype == "mxfp4":
        return tuple(mx.dequant_mxfp4(_np(wdict[n]).view(np.uint8), _np(wdict[n + "_s"]).view(np.uint8))
                     for n in ("gate", "up", "down"))
    if weight_dtype == "fp8_e4m3_g128":
        out = []
        for name in ("gate", "up", "down"):
            q = wdict[name]
            q = q.detach().cpu().numpy() if hasattr(q, "detach") else np.asarray(q)
            out.append(e4m3.dequantise_group128(q.view(np.uint8), as_f64(wdict[name + "_s"])))
        return tuple(out)
    return tuple(as_f64(wdict[n]) for n in ("gate", "up", "down"))


def _fp8_activation(v: np.ndarray) -> np.ndarray:
    q, s = e4m3.quantise_group128(v.astype(np.float32))
    return e4m3.dequantise_group128(q, s)


def _mx_activation(v: np.ndarray) -> np.ndarray:
    return mx.dequant_mxfp8(*mx.quantise_mxfp8(v.astype(np.float32)))


# Output variants of the expert math: name -> (quantise activations, round h to bf16).
#   "model":  the parity reference: activations quantised as the fp8 / MXFP4
#             contractions consume them (no-op for f32 / bf16 weights);
#   "bf16_h": the diagnostic of step 8, h rounded to bf16 before down;
#   "plain":  activations left unquantised (dequantised weights only).
VARIANTS = {"model": (True, False), "bf16_h": (False, True), "plain": (False, False)}


def swiglu_ffn(xrows: np.ndarray, wdict: Dict, weight_dtype: str, quantise_acts: bool = True,
               h_bf16: bool = False, weights=None) -> np.ndarray:
    """down(silu(gate x) * (up x)) for each row of xrows (float64).

    With fp8 weights the rows of x and of h are quantised per 128-group before
    they enter the contraction, matching what an fp8 x fp8 contraction consumes;
    with MXFP4 weights they are quantised to MXFP8 (32-element blocks, E8M0
    scales), what the block-scaled fp8 x fp4 contraction consumes.
    quantise_acts=False skips that (the plain layer of the dequantised weights);
    h_bf16 rounds h to bfloat16 before down.  `weights`: the float64 (gate, up,
    down) of wdict if already decoded.
    """
    wg, wu, wd = weights if weights is not None else _weights_f64(wdict, weight_dtype)
    quant = {"fp8_e4m3_g128": _fp8_activation, "mxfp4": _mx_activation}.get(weight_dtype)
    if not quantise_acts:
        quant = None
    xa = quant(xrows) if quant else xrows
    a = xa @ wg.T
    b = xa @ wu.T
    h = silu(a) * b
    if quant:
        h = quant(h.astype(np.float32))
    if h_bf16:
        h = round_bf16(h)
    return h @ wd.T


def moe_combine(x, ids, w, shared_gate: Optional[np.ndarray],
                expert: Callable[[int], Dict], shared: Optional[Dict],
                weight_dtype: str, tokens: Optional[Sequence[int]] = None,
                variants: Optional[Sequence[str]] = None):
    """y for the given tokens (all by default): sum over each token's kept slots of
    w * expert_e(x_t), plus sigmoid(g_t) * shared(x_t).

    `expert(e)` returns routed expert e's weight dict; `shared_gate` holds
    sigmoid(g) per token.  Experts are visited one at a time so the full weight set
    never has to sit in host memory.  Returns the "model" variant's y, or, if
    `variants` names several of VARIANTS, a dict of y per variant (each expert's
    weights decoded once for all of them).
    """
    names = ["model"] if variants is None else list(variants)
    x64 = as_f64(x)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    toks = np.arange(x64.shape[0]) if tokens is None else np.asarray(tokens, dtype=np.int64)
    ys = {n: np.zeros((len(toks), x64.shape[1]), dtype=np.float64) for n in names}
    sub_ids = ids[toks]
    sub_w = w[toks]
    for e in sorted({int(v) for v in sub_ids.ravel() if v >= 0}):
        rows, ks = np.nonzero(sub_ids == e)
        wdict = expert(e)
        wts = _weights_f64(wdict, weight_dtype)
        for n in names:
            q, hb = VARIANTS[n]
            out = swiglu_ffn(x64[toks[rows]], wdict, weight_dtype, q, hb, wts)
            ys[n][rows] += sub_w[rows, ks][:, None] * out
    if shared is not None:
        wts = _weights_f64(shared, weight_dtype)
        sg = np.asarray(shared_gate, dtype=np.float64)[toks][:, None]
        for n in names:
            q, hb = VARIANTS[n]
            ys[n] += sg * swiglu_ffn(x64[toks], shared, weight_dtype, q, hb, wts)
    return ys["model"] if variants is None else ys


# ----------------------------------------------------------------------------- whole layer


def route(x, w_router, w_shared_gate, logit_bias, K: int, norm_topk: bool = True, budget: int = 0,
          top_p: float = 0.0):
    """Steps 1-3: ids, weights, sigmoid(shared gate logit), budget stats, logits."""
    z = router_logits(x, w_router, logit_bias)
    ids, w = topk_softmax(z, K, norm_topk)
    ids, w = top_p_trim(z, ids, w, top_p, norm_topk)
    ids, w, stats = expert_budget(ids, w, budget, norm_topk)
    sg = sigmoid(shared_gate_logit(x, w_shared_gate)) if w_shared_gate is not None else None
    return {"ids": ids, "w": w, "shared_gate": sg, "stats": stats, "logits": z}


def moe_layer(x, w_router, w_shared_gate, logit_bias, K: int, E: int,
              expert: Callable[[int], Dict], shared: Optional[Dict], weight_dtype: str,
              norm_topk: bool = True, budget: int = 0, tokens=None, top_p: float = 0.0,
              variants: Optional[Sequence[str]] = None) -> Dict:
    """The whole forward: route, dispatch, y (for `tokens`, default all).  With
    `variants`, also y_<name> for each named output variant (y is "model")."""
    r = route(x, w_router, w_shared_gate, logit_bias, K, norm_topk, budget, top_p)
    counts, offsets, perm = dispatch(r["ids"], E)
    names = ["model"] + [n for n in (variants or []) if n != "model"]
    ys = moe_combine(x, r["ids"], r["w"], r["shared_gate"], expert, shared, weight_dtype, tokens, names)
    r.update(counts=counts, offsets=offsets, perm=perm, y=ys["model"])
    for n in names[1:]:
        r["y_" + n] = ys[n]
    return r
