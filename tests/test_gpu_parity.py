"""GPU parity: the HIP library through its C ABI vs the CPU oracle.

Ids, counts, offsets, the permutation and the budget statistics must match
bit-exactly; routing weights within 1e-5; y within the relative-L2 bar of its
weight dtype (fp32 1e-5, bf16 2e-3, fp8 1e-2).  Sizes the oracle finishes in
seconds are compared on every token; the full-size workloads on sampled tokens.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import harness as Hn

pytestmark = pytest.mark.gpu


def _run(shape, T, seed, alpha=None, tokens=None, condition=True, mutate=None):
    print(f"\n[case] {shape.name} T={T} seed={seed} alpha={alpha}", flush=True)
    case = Hn.make_case(shape, T, seed, alpha, condition=condition)
    if mutate:
        mutate(case)
    gpu = Hn.run_gpu(case)
    ora = Hn.run_oracle(case, tokens)
    errs = Hn.compare(case, gpu, ora)
    n = case.T if ora["tokens"] is None else len(ora["tokens"])
    print(f"[case] ok {errs} tokens_checked={n} redrawn_rows={case.redrawn_rows}", flush=True)
    return case, gpu, ora, errs


def test_tiny_fp32_layer():
    _run(W.TINY, 64, W.base_seed(0, 64))


@pytest.mark.parametrize("T", [7, 56, 224])
def test_drafter_layer(T):
    _run(W.DRAFTER, T, W.base_seed(1, T))


@pytest.mark.parametrize("T", [7, 56])
def test_narrow_layer(T):
    _run(W.NARROW, T, W.base_seed(2, T))


def test_narrow_layer_224_sampled():
    _run(W.NARROW, 224, W.base_seed(2, 224), tokens=48)


@pytest.mark.parametrize("alpha", [0.0, 1.5])
def test_large_layer_512(alpha):
    _run(W.LARGE, 512, W.base_seed(3, 512), alpha, tokens=64)


def test_large_layer_2048_uniform_sampled():
    _run(W.LARGE, 2048, W.base_seed(3, 2048), 0.0, tokens=128)


def test_large_layer_8192_skewed_sampled():
    _run(W.LARGE, 8192, W.base_seed(3, 8192), 1.5, tokens=128)


# The rest of the large layer's (T, alpha) grid, on sampled tokens: the middle
# skew at every size, the skewed middle size and the uniform full size.
@pytest.mark.parametrize("T,alpha", [(512, 1.0), (2048, 1.0), (2048, 1.5), (8192, 0.0), (8192, 1.0)])
def test_large_layer_grid_sampled(T, alpha):
    _run(W.LARGE, T, W.base_seed(3, T), alpha, tokens=64)


# MXFP4 expert weights x MXFP8 activations (block-scaled fp8 x fp4 contraction).
@pytest.mark.parametrize("shape,T,idx,alpha,tokens", [
    (W.DRAFTER_MX4, 7, 1, None, None),
    (W.DRAFTER_MX4, 56, 1, None, None),
    (W.DRAFTER_MX4, 224, 1, None, 48),
    (W.NARROW_MX4, 56, 2, None, None),
    (W.LARGE_MX4, 512, 3, 1.5, 24),
    (W.LARGE_MX4.with_(name="large_mxfp4_budget64", expert_budget=64), 512, 4, 1.5, 24),
])
def test_mxfp4_layer(shape, T, idx, alpha, tokens):
    _run(shape, T, W.base_seed(idx, T), alpha, tokens=tokens)


# fp8 e4m3 group-128 weights on the decode layers (two-group streaming stages).
@pytest.mark.parametrize("shape,T,idx,tokens", [
    (W.DRAFTER_FP8, 7, 1, None),
    (W.DRAFTER_FP8, 224, 1, 48),
    (W.NARROW_FP8, 56, 2, None),
])
def test_fp8_decode_layer(shape, T, idx, tokens):
    _run(shape, T, W.base_seed(idx, T), tokens=tokens)


# A small fp8 layer on the two-group stages (H, I, S multiples of 256; the down
# projection is one stage long) with ragged row tiles.
_SMALL_FP8 = W.LayerShape("small_fp8_wide", 512, 8, 256, 2, 256, W.DT_FP8, W.DT_BF16)


@pytest.mark.parametrize("T", [1, 13, 64])
def test_fp8_small_ragged(T):
    _run(_SMALL_FP8, T, W.base_seed(0, T) + 11)


# fp8 gate/up in four-group stages (H a multiple of 512): 16 x 128 tiles at 6 rows
# per expert, 32 x 64 at 16, 64 x 64 at 25, ragged in all three.
_SMALL_FP8_QUAD = W.LayerShape("small_fp8_quad", 1024, 8, 512, 2, 512, W.DT_FP8, W.DT_BF16)


@pytest.mark.parametrize("T", [24, 64, 100])
def test_fp8_quad_stages_ragged(T):
    _run(_SMALL_FP8_QUAD, T, W.base_seed(0, T) + 17)


# MXFP4 at prefill sizes (128 x 128 streaming tiles): few experts with many rows
# (partial row tiles), and the large layer at T = 8192 on sampled tokens.
@pytest.mark.parametrize("shape,T,seed,alpha,tokens", [
    (W.LayerShape("mx_tall", 512, 4, 512, 2, 512, W.DT_MXFP4, W.DT_BF16), 700, 731, None, None),
    (W.LARGE_MX4, 8192, W.base_seed(3, 8192), 1.5, 16),
])
def test_mxfp4_prefill(shape, T, seed, alpha, tokens):
    _run(shape, T, seed, alpha, tokens=tokens)


# A small MXFP4 layer (contraction of 2 stages) with ragged row tiles: one token,
# 13 tokens and 64 tokens (~16 rows per expert).
_SMALL_MX4 = W.LayerShape("small_mxfp4", 512, 8, 256, 2, 256, W.DT_MXFP4, W.DT_BF16)


@pytest.mark.parametrize("T", [1, 13, 64])
def test_mxfp4_small_ragged(T):
    _run(_SMALL_MX4, T, W.base_seed(0, T) + 7)


# Top-p trim before the budget [colibri issue_budget.md, "Relationship to existing
# features"]: the per-token trim alone, and composed with the budget.
@pytest.mark.parametrize("shape,T,seed,top_p,tokens", [
    (W.TINY.with_(name="tiny_topp", top_p=0.4), 64, W.base_seed(0, 64), 0.4, None),
    (W.DRAFTER.with_(name="drafter_topp", top_p=0.8), 224, W.base_seed(1, 224), 0.8, 48),
    (W.NARROW.with_(name="narrow_topp", top_p=0.5), 56, W.base_seed(2, 56), 0.5, None),
    (W.LARGE_FP8.with_(name="large_fp8_topp_budget", top_p=0.7), 512, W.base_seed(4, 512), 0.7, 24),
])
def test_top_p_trim(shape, T, seed, top_p, tokens):
    alpha = 1.5 if shape.weight_dtype == W.DT_FP8 else None
    case, gpu, ora, _ = _run(shape, T, seed, alpha, tokens=tokens)
    K = shape.num_experts_per_tok
    kept = (gpu["ids"] >= 0).sum(axis=1)
    assert kept.min() >= 1 and kept.max() <= K
    if shape.expert_budget == 0:
        assert (kept < K).any(), "the trim never dropped a slot on this case"


def test_expert_parallel_rank_share_sampled():
    """One GPU's share of the large layer under 8-way expert parallelism: the global
    256-expert routing, restricted to the busiest rank's experts [32r, 32r + 32)
    (local id = id - 32r, other slots -1 with weight 0), then dispatch + forward of
    the rank's 32-expert layer.  Both sides route the global layer on their own;
    ids, counts, offsets and perm bit-exact, y on sampled tokens."""
    import mixture_experts_layer_05_amd as moe
    from oracle import moe as O
    g, loc, T, alpha = W.LARGE, W.EP_RANK, 4096, 1.5
    seed = W.base_seed(5, T)
    print(f"\n[case] {loc.name} T={T} seed={seed} alpha={alpha}", flush=True)
    inp = W.layer_inputs(g, T, seed, alpha)
    Hn.condition_topk(g, inp)
    K, E = g.num_experts_per_tok, W.EP_RANK_LOCAL
    weights = W.stacked_expert_weights(loc, seed, "cuda")
    x, bias = inp.x.cuda(), inp.logit_bias.cuda()

    gcfg = Hn.config(g)
    gws = torch.empty(moe.workspace_size(gcfg, T), dtype=torch.uint8, device="cuda")
    gids = torch.empty(T, K, dtype=torch.int32, device="cuda")
    gw = torch.empty(T, K, dtype=torch.float32, device="cuda")
    moe.route(gcfg, x, inp.w_router.cuda(), None, bias, gids, gw, None, None, gws)
    rank = int(torch.bincount((gids // E).flatten().long(), minlength=W.EP_RANKS).argmax())
    lids = gids - rank * E
    local = (lids >= 0) & (lids < E)
    layer = moe.MoELayer(Hn.config(loc), weights, inp.w_router[:E].cuda(), None, None, max_tokens=T)
    layer.topk_ids.copy_(torch.where(local, lids, torch.full_like(lids, -1)))
    layer.topk_weights.copy_(torch.where(local, gw, torch.zeros_like(gw)))
    layer.dispatch(T)
    layer.forward(x)
    torch.cuda.synchronize()
    ids_g = layer.topk_ids.cpu().numpy()
    nkept = int(layer.offsets[-1].item())

    r = O.route(inp.x, inp.w_router, None, inp.logit_bias, K, bool(g.norm_topk_prob), 0)
    rank_o = int(np.argmax(np.bincount(r["ids"].ravel() // E, minlength=W.EP_RANKS)))
    assert rank_o == rank
    lid = r["ids"] - rank_o * E
    keep = (lid >= 0) & (lid < E)
    ids_o = np.where(keep, lid, -1)
    w_o = np.where(keep, r["w"], 0.0)
    assert np.array_equal(ids_g, ids_o), "rank-local expert ids differ"
    werr = float(np.abs(layer.topk_weights.cpu().numpy() - w_o).max())
    assert werr <= Hn.W_TOL, werr
    counts, offsets, perm = O.dispatch(ids_o, E)
    assert np.array_equal(layer.counts.cpu().numpy(), counts)
    assert np.array_equal(layer.offsets.cpu().numpy(), offsets)
    assert np.array_equal(layer.perm[:nkept].cpu().numpy(), perm)
    assert 0 < nkept < T * K
    # Covering tokens (every local expert's first and last row, the busiest ones'
    # tile boundaries, tokens the rank receives nothing for), y vs the oracle and
    # vs its bf16-h diagnostic.
    tokens = Hn.cover_tokens(ids_o, offsets, perm, K, 96, seed)
    expert_cpu = lambda e: {k: v[e].cpu() for k, v in weights.items()}  # noqa: E731
    ys = O.moe_combine(inp.x, ids_o, w_o, None, expert_cpu, None, loc.weight_dtype, tokens,
                       ["model", "bf16_h"])
    y_g = layer.y.cpu().numpy().astype(np.float64)
    err = Hn.rel_l2(y_g[tokens], ys["model"])
    assert err <= Hn.TOL[loc.weight_dtype], err
    bug = Hn.rel_l2(y_g[tokens], ys["bf16_h"])
    assert bug <= Hn.BUG_TOL["bf16"], bug
    tok = Hn.token_rel_l2(y_g[tokens], ys["bf16_h"])
    assert tok.max() <= Hn.TOKEN_TOL["bf16"], tok.max()
    empty = (ids_o < 0).all(axis=1)
    assert empty.any() and (y_g[empty] == 0).all()
    print(f"[case] ok y_rel_l2={err:.3e} y_bug_rel_l2={bug:.3e} y_token_max={tok.max():.3e} "
          f"w_max_abs={werr:.1e} rank={rank} kept={nkept} of {T * K} slots", flush=True)


def test_fp8_budget_layer_8192_sampled():
    case, gpu, ora, errs = _run(W.LARGE_FP8, 8192, W.base_seed(4, 8192), 1.5, tokens=128)
    assert gpu["stats"][1] == 64 and gpu["stats"][0] > 64


def test_fp8_small_budget_drops_experts():
    shape = W.LARGE_FP8.with_(expert_budget=32)
    case, gpu, ora, errs = _run(shape, 512, W.base_seed(4, 512), 1.5, tokens=64)
    assert gpu["stats"][0] > 32 and gpu["stats"][1] == 32 and gpu["stats"][2] > 0
    # Same quantisation decisions on both sides: far below the fp8 bar.
    assert errs["y_rel_l2"] < 1e-3


def test_budget_without_statistics_routes_the_same():
    """MoELayer asks for no routing statistics by default: the budget pass then runs
    with a null statistics pointer and must route and compute exactly as with one."""
    import mixture_experts_layer_05_amd as moe
    shape = W.LayerShape("small_budget", 512, 16, 256, 4, 256, W.DT_FP8, W.DT_BF16, expert_budget=6)
    print(f"\n[case] {shape.name} budget without statistics", flush=True)
    case = Hn.make_case(shape, 96, W.base_seed(5, 96), 1.5)
    with_stats = Hn.run_gpu(case)
    assert with_stats["stats"][0] > 6 and with_stats["stats"][1] == 6
    layer = moe.MoELayer(Hn.config(shape), case.weights, case.inp.w_router.cuda(),
                         case.inp.w_shared_gate.cuda(), case.shared, max_tokens=96)
    assert layer.route_stats is None
    plain = Hn.run_gpu(case, layer)
    for k in ("ids", "w", "counts", "offsets", "perm", "y"):
        assert np.array_equal(plain[k], with_stats[k]), k


def test_large_budget_empties_tokens_full_size():
    """The large layer with uniform routing (alpha 0) and a budget of 64 at T = 8192:
    hundreds of tokens lose every slot [colibri issue_budget.md, "How it works"
    step 4, "Safety"]; with no shared expert their y must be exactly 0."""
    shape = W.LARGE.with_(name="large_budget64", expert_budget=64)
    case, gpu, ora, errs = _run(shape, 8192, W.base_seed(3, 8192) + 64, 0.0, tokens=128)
    assert gpu["stats"][0] > 64 and gpu["stats"][1] == 64 and gpu["stats"][3] > 100, gpu["stats"]
    assert errs["empty_tokens_checked"] > 0
    empty = (gpu["ids"] < 0).all(axis=1)
    assert (gpu["y"][empty] == 0).all()          # every emptied token, not only the checked ones


# A mid-size layer for the tile override: about 128 rows per expert, so every
# streaming tile height and the 256-row kernels each see full and partial tiles.
_INVARIANCE = W.LayerShape("tile_invariance", 1024, 16, 512, 4, 512, W.DT_BF16, W.DT_BF16)


@pytest.mark.parametrize("dt", [W.DT_BF16, W.DT_FP8, W.DT_MXFP4])
def test_tile_override_config_invariance(dt, monkeypatch):
    """Every setting of the tile override (MOE_FORCE_TILE) on one case: routing and
    dispatch bit-identical, y within the parity and kernel-bug bars for each, and y
    bit-identical to the default's [DeepGEMM PR #381, "Validation": bit-exact output
    across forced settings].  Every kernel family walks each output's contraction
    in the same order, 128-element stages in ascending order with the same MFMA
    accumulation inside a stage, so the tile shape does not change a single bit."""
    import mixture_experts_layer_05_amd as moe
    shape = _INVARIANCE.with_(name=f"tile_invariance_{dt}", weight_dtype=dt)
    T = 512
    case = Hn.make_case(shape, T, W.base_seed(6, T), 1.0)
    ora = Hn.run_oracle(case)
    settings = ["auto", "stream16", "stream32", "stream64", "stream128", "split"]
    base = None
    for st in settings:
        print(f"\n[case] {shape.name} T={T} MOE_FORCE_TILE={st}", flush=True)
        monkeypatch.setenv("MOE_FORCE_TILE", st)
        gpu = Hn.run_gpu(case)
        errs = Hn.compare(case, gpu, ora)
        if base is None:
            base = gpu
        for k in ("ids", "w", "counts", "offsets", "perm", "stats"):
            assert np.array_equal(gpu[k], base[k]), (st, k)
        d = Hn.rel_l2(gpu["y"], base["y"])
        assert np.array_equal(gpu["y"], base["y"]), (st, d)
        print(f"[case] ok {st}: {errs} vs default {d:.2e}", flush=True)


def test_invalid_tile_override_launches_nothing(monkeypatch):
    import mixture_experts_layer_05_amd as moe
    case = Hn.make_case(_INVARIANCE, 64, 77)
    layer = moe.MoELayer(Hn.config(case.shape), case.weights, case.inp.w_router.cuda(),
                         case.inp.w_shared_gate.cuda(), case.shared, max_tokens=64)
    x = case.inp.x.cuda()
    layer.route(x)
    layer.dispatch(64)
    layer.y.fill_(float("nan"))
    torch.cuda.synchronize()
    for bad in ("stream48", "tall", "SPLIT", "1"):
        monkeypatch.setenv("MOE_FORCE_TILE", bad)
        with pytest.raises(moe.MoEError) as ei:
            layer.forward(x)
        assert ei.value.status == -2
    torch.cuda.synchronize()
    assert torch.isnan(layer.y).all()          # nothing was launched


@pytest.mark.parametrize("poison", ["-inf", "nan"])
def test_masked_experts_fewer_finite_than_k(poison):
    """A bias that masks E - K + 2 experts leaves K - 2 finite logits per token: the
    top-k still returns K distinct valid ids (the masked ones after the finite ones,
    lower id first, weight 0), and the layer matches the oracle."""
    shape = W.LayerShape("masked_experts", 256, 8, 256, 4, 128, W.DT_BF16, W.DT_BF16)
    T = 24

    def mask(case):
        # Mask every expert but each token's two largest logits (whose gap the
        # conditioned inputs keep above the top-k margin).
        from oracle import moe as O
        z = O.router_logits(case.inp.x, case.inp.w_router)
        b = torch.zeros(T, shape.n_routed_experts)
        for t in range(T):
            off = np.argsort(-z[t])[2:]
            b[t, torch.as_tensor(off)] = float(poison)
        case.inp.logit_bias = b
    case, gpu, ora, _ = _run(shape, T, 66, mutate=mask)
    ids = gpu["ids"]
    assert ((ids >= 0) & (ids < shape.n_routed_experts)).all()
    assert all(len(set(r)) == len(r) for r in ids.tolist())
    assert (gpu["w"][:, 2:] == 0).all()


# ----------------------------------------------------------------------------- edge cases

EDGE = W.LayerShape("edge_k_eq_e", 256, 4, 256, 4, 128, W.DT_BF16, W.DT_BF16)


# Few experts, many rows each: the LDS-tiled kernels with partial 128- and 256-row
# tiles.  These calls are smaller than the size from which the launcher divides
# rows by itself (T*K*I >= 256 x 256 x 128), so the tile override forces the
# division and the 256-row kernels run at sizes the oracle checks on every token.
TILED = W.LayerShape("tiled_rows", 512, 4, 256, 2, 256, W.DT_BF16, W.DT_BF16)


@pytest.mark.parametrize("dt", [W.DT_BF16, W.DT_FP8, W.DT_MXFP4])
@pytest.mark.parametrize("T", [300, 700])
def test_tiled_kernels_with_partial_tiles(T, dt, monkeypatch):
    monkeypatch.setenv("MOE_FORCE_TILE", "split")
    _run(TILED.with_(name=f"tiled_rows_{dt}", weight_dtype=dt), T, 20 + T + (10 if dt != W.DT_BF16 else 0))


# Rows on both sides of the split between the 256-row LDS-tiled kernel and the
# streaming kernel's 128-row tiles (Zipf-skewed counts: short groups, and long
# groups whose short tails go to the streaming kernel), checked on every token;
# the shared expert (600 rows) runs whole on the tiled kernel.  Forced as above.
MIXED = W.LayerShape("mixed_groups", 512, 8, 256, 2, 256, W.DT_BF16, W.DT_BF16)


@pytest.mark.parametrize("dt", [W.DT_BF16, W.DT_FP8, W.DT_MXFP4])
def test_groups_split_between_kernels_by_rows(dt, monkeypatch):
    monkeypatch.setenv("MOE_FORCE_TILE", "split")
    shape = MIXED.with_(name=f"mixed_groups_{dt}", weight_dtype=dt)
    case, gpu, ora, _ = _run(shape, 600, 61, 1.5)
    counts = gpu["counts"]
    tail = counts % 256
    assert ((counts >= 256) & (tail > 0) & (tail < 128)).any(), counts   # a long group's short tail
    assert ((counts > 0) & (counts < 128)).any(), counts                  # a short group


# 256-row tiles with the shortest contractions the kernels accept (128 elements;
# 256 with MXFP4) and a single n-tile per group.  Forced as above.
SHORT_K = W.LayerShape("tiled_short_k", 256, 2, 128, 1, 128, W.DT_BF16, W.DT_BF16)


def test_tall_tiles_with_short_contractions(monkeypatch):
    monkeypatch.setenv("MOE_FORCE_TILE", "split")
    _run(SHORT_K, 600, 41)


def test_tall_fp8_tiles_with_short_contractions(monkeypatch):
    # fp8 256-row tiles: gate/up over 2 scale groups, down over 1 (a one-stage pipeline).
    monkeypatch.setenv("MOE_FORCE_TILE", "split")
    _run(SHORT_K.with_(name="tiled_short_k_fp8", weight_dtype=W.DT_FP8), 600, 42)


def test_tall_mxfp4_tiles_with_short_contractions(monkeypatch):
    # MXFP4 256-row tiles over two 128-element stages (gate/up and down).
    monkeypatch.setenv("MOE_FORCE_TILE", "split")
    _run(W.LayerShape("tiled_short_k_mxfp4", 256, 2, 256, 1, 256, W.DT_MXFP4, W.DT_BF16), 600, 43)


def test_k_equals_e_with_ragged_tokens():
    _run(EDGE, 13, 5)


def test_single_expert_top1():
    _run(W.LayerShape("one_expert", 128, 1, 128, 1, 0, W.DT_BF16, W.DT_BF16), 5, 6)


def test_single_token():
    _run(W.DRAFTER, 1, 7)


def test_budget_of_one_empties_tokens():
    shape = W.LayerShape("budget1", 256, 8, 128, 2, 0, W.DT_BF16, W.DT_BF16, expert_budget=1)
    case, gpu, ora, _ = _run(shape, 40, 8)
    assert gpu["stats"][1] == 1 and gpu["stats"][3] > 0   # some tokens lose every expert


def test_budget_at_union_is_a_noop():
    shape = W.LayerShape("budget16", 256, 16, 128, 2, 0, W.DT_BF16, W.DT_BF16, expert_budget=16)
    case, gpu, ora, _ = _run(shape, 64, 9)
    assert gpu["stats"].tolist()[1:] == [gpu["stats"][0], 0, 0]


def test_plain_softmax_without_renormalisation():
    shape = W.LayerShape("no_norm", 256, 8, 128, 3, 128, W.DT_BF16, W.DT_BF16, norm_topk_prob=0)
    case, gpu, ora, _ = _run(shape, 33, 10)
    assert (gpu["w"].sum(axis=1) < 1.0).all()


def test_fp8_zero_activation_row():
    shape = W.LayerShape("fp8_zero_row", 256, 8, 256, 2, 128, W.DT_FP8, W.DT_BF16)

    def zero_row(case):
        case.inp.x[3] = 0   # logits exactly 0: ids 0..K-1 by the tie rule; fp8 group amax = 0
    case, gpu, ora, _ = _run(shape, 20, 11, mutate=zero_row)
    assert gpu["ids"][3].tolist() == [0, 1]


def test_zero_tokens_is_a_noop():
    import mixture_experts_layer_05_amd as moe
    case = Hn.make_case(W.DRAFTER.with_(n_routed_experts=16), 0, 1)
    layer = moe.MoELayer(Hn.config(case.shape), case.weights, case.inp.w_router.cuda(),
                         case.inp.w_shared_gate.cuda(), case.shared, max_tokens=4)
    x = torch.empty(0, case.shape.hidden_size, dtype=torch.bfloat16, device="cuda")
    y = layer(x)
    torch.cuda.synchronize()
    assert y.shape == (0, case.shape.hidden_size)
    assert int(layer.offsets[-1].item()) == 0 and int(layer.counts.sum().item()) == 0


def test_routing_is_deterministic():
    case = Hn.make_case(W.NARROW, 56, 12)
    a = Hn.run_gpu(case)
    b = Hn.run_gpu(case)
    for k in ("ids", "w", "counts", "offsets", "perm", "stats"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["y"], b["y"])   # no atomics: bit-reproducible


def test_split_budget_path_is_deterministic():
    """The rows-divided (256-row + streaming) kernels with fp8 weights and the
    expert budget, twice on the same inputs: routing, the budget's keep-set
    (order-independent fixed-point aggregates) and y are bit-identical
    [colibri issue_budget.md, "How it works"]."""
    case = Hn.make_case(W.LARGE_FP8, 512, W.base_seed(4, 512), 1.5)
    a = Hn.run_gpu(case)
    b = Hn.run_gpu(case)
    for k in ("ids", "w", "counts", "offsets", "perm", "stats"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["y"], b["y"])


def test_halves_equal_forward():
    import mixture_experts_layer_05_amd as moe
    case = Hn.make_case(W.DRAFTER, 56, 13)
    layer = moe.MoELayer(Hn.config(case.shape), case.weights, case.inp.w_router.cuda(),
                         case.inp.w_shared_gate.cuda(), case.shared, max_tokens=56)
    x = case.inp.x.cuda()
    bias = case.inp.logit_bias.cuda()
    y1 = layer(x, bias).clone()
    layer.forward(x, half="gate_up")
    layer.forward(x, half="down")
    torch.cuda.synchronize()
    assert Hn.rel_l2(layer.views(56)["y"].cpu().numpy(), y1.cpu().numpy()) < 1e-6


# fp32 with H, I, S not multiples of 4: the combine pass adds and stores element by
# element.
_TINY_ODD = W.TINY.with_(name="tiny_fp32_odd", hidden_size=250, moe_intermediate_size=100,
                         shared_expert_intermediate_size=60)


def test_fp32_layer_with_odd_widths():
    _run(_TINY_ODD, 40, W.base_seed(0, 40) + 23)


@pytest.mark.parametrize("shape,T", [(W.DRAFTER, 56), (W.TINY, 40), (_TINY_ODD, 40)])
@pytest.mark.parametrize("element_aligned", [False, True])
def test_activation_dtype_output(shape, T, element_aligned):
    """The optional y_act output: the cast of the float32 y to the activation dtype.
    element_aligned: y_act starts one element into an allocation, aligned only to
    its element size (the combine pass then stores element by element)."""
    import mixture_experts_layer_05_amd as moe
    print(f"\n[case] y_act {shape.name} T={T} element_aligned={element_aligned}", flush=True)
    case = Hn.make_case(shape, T, 14)
    sg = None if case.inp.w_shared_gate is None else case.inp.w_shared_gate.cuda()
    layer = moe.MoELayer(Hn.config(shape), case.weights, case.inp.w_router.cuda(), sg, case.shared,
                         max_tokens=T, act_output=True)
    if element_aligned:
        buf = torch.empty(T * shape.hidden_size + 1, dtype=layer.y_act.dtype, device="cuda")
        layer.y_act = buf[1:].view(T, shape.hidden_size)
        assert layer.y_act.data_ptr() % 8 != 0
    bias = None if case.inp.logit_bias is None else case.inp.logit_bias.cuda()
    y = layer(case.inp.x.cuda(), bias)
    torch.cuda.synchronize()
    y_act = layer.views(T)["y_act"].cpu()
    y_host = y.cpu()
    if shape.act_dtype == W.DT_BF16:
        # Bit-exact against torch's host cast (round to nearest, ties to even).
        ref = y_host.to(torch.bfloat16)
        assert torch.equal(y_act.view(torch.int16), ref.view(torch.int16))
        # Against the oracle: bf16 rounding adds at most 2^-9 relative error per element.
        ora = Hn.run_oracle(case)
        err = Hn.rel_l2(y_act.float().numpy().astype(np.float64), ora["y"])
        assert err <= Hn.TOL["bf16"] + 2.0 ** -9, err
    else:
        assert torch.equal(y_act, y_host)


# ----------------------------------------------------------------------------- seeded shape sweep

def _sweep_shapes(n=40, seed=7):
    """Small random layers over every dtype, with and without shared expert, budget
    and top-p, sized so that some calls take the decode streaming kernels and some
    the LDS-tiled ones."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = (W.DT_BF16, W.DT_FP8, W.DT_MXFP4, W.DT_F32)[i % 4]
        q = 256 if dt == W.DT_MXFP4 else 128
        H = int(rng.integers(1, 4)) * q if dt != W.DT_MXFP4 else int(rng.integers(1, 3)) * q
        E = int(rng.integers(1, 41))
        K = int(rng.integers(1, min(E, 8) + 1))
        I = min(int(rng.choice([1, 2, 4])) * q, 512)
        S = int(rng.choice([0, 1, 2])) * q
        T = int(rng.choice([1, 5, 37, 100, 300, 640]))
        budget = int(rng.integers(1, E + 1)) if rng.random() < 0.3 else 0
        top_p = float(np.round(rng.uniform(0.3, 0.9), 2)) if rng.random() < 0.3 else 0.0
        act = W.DT_F32 if dt == W.DT_F32 else W.DT_BF16
        shape = W.LayerShape(f"sweep{i}_{dt}", H, E, I, K, S, dt, act, expert_budget=budget, top_p=top_p)
        out.append((shape, T, 500 + i))
    return out


@pytest.mark.parametrize("shape,T,seed", _sweep_shapes(), ids=lambda v: getattr(v, "name", str(v)))
def test_seeded_shape_sweep(shape, T, seed):
    _run(shape, T, seed)


def _large_sweep_shapes(n=9, seed=11):
    """Larger random layers whose calls divide their rows between the 256-row and the
    streaming kernels (bf16, fp8: at least 16 rows per expert and T*K*I of at least
    twice 256 x 256 x 128) or run the 128-row streaming tiles (MXFP4: 128 x 256), with Zipf
    router skew, shared expert, budget and top-p drawn at random.  H is a multiple
    of 512, so the fp8 and MXFP4 decode stages take their widest forms."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = (W.DT_BF16, W.DT_FP8, W.DT_MXFP4)[i % 3]
        H = int(rng.choice([512, 1024, 1536]))
        I = int(rng.choice([512, 1024]))
        E = int(rng.integers(8, 33))
        K = int(rng.integers(2, 9))
        S = int(rng.choice([0, 256, 512]))
        T = int(rng.choice([2048, 3072, 4096]))
        while T * K * I < 2 * 256 * 256 * 128 or T * K // E < 16:
            K = min(K + 1, E)
            T *= 2
        alpha = float(rng.choice([0.0, 1.0, 1.5]))
        budget = int(rng.integers(max(1, E // 2), E + 1)) if rng.random() < 0.3 else 0
        top_p = float(np.round(rng.uniform(0.5, 0.9), 2)) if rng.random() < 0.3 else 0.0
        shape = W.LayerShape(f"lsweep{i}_{dt}", H, E, I, K, S, dt, W.DT_BF16, expert_budget=budget, top_p=top_p)
        out.append((shape, T, 900 + i, alpha))
    return out


@pytest.mark.parametrize("shape,T,seed,alpha", _large_sweep_shapes(), ids=lambda v: getattr(v, "name", str(v)))
def test_seeded_large_shape_sweep(shape, T, seed, alpha):
    _run(shape, T, seed, alpha, tokens=48)


# Row-divided calls from 192 rows per expert give the streaming kernel's share to
# two launches by group: groups left with more than 64 rows (128-row tiles) and the
# rest (64-row tiles, 64 columns wide in narrow gate/up calls), when the former fill
# the GPU.  Both launches must divide alike: 9 such groups in a narrow call (too few
# to divide, although the narrow launch's own tile count would say enough), and 27
# groups' long tails (gate/up divided, down not), bf16 and fp8.
@pytest.mark.parametrize("name,H,E,I,K,S,dt,T,alpha", [
    ("restdiv_narrow_bf16", 1024, 31, 1024, 7, 512, W.DT_BF16, 3072, 1.5),
    ("restdiv_tails_bf16", 1024, 32, 1024, 8, 0, W.DT_BF16, 1360, 0.0),
    ("restdiv_tails_fp8", 1024, 32, 1024, 8, 256, W.DT_FP8, 1360, 0.0),
])
def test_rest_rows_divided_by_group_size(name, H, E, I, K, S, dt, T, alpha):
    shape = W.LayerShape(name, H, E, I, K, S, dt, W.DT_BF16)
    _run(shape, T, 950 + E, alpha, tokens=128)


def test_graph_capture_replays_match_eager():
    """route -> dispatch -> forward captured once into a HIP graph: the library
    launches on the caller's stream with no host synchronisation, copy back or
    allocation.  Each replay (with eager work and synchronisations in between)
    must reproduce the eager result bit for bit."""
    import mixture_experts_layer_05_amd as moe
    shape, T = W.DRAFTER, 56
    case = Hn.make_case(shape, T, W.base_seed(1, T))
    layer = moe.MoELayer(Hn.config(shape), case.weights, case.inp.w_router.cuda(),
                         case.inp.w_shared_gate.cuda(), case.shared, max_tokens=T)
    x, bias = case.inp.x.cuda(), case.inp.logit_bias.cuda()
    eager = layer(x, bias).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(x, bias)                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(x, bias)
    for rep in range(4):
        layer.y.fill_(float("nan"))
        layer.perm.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.y[:T], eager), f"replay {rep} differs from the eager result"
    print(f"[case] ok graph replays x4 bit-exact, T={T}", flush=True)
