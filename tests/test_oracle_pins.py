"""Pins of the CPU oracle against things other than itself: closed forms,
invariants, brute-force enumeration, library routines, and numbers the pages print.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import workloads as W
from oracle import e4m3
from oracle import moe as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val, unit, src = [p.strip() for p in line.split("|")]
        out[key] = (val, unit, src)
    return out


def _printed(val: str) -> float:
    mult = {"M": 1e6, "B": 1e9}
    return float(val[:-1]) * mult[val[-1]] if val[-1] in mult else float(val)


# ----------------------------------------------------------------------------- top-k

def test_topk_weights_sum_to_one():
    rng = np.random.default_rng(1)
    z = rng.normal(size=(50, 16))
    for K in (1, 2, 5, 16):
        _, w = O.topk_softmax(z, K, norm_topk=True)
        assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)


def test_topk_bruteforce_tiny():
    rng = np.random.default_rng(2)
    for trial in range(40):
        E = int(rng.integers(2, 9))
        K = int(rng.integers(1, min(E, 3) + 1))
        T = int(rng.integers(1, 6))
        # distinct integer-spaced logits
        z = np.stack([rng.permutation(E).astype(np.float64) * 0.75 - 2.0 for _ in range(T)])
        ids, w = O.topk_softmax(z, K, norm_topk=True)
        ids0, w0 = O.topk_softmax(z, K, norm_topk=False)
        assert np.array_equal(ids, ids0)
        for t in range(T):
            best = max(itertools.combinations(range(E), K), key=lambda c: sum(z[t, list(c)]))
            assert set(ids[t].tolist()) == set(best)
            assert all(z[t, ids[t, i]] > z[t, ids[t, i + 1]] for i in range(K - 1))
            assert np.allclose(w[t], scipy.special.softmax(z[t, ids[t]]), rtol=0, atol=1e-14)
            assert np.allclose(w0[t], scipy.special.softmax(z[t])[ids[t]], rtol=0, atol=1e-14)


def test_topk_ties_go_to_lower_id():
    z = np.array([[1.0, 3.0, 3.0, 0.0, 3.0]])
    ids, w = O.topk_softmax(z, 2)
    assert ids.tolist() == [[1, 2]]
    assert np.allclose(w, 0.5)


def test_topk_per_token_shift_invariance():
    rng = np.random.default_rng(3)
    z = rng.integers(-20, 20, size=(30, 12)).astype(np.float64) / 4.0
    shift = rng.integers(-8, 8, size=(30, 1)).astype(np.float64)  # exact in binary
    a = O.topk_softmax(z, 3)
    b = O.topk_softmax(z + shift, 3)
    assert np.array_equal(a[0], b[0])
    assert np.allclose(a[1], b[1], atol=1e-15)


# ----------------------------------------------------------------------------- top-p trim

def test_top_p_worked_example():
    # Probabilities 0.5 / 0.3 / 0.2 over three experts: cumulative 0.5, 0.8, 1.0.
    z = np.log(np.array([[0.5, 0.3, 0.2]]))
    ids, w = O.topk_softmax(z, 3)
    for p, keep in ((0.45, 1), (0.7, 2), (0.79, 2), (0.81, 3), (0.99, 3)):
        i2, w2 = O.top_p_trim(z, ids, w, p, norm_topk=True)
        assert i2[0].tolist() == [0, 1, 2][:keep] + [-1] * (3 - keep), p
        assert np.allclose(w2[0, :keep], np.array([0.5, 0.3, 0.2])[:keep] / [0.5, 0.8, 1.0][keep - 1], atol=1e-15)
        assert (w2[0, keep:] == 0).all()
    # Without renormalisation the kept slots keep their softmax probabilities.
    ids0, w0 = O.topk_softmax(z, 3, norm_topk=False)
    i2, w2 = O.top_p_trim(z, ids0, w0, 0.7, norm_topk=False)
    assert i2[0].tolist() == [0, 1, -1]
    assert np.allclose(w2[0], [0.5, 0.3, 0.0], atol=1e-15)


def test_top_p_off_values_are_no_ops():
    rng = np.random.default_rng(11)
    z = rng.normal(size=(20, 9))
    ids, w = O.topk_softmax(z, 4)
    for p in (0.0, 1.0, -0.5, 1.5):
        i2, w2 = O.top_p_trim(z, ids, w, p)
        assert np.array_equal(i2, ids) and np.array_equal(w2, w)


def test_top_p_matches_its_definition_on_random_tokens():
    # Shortest prefix of the descending top-k probabilities whose sum reaches p of
    # their total, computed here in float64 with scipy's softmax; tokens whose
    # prefix sums sit within 1e-4 of the cut are skipped (the oracle decides in
    # float32).
    rng = np.random.default_rng(12)
    checked = 0
    for trial in range(30):
        E, K = int(rng.integers(4, 20)), int(rng.integers(2, 5))
        K = min(K, E)
        z = rng.normal(scale=1.5, size=(40, E))
        p = float(rng.uniform(0.2, 0.95))
        ids, w = O.topk_softmax(z, K)
        i2, w2 = O.top_p_trim(z, ids, w, p)
        for t in range(z.shape[0]):
            probs = scipy.special.softmax(z[t])[ids[t]]
            cums = np.cumsum(probs) / probs.sum()
            if np.min(np.abs(cums[:-1] - p)) < 1e-4:
                continue
            n = int(np.argmax(cums >= p)) + 1
            assert i2[t].tolist() == ids[t, :n].tolist() + [-1] * (K - n)
            assert np.allclose(w2[t, :n], probs[:n] / probs[:n].sum(), atol=1e-13)
            checked += 1
    assert checked > 1000


def test_top_p_keeps_the_first_pick_and_a_prefix():
    rng = np.random.default_rng(13)
    z = rng.normal(scale=3.0, size=(200, 12))
    ids, w = O.topk_softmax(z, 6)
    i2, w2 = O.top_p_trim(z, ids, w, 1e-6)
    assert (i2[:, 0] == ids[:, 0]).all() and (i2[:, 1:] == -1).all() and np.allclose(w2[:, 0], 1.0)
    i3, w3 = O.top_p_trim(z, ids, w, 0.6)
    n = (i3 >= 0).sum(axis=1)
    for t in range(z.shape[0]):
        assert i3[t, :n[t]].tolist() == ids[t, :n[t]].tolist() and (i3[t, n[t]:] == -1).all()
    assert np.allclose(w3.sum(axis=1), 1.0, atol=1e-12)


def test_top_p_per_token_shift_invariance():
    rng = np.random.default_rng(14)
    z = rng.integers(-20, 20, size=(30, 12)).astype(np.float64) / 4.0
    shift = rng.integers(-8, 8, size=(30, 1)).astype(np.float64)  # exact in binary
    a = O.top_p_trim(z, *O.topk_softmax(z, 4), 0.55)
    b = O.top_p_trim(z + shift, *O.topk_softmax(z + shift, 4), 0.55)
    assert np.array_equal(a[0], b[0]) and np.allclose(a[1], b[1], atol=1e-15)


def test_top_p_runs_before_the_budget():
    # Token 0 routes 0.55 / 0.45 to experts 0 / 1, tokens 1-2 route 0.9 / 0.1 to
    # experts 2 / 1.  Budget 2 on the untrimmed routing keeps {1, 2} (aggregates
    # 0.65 and 1.8 against 0.55 for expert 0); with top-p 0.8 first, tokens 1-2
    # drop expert 1 and the budget keeps {0, 2} instead.
    wr = np.log(np.array([[0.55, 1e-9, 1e-9], [0.45, 0.1, 0.1], [1e-9, 0.9, 0.9]]))
    x = np.array([[1.0, 0, 0], [0, 1.0, 0], [0, 0, 1.0]])
    r_plain = O.route(x, wr, None, None, 2, True, 2, 0.0)
    r_topp = O.route(x, wr, None, None, 2, True, 2, 0.8)
    assert set(r_plain["ids"].ravel().tolist()) - {-1} == {1, 2}
    assert set(r_topp["ids"].ravel().tolist()) - {-1} == {0, 2}
    assert r_topp["ids"].tolist() == [[0, -1], [2, -1], [2, -1]]
    assert r_topp["stats"].tolist() == [3, 2, 1, 0]


# ----------------------------------------------------------------------------- budget

def _random_routing(rng, T, E, K):
    z = rng.normal(size=(T, E))
    return z, *O.topk_softmax(z, K)


def test_budget_noop_when_off_or_at_or_above_union():
    rng = np.random.default_rng(4)
    _, ids, w = _random_routing(rng, 40, 16, 3)
    nu = len(set(ids.ravel().tolist()))
    for B in (0, nu, nu + 1, 10 * nu):
        i2, w2, st = O.expert_budget(ids, w, B)
        assert np.array_equal(i2, ids) and np.array_equal(w2, w)
        assert st.tolist() == [nu, nu, 0, 0]


def test_budget_bruteforce_tiny():
    rng = np.random.default_rng(5)
    for trial in range(25):
        T, E, K = int(rng.integers(2, 6)), int(rng.integers(4, 9)), 2
        z, ids, w = _random_routing(rng, T, E, K)
        U = sorted(set(ids.ravel().tolist()))
        if len(U) < 2:
            continue
        B = int(rng.integers(1, len(U)))
        i2, w2, st = O.expert_budget(ids, w, B)
        agg = {e: w[ids == e].sum() for e in U}
        best = max(itertools.combinations(U, B), key=lambda c: sum(agg[e] for e in c))
        kept = set(i2.ravel().tolist()) - {-1}
        assert kept == set(best)
        assert st[0] == len(U) and st[1] == B
        for t in range(T):
            kt = [e for e in ids[t].tolist() if e in kept]
            assert i2[t, :len(kt)].tolist() == kt            # original order, compacted
            assert (i2[t, len(kt):] == -1).all() and (w2[t, len(kt):] == 0).all()
            if kt:  # renormalised kept weights = softmax over the token's kept logits
                assert np.allclose(w2[t, :len(kt)], scipy.special.softmax(z[t, kt]), atol=1e-13)
        assert st[2] == (ids >= 0).sum() - (i2 >= 0).sum()
        assert st[3] == int(((i2 >= 0).sum(axis=1) == 0).sum())


def test_budget_token_loses_every_expert():
    ids = np.array([[0, 1], [0, 1], [2, 3]], dtype=np.int32)
    w = np.array([[0.6, 0.4], [0.7, 0.3], [0.55, 0.45]])
    i2, w2, st = O.expert_budget(ids, w, 2)
    assert i2.tolist() == [[0, 1], [0, 1], [-1, -1]]
    assert w2[2].tolist() == [0.0, 0.0]
    assert st.tolist() == [4, 2, 2, 1]


def test_budget_without_norm_topk_keeps_raw_weights():
    ids = np.array([[0, 1], [2, 1]], dtype=np.int32)
    w = np.array([[0.5, 0.2], [0.1, 0.3]])
    i2, w2, st = O.expert_budget(ids, w, 2, norm_topk=False)
    assert i2.tolist() == [[0, 1], [1, -1]]
    assert w2.tolist() == [[0.5, 0.2], [0.3, 0.0]]


# ----------------------------------------------------------------------------- routing statistics from the pages

def test_union_of_16_experts_top2_block7_is_at_most_14():
    g = _golden()
    assert int(g["max_experts_touched_16_top2_block7"][0]) == 14
    shape = W.DRAFTER
    sizes = []
    for seed in range(6):
        inp = W.layer_inputs(shape, 224, 777 + seed)
        z = O.router_logits(inp.x, inp.w_router, inp.logit_bias)
        ids, _ = O.topk_softmax(z, shape.num_experts_per_tok)
        for b in range(0, 224, 7):
            sizes.append(len(set(ids[b:b + 7].ravel().tolist())))
    assert max(sizes) <= 14 and min(sizes) >= 2
    assert max(sizes) >= 11 and min(sizes) <= 4   # the block bias spreads the union over 2..14


def test_uniform_routing_512_top10_block7_union():
    g = _golden()
    printed = float(g["experts_touched_512_top10_block7"][0])
    E, K, T = 512, 10, 7
    closed = E * (1 - (1 - K / E) ** T)                # 65.96 for independent uniform picks
    rng = np.random.default_rng(6)
    sizes = []
    for _ in range(300):
        ids, _ = O.topk_softmax(rng.normal(size=(T, E)), K)
        sizes.append(len(set(ids.ravel().tolist())))
    mean = float(np.mean(sizes))
    assert abs(mean - closed) < 1.0
    assert abs(mean - printed) < 2.5
    # ~1 GB of expert weights per step vs 0.53 GB dense (bf16, H = 5120)
    per_expert = 3 * 5120 * 512 * 2
    assert abs(printed * per_expert / 1e9 - float(g["expert_bytes_512x512_top10_block7"][0])) < 0.1
    assert abs(267_386_880 * 2 / 1e9 - float(g["dense_ffn_bytes"][0])) < 0.01


def _ffn_params(H, I, E, S):
    return 3 * H * I * E + 3 * H * S


@pytest.mark.parametrize("key,H,I,E,K,S,which", [
    ("ffn_params_16x1024_top2_shared2048", 5120, 1024, 16, 2, 2048, "all"),
    ("active_params_16x1024_top2_shared2048", 5120, 1024, 16, 2, 2048, "active"),
    ("ffn_params_16x2048_top2_shared2048", 5120, 2048, 16, 2, 2048, "all"),
    ("active_params_16x2048_top2_shared2048", 5120, 2048, 16, 2, 2048, "active"),
    ("active_params_16x2048_top4_shared2048", 5120, 2048, 16, 4, 2048, "active"),
    ("ffn_params_512x512_top10_shared2048", 5120, 512, 512, 10, 2048, "all"),
    ("active_params_512x512_top10_shared2048", 5120, 512, 512, 10, 2048, "active"),
    ("dense_ffn_params_17408", 5120, 17408, 1, 1, 0, "all"),
])
def test_parameter_counts_match_the_pages(key, H, I, E, K, S, which):
    """SwiGLU with three bias-free matrices per expert reproduces every printed count."""
    val, _, _ = _golden()[key]
    n = _ffn_params(H, I, E, S) if which == "all" else _ffn_params(H, I, K, S)
    digits = len(val.rstrip("MB").split(".")[-1]) if "." in val else 0
    scale = 1e9 if val.endswith("B") else 1e6
    assert round(n / scale, digits) == _printed(val) / scale


def test_workload_shapes_have_the_drafter_parameter_count():
    shape = W.DRAFTER
    w0 = W.expert_weights(shape, 1, 0)
    sh = W.shared_expert_weights(shape, 1)
    n = shape.n_routed_experts * sum(w0[k].numel() for k in ("gate", "up", "down"))
    n += sum(sh[k].numel() for k in ("gate", "up", "down"))
    assert n == 283_115_520
    active = shape.num_experts_per_tok * sum(w0[k].numel() for k in ("gate", "up", "down")) \
        + sum(sh[k].numel() for k in ("gate", "up", "down"))
    assert active == 62_914_560


# ----------------------------------------------------------------------------- dispatch

def test_dispatch_matches_library_sort():
    rng = np.random.default_rng(7)
    for T, E, K in ((1, 1, 1), (13, 8, 3), (200, 64, 6), (64, 512, 10)):
        z = rng.normal(size=(T, E))
        ids, w = O.topk_softmax(z, K)
        if T > 10:  # drop some slots the way the budget does
            ids, w, _ = O.expert_budget(ids, w, max(1, E // 3))
        counts, offsets, perm = O.dispatch(ids, E)
        kept = np.nonzero(ids.ravel() >= 0)[0]
        e = ids.ravel()[kept].astype(np.int64)
        t = kept // K
        expect = kept[np.argsort(e * T + t, kind="stable")]
        assert np.array_equal(perm, expect)
        assert np.array_equal(counts, np.bincount(e, minlength=E))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(e, minlength=E))]))


# ----------------------------------------------------------------------------- expert math

def _torch_swiglu(x, wd):
    x = torch.as_tensor(x, dtype=torch.float64)
    g = torch.as_tensor(O.as_f64(wd["gate"]))
    u = torch.as_tensor(O.as_f64(wd["up"]))
    d = torch.as_tensor(O.as_f64(wd["down"]))
    return torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(x, g))
                                      * torch.nn.functional.linear(x, u), d).numpy()


def _tiny_layer(E=6, H=32, I=24, S=0, seed=8):
    rng = np.random.default_rng(seed)
    experts = [{k: rng.normal(scale=0.2, size=s) for k, s in
                (("gate", (I, H)), ("up", (I, H)), ("down", (H, I)))} for _ in range(E)]
    shared = None if S == 0 else {k: rng.normal(scale=0.2, size=s) for k, s in
                                  (("gate", (S, H)), ("up", (S, H)), ("down", (H, S)))}
    return rng, experts, shared


def test_identical_experts_reduce_to_one_dense_ffn():
    rng, experts, shared = _tiny_layer(E=5, S=16)
    same = experts[0]
    T, H = 9, 32
    x = rng.normal(size=(T, H))
    wr = rng.normal(size=(5, H))
    wgate = rng.normal(size=H)
    r = O.moe_layer(x, wr, wgate, None, 2, 5, lambda e: same, shared, "f32")
    sg = 1 / (1 + np.exp(-(x @ wgate)))
    expect = _torch_swiglu(x, same) + sg[:, None] * _torch_swiglu(x, shared)
    assert np.allclose(r["y"], expect, rtol=1e-12, atol=1e-12)


def test_single_expert_top1_is_the_ffn():
    rng, experts, _ = _tiny_layer(E=1)
    x = rng.normal(size=(7, 32))
    r = O.moe_layer(x, rng.normal(size=(1, 32)), None, None, 1, 1, lambda e: experts[e], None, "f32")
    assert np.allclose(r["y"], _torch_swiglu(x, experts[0]), rtol=1e-12, atol=1e-12)
    assert r["w"].ravel().tolist() == [1.0] * 7


def test_layer_equals_dense_masked_mixture():
    """y = sum_e gate[t,e] * FFN_e(x_t) with the gate matrix built by torch.topk + softmax."""
    rng, experts, shared = _tiny_layer(E=6, S=8, seed=9)
    T, H, K = 11, 32, 3
    x = rng.normal(size=(T, H))
    wr = rng.normal(size=(6, H))
    wgate = rng.normal(size=H)
    r = O.moe_layer(x, wr, wgate, None, K, 6, lambda e: experts[e], shared, "f32")
    z = torch.as_tensor(x @ wr.T)
    top = torch.topk(z, K, dim=1)
    gate = torch.zeros_like(z).scatter(1, top.indices, torch.softmax(top.values, dim=1)).numpy()
    expect = sum(gate[:, e:e + 1] * _torch_swiglu(x, experts[e]) for e in range(6))
    expect = expect + torch.sigmoid(torch.as_tensor(x @ wgate)).numpy()[:, None] * _torch_swiglu(x, shared)
    assert np.allclose(r["y"], expect, rtol=1e-11, atol=1e-12)
    # subset evaluation equals the full evaluation row by row
    sub = [10, 0, 5]
    r2 = O.moe_combine(x, r["ids"], r["w"], r["shared_gate"], lambda e: experts[e], shared, "f32", sub)
    assert np.allclose(r2, r["y"][sub], rtol=1e-13, atol=1e-14)


def test_token_with_no_kept_expert_and_no_shared_is_exactly_zero():
    rng, experts, _ = _tiny_layer(E=4, seed=10)
    x = rng.normal(size=(3, 32))
    ids = np.array([[0, 1], [-1, -1], [2, -1]], dtype=np.int32)
    w = np.array([[0.5, 0.5], [0.0, 0.0], [1.0, 0.0]])
    y = O.moe_combine(x, ids, w, None, lambda e: experts[e], None, "f32")
    assert (y[1] == 0).all() and (y[0] != 0).all()


# ----------------------------------------------------------------------------- e4m3 codec (OCP spec)

def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3.decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_on_dense_sweep():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.uniform(-448, 448, 200_000),
        rng.normal(scale=0.01, size=100_000),
        np.exp2(rng.uniform(-12, 8.8, 100_000)) * rng.choice([-1, 1], 100_000),
        e4m3.decode(np.arange(256, dtype=np.uint8)[[c for c in range(256) if c not in (0x7F, 0xFF)]]),
    ]).astype(np.float32)
    # exact midpoints between neighbouring codes exercise ties-to-even
    fin = np.sort(np.unique(e4m3.decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    v = np.clip(np.concatenate([v, mids, -mids]), -448, 448).astype(np.float32)
    mine = e4m3.encode_rne(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    same = (mine == ref) | ((mine & 0x7F) == 0) & ((ref & 0x7F) == 0)
    assert same.all(), v[~same][:10]


def test_e4m3_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for s in (1.0, 2.0 ** -7, 2.0 ** 5):
        back = e4m3.encode_rne(e4m3.decode(codes) * s / s)
        assert np.array_equal(back, codes)


def test_quantise_group128_bounds_and_special_cases():
    rng = np.random.default_rng(12)
    v = rng.normal(size=(5, 384)).astype(np.float32)
    v[2, 128:256] = 0.0
    q, s = e4m3.quantise_group128(v)
    assert s.shape == (5, 3) and s[2, 1] == 1.0 and (q[2, 128:256] & 0x7F == 0).all()
    d = e4m3.dequantise_group128(q, s)
    # at most half an e4m3 step of the scaled value (3 mantissa bits; 2^-9 in the subnormal range),
    # plus the float32 rounding of v / s
    sr = np.repeat(s, 128, axis=1).astype(np.float64)
    a = np.abs(v / sr)
    step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(a, 1e-30))) - 3), 2.0 ** -9)
    assert (np.abs(d - v) <= sr * (step / 2 + a * 2.0 ** -23)).all()
    # the amax element of each non-zero group lands on +-448 (or its neighbour under fp32 rounding of s)
    amax_codes = np.abs(e4m3.decode(q)).reshape(5, 3, 128).max(axis=2)
    assert ((amax_codes[s != 1.0] >= 416) & (amax_codes[s != 1.0] <= 448)).all()


def test_fp8_swiglu_matches_torch_float8_pipeline():
    """The fp8 expert path vs the same pipeline built from torch's float8_e4m3fn casts."""
    shape = W.LARGE_FP8.with_(hidden_size=256, moe_intermediate_size=256)
    wd = W.expert_weights(shape, 3, 0)
    x = torch.randn(6, 256, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    mine = O.swiglu_ffn(O.as_f64(x), wd, "fp8_e4m3_g128")

    def tq(v):  # torch: fp32 amax/448, fp32 divide, clamp, float8 cast, dequantise in float64
        v = v.to(torch.float32).reshape(v.shape[0], -1, 128)
        amax = v.abs().amax(dim=2, keepdim=True)
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (v / s).clamp(-448, 448).to(torch.float8_e4m3fn)
        return (q.to(torch.float64) * s.to(torch.float64)).reshape(v.shape[0], -1)

    def tw(name):
        q = wd[name].view(torch.float8_e4m3fn).to(torch.float64)
        s = wd[name + "_s"].to(torch.float64)
        return (q.reshape(q.shape[0], -1, 128) * s[:, :, None]).reshape(q.shape)

    xa = tq(x)
    a = xa @ tw("gate").T
    b = xa @ tw("up").T
    h = torch.nn.functional.silu(a) * b
    ref = tq(h.to(torch.float32)) @ tw("down").T
    assert np.allclose(mine, ref.numpy(), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- router bias, NaN logits

def test_logit_bias_is_added_to_the_logits():
    """A one-hot bias of +20 on expert e must make e the first pick of that token
    (a subtracted bias would make it the last), and a -inf bias masks an expert."""
    rng = np.random.default_rng(30)
    T, H, E, K = 12, 16, 8, 2
    x = rng.normal(size=(T, H))
    wr = rng.normal(scale=0.1, size=(E, H))
    target = rng.integers(0, E, size=T)
    bias = np.zeros((T, E))
    bias[np.arange(T), target] = 20.0
    r = O.route(x, wr, None, bias, K)
    assert np.array_equal(r["ids"][:, 0], target)
    assert np.allclose(r["logits"] - x @ wr.T, bias)
    masked = np.zeros((T, E))
    masked[:, 0] = -np.inf
    r0 = O.route(x, wr, None, None, K)
    r1 = O.route(x, wr, None, masked, K)
    assert not (r1["ids"] == 0).any()
    keep = (r0["ids"] != 0).all(axis=1)        # tokens whose picks never included expert 0
    assert np.array_equal(r1["ids"][keep], r0["ids"][keep])


def test_nan_logits_count_as_minus_infinity():
    rng = np.random.default_rng(31)
    z = rng.normal(size=(20, 10))
    z[:, [1, 4, 7]] = np.nan
    z[3, :] = np.nan
    z[3, 5] = 0.5                               # one finite expert: the other picks follow by id
    ref = np.where(np.isnan(z), -np.inf, z)
    for K in (2, 8):
        a = O.topk_softmax(z, K)
        b = O.topk_softmax(ref, K)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    ids, w = O.topk_softmax(z, 3)
    assert ids[3].tolist() == [5, 0, 1] and w[3].tolist() == [1.0, 0.0, 0.0]
    # brute force on the finite experts: the picks maximise the summed finite logits first
    for t in range(20):
        if t == 3:
            continue
        fin = [e for e in range(10) if not np.isnan(z[t, e])]
        best = max(itertools.combinations(fin, 2), key=lambda c: sum(z[t, list(c)]))
        assert set(O.topk_softmax(z[t:t + 1], 2)[0][0].tolist()) == set(best)


# ----------------------------------------------------------------------------- bf16 rounding, output variants

def test_round_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(32)
    v = np.concatenate([
        rng.normal(scale=0.05, size=200_000),
        np.exp2(rng.uniform(-140, 127.9, 100_000)) * rng.choice([-1, 1], 100_000),
        [0.0, -0.0, 1.0, 3.3895313892515355e38, 3.4e38, -3.4e38, 1e-45, 2.0 ** -126, 2.0 ** -133],
    ]).astype(np.float32)
    # exact ties between neighbouring bf16 values: bf16 bits b and b+1 share the top 16 bits of a float32
    bits = rng.integers(0, 0x7F7F, size=50_000, dtype=np.uint32)
    ties = ((bits << 16) | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties])
    mine = O.round_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)


def test_round_bf16_rounds_float64_once():
    # 1 + 2^-8 is the midpoint of bf16 1 and 1 + 2^-7; a hair above it must round up.
    # Rounding to float32 first (spacing 2^-23) would land on the midpoint and tie to 1.
    assert O.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert O.round_bf16(1.0 + 2.0 ** -8 - 2.0 ** -40) == 1.0
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0                      # tie to even
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2 * 2.0 ** -7  # tie to even (up)
    assert np.isinf(O.round_bf16(3.4e38)) and O.round_bf16(np.inf) == np.inf
    assert np.isnan(O.round_bf16(np.nan))


def test_bf16_h_variant_rounds_h_before_down():
    """The diagnostic variant equals torch's pipeline: h = silu(a) * b in float64,
    cast to bfloat16 (through float32, checked to be away from any bf16 tie so that
    the two roundings agree), then the down contraction in float64."""
    rng, experts, shared = _tiny_layer(E=3, H=32, I=24, S=16, seed=33)
    T = 10
    x = rng.normal(size=(T, 32))
    wr = rng.normal(size=(3, 32))
    wgate = rng.normal(size=32)
    r = O.moe_layer(x, wr, wgate, None, 2, 3, lambda e: experts[e], shared, "f32",
                    variants=["bf16_h", "plain"])
    assert np.array_equal(r["y_plain"], r["y"])      # no activation quantisation with f32 weights

    def torch_ffn(xr, wdict):
        xt = torch.as_tensor(xr)
        h = torch.nn.functional.silu(xt @ torch.as_tensor(wdict["gate"]).T) * (xt @ torch.as_tensor(wdict["up"]).T)
        h32 = h.to(torch.float32)
        # away from ties: h lies closer to its bf16 value than the float32 step can
        # move it (half a bf16 step is 2^(e-9) for h = m 2^e, 0.5 <= |m| < 1)
        hn = h.numpy()
        half = np.ldexp(1.0, np.frexp(hn)[1] - 9)
        to_mid = half - np.abs(hn - h.to(torch.bfloat16).to(torch.float64).numpy())
        assert (np.abs(hn - h32.to(torch.float64).numpy()) < to_mid).all()
        return (h32.to(torch.bfloat16).to(torch.float64) @ torch.as_tensor(wdict["down"]).T).numpy()

    expect = np.zeros((T, 32))
    for t in range(T):
        for k in range(2):
            e = int(r["ids"][t, k])
            expect[t] += r["w"][t, k] * torch_ffn(x[t:t + 1], experts[e])[0]
    expect += r["shared_gate"][:, None] * torch_ffn(x, shared)
    assert np.allclose(r["y_bf16_h"], expect, rtol=1e-12, atol=1e-13)
    # bf16 h moves y by about the bf16 step (2^-9 relative per element of h)
    rel = np.linalg.norm(r["y_bf16_h"] - r["y"]) / np.linalg.norm(r["y"])
    assert 1e-4 < rel < 2.0 ** -8


def test_plain_variant_leaves_fp8_activations_unquantised():
    """fp8 weights: "plain" is the layer of the dequantised weights (torch float8
    decode) on unquantised activations; "model" quantises x and h as well."""
    shape = W.LARGE_FP8.with_(hidden_size=256, moe_intermediate_size=256)
    wd = W.expert_weights(shape, 4, 0)
    x = torch.randn(5, 256, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)

    def tw(name):
        q = wd[name].view(torch.float8_e4m3fn).to(torch.float64)
        s = wd[name + "_s"].to(torch.float64)
        return (q.reshape(q.shape[0], -1, 128) * s[:, :, None]).reshape(q.shape)

    xt = x.to(torch.float64)
    h = torch.nn.functional.silu(xt @ tw("gate").T) * (xt @ tw("up").T)
    ref = (h @ tw("down").T).numpy()
    plain = O.swiglu_ffn(O.as_f64(x), wd, "fp8_e4m3_g128", quantise_acts=False)
    model = O.swiglu_ffn(O.as_f64(x), wd, "fp8_e4m3_g128")
    assert np.allclose(plain, ref, rtol=1e-12, atol=1e-14)
    rel = np.linalg.norm(model - plain) / np.linalg.norm(plain)
    assert 5e-3 < rel < 0.1        # the activation quantisation error, a few percent
