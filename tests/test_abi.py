"""The C-ABI library: it loads, exports every declared entry point, and rejects
invalid arguments with the documented status before launching anything.
These calls never reach a kernel, so they run without a GPU."""
import ctypes
import re

import pytest

import mixture_experts_layer_05_amd as moe

OK, NULL_PTR, BAD_SHAPE, BAD_DTYPE, UNSUPPORTED, WS_SMALL = 0, -1, -2, -3, -4, -5


def _declared_functions():
    text = open(moe.HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_entry_points():
    assert set(_declared_functions()) == set(moe.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.moe_version() == 0x000100
    for st in (0, -1, -2, -3, -4, -5, -6, -7, 99):
        assert moe.status_string(st)


def _cfg(**kw):
    base = dict(hidden_size=5120, n_routed_experts=16, moe_intermediate_size=1024, num_experts_per_tok=2,
                shared_expert_intermediate_size=2048, weight_dtype="bf16", act_dtype="bf16",
                norm_topk_prob=1, expert_budget=0)
    base.update(kw)
    return moe.MoEConfig(**base)


def _ws(cfg, T=4):
    n = ctypes.c_size_t(0)
    st = moe.lib().moe_workspace_size(ctypes.byref(cfg.c()), T, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    ({}, OK),
    (dict(num_experts_per_tok=17, n_routed_experts=32), UNSUPPORTED),
    (dict(num_experts_per_tok=3, n_routed_experts=2), BAD_SHAPE),
    (dict(n_routed_experts=513), UNSUPPORTED),
    (dict(n_routed_experts=0), BAD_SHAPE),
    (dict(hidden_size=0), BAD_SHAPE),
    (dict(hidden_size=5000), UNSUPPORTED),
    (dict(weight_dtype="fp8_e4m3_g128", moe_intermediate_size=1000), UNSUPPORTED),
    (dict(shared_expert_intermediate_size=100), UNSUPPORTED),
    (dict(weight_dtype="mxfp4"), OK),
    (dict(weight_dtype="mxfp4", moe_intermediate_size=384), UNSUPPORTED),
    (dict(weight_dtype="mxfp4", shared_expert_intermediate_size=128), UNSUPPORTED),
    (dict(weight_dtype="mxfp4", act_dtype="f32"), BAD_DTYPE),
    (dict(weight_dtype="f32"), BAD_DTYPE),
    (dict(act_dtype="f32", weight_dtype="fp8_e4m3_g128"), BAD_DTYPE),
    (dict(act_dtype="fp8_e4m3_g128", weight_dtype="fp8_e4m3_g128"), BAD_DTYPE),
    (dict(expert_budget=-1), BAD_SHAPE),
    (dict(norm_topk_prob=2), BAD_SHAPE),
    (dict(shared_expert_intermediate_size=-128), BAD_SHAPE),
    (dict(weight_dtype="f32", act_dtype="f32", hidden_size=100, moe_intermediate_size=30), OK),
    (dict(top_p=0.0), OK),
    (dict(top_p=0.7), OK),
    (dict(top_p=1.0), OK),
    (dict(top_p=-0.1), BAD_SHAPE),
    (dict(top_p=1.5), BAD_SHAPE),
    (dict(top_p=float("nan")), BAD_SHAPE),
])
def test_workspace_size_validation(kw, status):
    assert _ws(_cfg(**kw))[0] == status


def test_workspace_size_null_arguments_and_tokens():
    lib = moe.lib()
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(None, 4, ctypes.byref(n)) == NULL_PTR
    assert lib.moe_workspace_size(ctypes.byref(_cfg().c()), 4, None) == NULL_PTR
    assert lib.moe_workspace_size(ctypes.byref(_cfg().c()), -1, ctypes.byref(n)) == BAD_SHAPE
    a, b = _ws(_cfg(), 7)[1], _ws(_cfg(), 224)[1]
    assert 0 < a < b


FAKE = 0x1000  # never dereferenced: every call below returns before any launch


def _route(cfg, T=4, ws_bytes=None, **ptrs):
    p = dict(x=FAKE, w_router=FAKE, w_shared_gate=FAKE, logit_bias=None, ids=FAKE, w=FAKE, sg=FAKE,
             stats=None, ws=FAKE)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = _ws(cfg, max(T, 0))[1]
    return moe.lib().moe_route(ctypes.byref(cfg.c()), T, p["x"], p["w_router"], p["w_shared_gate"],
                               p["logit_bias"], p["ids"], p["w"], p["sg"], p["stats"], p["ws"], ws_bytes,
                               None)


def test_route_validation():
    cfg = _cfg()
    assert _route(cfg, x=None) == NULL_PTR
    assert _route(cfg, w_router=None) == NULL_PTR
    assert _route(cfg, ids=None) == NULL_PTR
    assert _route(cfg, w_shared_gate=None) == NULL_PTR     # S > 0 needs the gate vector
    assert _route(cfg, sg=None) == NULL_PTR
    assert _route(cfg, ws=None) == NULL_PTR
    assert _route(cfg, T=4, ws_bytes=16) == WS_SMALL
    assert _route(cfg, T=-2) == BAD_SHAPE
    assert _route(cfg, T=0) == OK                           # nothing to do, nothing launched
    assert _route(_cfg(shared_expert_intermediate_size=0), T=0, w_shared_gate=None, sg=None) == OK


def _forward(cfg, T=4, name="moe_forward", y=FAKE, **ptrs):
    w = moe._Weights(FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE, None, None, None)
    for k, v in ptrs.items():
        if hasattr(w, k):
            setattr(w, k, v)
    g = lambda k: ptrs.get(k, FAKE)  # noqa: E731
    return getattr(moe.lib(), name)(ctypes.byref(cfg.c()), T, g("x"), g("topk_w"), g("shared_gate"),
                                    g("counts"), g("offsets"), g("perm"), ctypes.byref(w), y,
                                    ptrs.get("y_act"), g("ws"), _ws(cfg, max(T, 0))[1], None)


def test_forward_validation():
    cfg = _cfg()
    for name in ("moe_forward", "moe_forward_gate_up", "moe_forward_down"):
        assert _forward(cfg, name=name, x=None) == NULL_PTR
        assert _forward(cfg, name=name, counts=None) == NULL_PTR
        assert _forward(cfg, name=name, ws_down=None) == NULL_PTR
        assert _forward(cfg, name=name, shared_gate=None) == NULL_PTR
        assert _forward(cfg, name=name, y=FAKE + 4) == UNSUPPORTED       # y must be 16-byte aligned
        assert _forward(cfg, name=name, T=0) == OK
    # The optional bf16 output: 2-byte aligned (checked before anything launches).
    assert _forward(cfg, name="moe_forward_down", y_act=FAKE + 1) == UNSUPPORTED
    fp8 = _cfg(weight_dtype="fp8_e4m3_g128")
    assert _forward(fp8) == NULL_PTR                                      # scales missing
    assert _forward(_cfg(shared_expert_intermediate_size=0), T=0, ws_gate=None, ws_up=None,
                    ws_down=None, shared_gate=None) == OK


def test_forward_size_limit():
    # x and the intermediate activations are addressed with 32-bit offsets: each
    # must stay below 3 GiB, checked before anything launches.
    big = dict(hidden_size=7168, moe_intermediate_size=2048, n_routed_experts=256, num_experts_per_tok=8,
               shared_expert_intermediate_size=0)
    for name in ("moe_forward", "moe_forward_gate_up", "moe_forward_down"):
        # h: 110000 * 8 * 2048 bf16 = 3.6 GB
        assert _forward(_cfg(**big), T=110000, name=name, ws_gate=None, ws_up=None, ws_down=None,
                        shared_gate=None) == UNSUPPORTED
        # x: 230000 * 7168 bf16 = 3.3 GB
        assert _forward(_cfg(**dict(big, moe_intermediate_size=128, num_experts_per_tok=1)), T=230000,
                        name=name, ws_gate=None, ws_up=None, ws_down=None, shared_gate=None) == UNSUPPORTED


def test_dispatch_validation():
    lib = moe.lib()
    cfg = _cfg()
    ws = _ws(cfg)[1]
    assert lib.moe_dispatch(ctypes.byref(cfg.c()), 4, None, FAKE, FAKE, FAKE, FAKE, ws, None) == NULL_PTR
    assert lib.moe_dispatch(ctypes.byref(cfg.c()), 4, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None) == WS_SMALL
    assert lib.moe_dispatch(ctypes.byref(cfg.c()), -1, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == BAD_SHAPE


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(ImportError):
        moe.lib()


@pytest.mark.parametrize("kw", [
    {},
    dict(weight_dtype="fp8_e4m3_g128"),
    dict(weight_dtype="mxfp4"),
    dict(n_routed_experts=256, moe_intermediate_size=2048, num_experts_per_tok=8, hidden_size=7168,
         shared_expert_intermediate_size=0),
    dict(weight_dtype="f32", act_dtype="f32", hidden_size=256, n_routed_experts=8, moe_intermediate_size=512,
         shared_expert_intermediate_size=0),
])
def test_workspace_size_is_monotone_in_tokens(kw):
    # A workspace sized for max_tokens must serve every smaller call.
    cfg = _cfg(**kw)
    sizes = []
    for T in (1, 2, 7, 56, 224, 255, 256, 257, 1000, 1024, 1025, 4096, 8192):
        st, n = _ws(cfg, T)
        assert st == OK
        sizes.append(n)
    assert all(b >= a for a, b in zip(sizes, sizes[1:])), sizes


@pytest.mark.parametrize("value,kw,status", [
    ("bogus", {}, BAD_SHAPE),
    ("stream48", {}, BAD_SHAPE),
    ("Split", {}, BAD_SHAPE),
    ("stream16", dict(weight_dtype="f32", act_dtype="f32"), BAD_SHAPE),
    ("split", dict(weight_dtype="f32", act_dtype="f32"), BAD_SHAPE),
])
def test_tile_override_rejects_bad_values_before_launching(monkeypatch, value, kw, status):
    # The bench-only tile override fails loudly: every forward entry point returns
    # the status before touching a pointer (FAKE pointers are never dereferenced).
    monkeypatch.setenv("MOE_FORCE_TILE", value)
    cfg = _cfg(**kw)
    extra = {} if cfg.weight_dtype != "mxfp4" else dict(s_gate=FAKE, s_up=FAKE, s_down=FAKE,
                                                          ss_gate=FAKE, ss_up=FAKE, ss_down=FAKE)
    for name in ("moe_forward", "moe_forward_gate_up", "moe_forward_down"):
        assert _forward(cfg, name=name, **extra) == status
        assert _forward(cfg, T=0, name=name, **extra) == status


@pytest.mark.parametrize("value", ["", "auto", "stream16", "stream32", "stream64", "stream128", "split"])
@pytest.mark.parametrize("wdt", ["bf16", "fp8_e4m3_g128", "mxfp4"])
def test_tile_override_accepts_documented_values(monkeypatch, value, wdt):
    monkeypatch.setenv("MOE_FORCE_TILE", value)
    cfg = _cfg(weight_dtype=wdt)
    extra = {} if wdt == "bf16" else dict(s_gate=FAKE, s_up=FAKE, s_down=FAKE,
                                          ss_gate=FAKE, ss_up=FAKE, ss_down=FAKE)
    for name in ("moe_forward", "moe_forward_gate_up", "moe_forward_down"):
        assert _forward(cfg, T=0, name=name, **extra) == OK


def test_noalloc_forward_checks_before_launching():
    """moe_forward_noalloc: moe_forward's argument checks, then the workspace the
    call needs against the 64 MiB static scratch, all before any HIP call."""
    lib = moe.lib()
    cfg = _cfg()
    w = moe._Weights(FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE, None, None, None)

    def call(c, T, x=FAKE, y=FAKE):
        return lib.moe_forward_noalloc(ctypes.byref(c.c()), T, x, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       ctypes.byref(w), y, None, None)
    assert call(cfg, 4, x=None) == NULL_PTR
    assert call(cfg, 4, y=FAKE + 4) == UNSUPPORTED
    assert call(cfg, -1) == BAD_SHAPE
    assert call(cfg, 0) == OK
    # The drafter layer at T = 224 fits; at T = 4096 it needs more than 64 MiB.
    assert _ws(cfg, 224)[1] <= moe.NOALLOC_SCRATCH_BYTES < _ws(cfg, 4096)[1]
    assert call(cfg, 4096) == -7
    assert "scratch" in moe.status_string(-7)
