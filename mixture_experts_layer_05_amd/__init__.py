"""Python binding of the MI355X routed-MoE library (libmoe_mi355x.so).

Argument marshalling only: every step of the layer runs in the HIP kernels behind
the C ABI declared in include/moe_mi355x.h.  PyTorch provides device memory and
the stream.  There is no fallback: if the shared library is missing, every call
raises.

    cfg = moe.MoEConfig(hidden_size=5120, n_routed_experts=16, moe_intermediate_size=1024,
                        num_experts_per_tok=2, shared_expert_intermediate_size=2048,
                        weight_dtype="bf16", act_dtype="bf16")
    layer = moe.MoELayer(cfg, weights, w_router, w_shared_gate, max_tokens=224)
    y = layer(x)                      # route -> dispatch -> forward on the current stream
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe_mi355x.h")

DTYPES = {"f32": 0, "bf16": 1, "fp8_e4m3_g128": 2, "mxfp4": 3}
ENTRY_POINTS = ("moe_workspace_size", "moe_route", "moe_dispatch", "moe_forward",
                "moe_forward_gate_up", "moe_forward_down", "moe_forward_noalloc", "moe_status_string",
                "moe_version")
# Static scratch of moe_forward_noalloc (bytes), as the header states it.
NOALLOC_SCRATCH_BYTES = 64 << 20


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_string(status)})")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden_size", "n_routed_experts", "moe_intermediate_size", "num_experts_per_tok",
        "shared_expert_intermediate_size", "weight_dtype", "act_dtype", "norm_topk_prob",
        "expert_budget")] + [("top_p", ctypes.c_float)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
        "ws_gate", "ws_up", "ws_down", "ss_gate", "ss_up", "ss_down")]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with mixture_experts_layer_05_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        cfgp = ctypes.POINTER(_Config)
        L.moe_workspace_size.argtypes = [cfgp, i32, ctypes.POINTER(sz)]
        L.moe_route.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_dispatch.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, sz, vp]
        fwd = [cfgp, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(_Weights), vp, vp, vp, sz, vp]
        for name in ("moe_forward", "moe_forward_gate_up", "moe_forward_down"):
            getattr(L, name).argtypes = fwd
        L.moe_forward_noalloc.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(_Weights), vp, vp,
                                          vp]
        for name in ("moe_workspace_size", "moe_route", "moe_dispatch", "moe_forward",
                     "moe_forward_gate_up", "moe_forward_down", "moe_forward_noalloc", "moe_version"):
            getattr(L, name).restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MoEError(status, what)


@dataclasses.dataclass
class MoEConfig:
    hidden_size: int
    n_routed_experts: int
    moe_intermediate_size: int
    num_experts_per_tok: int
    shared_expert_intermediate_size: int = 0
    weight_dtype: str = "bf16"
    act_dtype: str = "bf16"
    norm_topk_prob: int = 1
    expert_budget: int = 0
    top_p: float = 0.0

    def c(self) -> _Config:
        return _Config(self.hidden_size, self.n_routed_experts, self.moe_intermediate_size,
                       self.num_experts_per_tok, self.shared_expert_intermediate_size,
                       DTYPES[self.weight_dtype], DTYPES[self.act_dtype], self.norm_topk_prob,
                       self.expert_budget, self.top_p)

    @property
    def act_torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.act_dtype == "f32" else torch.bfloat16


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the MoE library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _expect(t: Optional[torch.Tensor], shape, dtype, name: str) -> None:
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def workspace_size(cfg: MoEConfig, max_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(cfg.c()), int(max_tokens), ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def route(cfg: MoEConfig, x, w_router, w_shared_gate, logit_bias, topk_ids, topk_weights,
          shared_gate, route_stats, workspace, stream=None) -> None:
    T, E, K, H = x.shape[0], cfg.n_routed_experts, cfg.num_experts_per_tok, cfg.hidden_size
    _expect(x, (T, H), cfg.act_torch_dtype, "x")
    _expect(w_router, (E, H), cfg.act_torch_dtype, "w_router")
    _expect(w_shared_gate, (H,), cfg.act_torch_dtype, "w_shared_gate")
    _expect(logit_bias, (T, E), torch.float32, "logit_bias")
    _expect(topk_ids, (T, K), torch.int32, "topk_ids")
    _expect(topk_weights, (T, K), torch.float32, "topk_weights")
    _expect(shared_gate, (T,), torch.float32, "shared_gate")
    _expect(route_stats, (4,), torch.int32, "route_stats")
    _check(lib().moe_route(ctypes.byref(cfg.c()), T, _ptr(x), _ptr(w_router), _ptr(w_shared_gate),
                           _ptr(logit_bias), _ptr(topk_ids), _ptr(topk_weights), _ptr(shared_gate),
                           _ptr(route_stats), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_route")


def dispatch(cfg: MoEConfig, topk_ids, counts, offsets, perm, workspace, stream=None) -> None:
    T, E, K = topk_ids.shape[0], cfg.n_routed_experts, cfg.num_experts_per_tok
    _expect(topk_ids, (T, K), torch.int32, "topk_ids")
    _expect(counts, (E,), torch.int32, "counts")
    _expect(offsets, (E + 1,), torch.int32, "offsets")
    _expect(perm, (T * K,), torch.int32, "perm")
    _check(lib().moe_dispatch(ctypes.byref(cfg.c()), T, _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                              _ptr(perm), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_dispatch")


def expert_weights_struct(cfg: MoEConfig, w: Dict[str, torch.Tensor],
                          shared: Optional[Dict[str, torch.Tensor]]) -> _Weights:
    """Routed weights {gate, up, down[, *_s]} stacked over experts; shared likewise."""
    E, I, H, S = cfg.n_routed_experts, cfg.moe_intermediate_size, cfg.hidden_size, \
        cfg.shared_expert_intermediate_size
    fp8 = cfg.weight_dtype == "fp8_e4m3_g128"
    mx = cfg.weight_dtype == "mxfp4"
    quant = fp8 or mx
    wdt = torch.uint8 if quant else cfg.act_torch_dtype
    per = 2 if mx else 1                         # elements per stored byte along the contraction
    sdt, sgroup = (torch.uint8, 32) if mx else (torch.float32, 128)
    _expect(w["gate"], (E, I, H // per), wdt, "w_gate")
    _expect(w["up"], (E, I, H // per), wdt, "w_up")
    _expect(w["down"], (E, H, I // per), wdt, "w_down")
    s = _Weights(_ptr(w["gate"]), _ptr(w["up"]), _ptr(w["down"]))
    if quant:
        _expect(w["gate_s"], (E, I, H // sgroup), sdt, "s_gate")
        _expect(w["up_s"], (E, I, H // sgroup), sdt, "s_up")
        _expect(w["down_s"], (E, H, I // sgroup), sdt, "s_down")
        s.s_gate, s.s_up, s.s_down = _ptr(w["gate_s"]), _ptr(w["up_s"]), _ptr(w["down_s"])
    if S > 0:
        if shared is None:
            raise ValueError("shared expert weights are required when shared_expert_intermediate_size > 0")
        _expect(shared["gate"], (S, H // per), wdt, "ws_gate")
        _expect(shared["up"], (S, H // per), wdt, "ws_up")
        _expect(shared["down"], (H, S // per), wdt, "ws_down")
        s.ws_gate, s.ws_up, s.ws_down = _ptr(shared["gate"]), _ptr(shared["up"]), _ptr(shared["down"])
        if quant:
            _expect(shared["gate_s"], (S, H // sgroup), sdt, "ss_gate")
            _expect(shared["up_s"], (S, H // sgroup), sdt, "ss_up")
            _expect(shared["down_s"], (H, S // sgroup), sdt, "ss_down")
            s.ss_gate, s.ss_up, s.ss_down = _ptr(shared["gate_s"]), _ptr(shared["up_s"]), _ptr(shared["down_s"])
    return s


def _forward_call(name, cfg, x, topk_weights, shared_gate, counts, offsets, perm, weights, y,
                  workspace, stream, y_act=None):
    T, H = x.shape[0], cfg.hidden_size
    _expect(y, (T, H), torch.float32, "y")
    _expect(topk_weights, (T, cfg.num_experts_per_tok), torch.float32, "topk_weights")
    if y_act is not None:
        act = torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32
        _expect(y_act, (T, H), act, "y_act")
    _check(getattr(lib(), name)(ctypes.byref(cfg.c()), T, _ptr(x), _ptr(topk_weights), _ptr(shared_gate),
                                _ptr(counts), _ptr(offsets), _ptr(perm), ctypes.byref(weights), _ptr(y),
                                _ptr(y_act), _ptr(workspace), workspace.numel(), _stream(stream)), name)


def forward(cfg, x, topk_weights, shared_gate, counts, offsets, perm, weights: _Weights, y, workspace,
            stream=None, y_act=None) -> None:
    _forward_call("moe_forward", cfg, x, topk_weights, shared_gate, counts, offsets, perm, weights, y,
                  workspace, stream, y_act)


def forward_gate_up(cfg, x, topk_weights, shared_gate, counts, offsets, perm, weights, y, workspace,
                    stream=None, y_act=None) -> None:
    _forward_call("moe_forward_gate_up", cfg, x, topk_weights, shared_gate, counts, offsets, perm,
                  weights, y, workspace, stream, y_act)


def forward_down(cfg, x, topk_weights, shared_gate, counts, offsets, perm, weights, y, workspace,
                 stream=None, y_act=None) -> None:
    _forward_call("moe_forward_down", cfg, x, topk_weights, shared_gate, counts, offsets, perm,
                  weights, y, workspace, stream, y_act)


def forward_noalloc(cfg, x, topk_weights, shared_gate, counts, offsets, perm, weights: _Weights, y,
                    stream=None, y_act=None) -> None:
    """moe_forward on the library's static per-GPU scratch (no workspace argument)."""
    T, H = x.shape[0], cfg.hidden_size
    _expect(y, (T, H), torch.float32, "y")
    _expect(topk_weights, (T, cfg.num_experts_per_tok), torch.float32, "topk_weights")
    if y_act is not None:
        _expect(y_act, (T, H), torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32, "y_act")
    _check(lib().moe_forward_noalloc(ctypes.byref(cfg.c()), T, _ptr(x), _ptr(topk_weights), _ptr(shared_gate),
                                     _ptr(counts), _ptr(offsets), _ptr(perm), ctypes.byref(weights), _ptr(y),
                                     _ptr(y_act), _stream(stream)), "moe_forward_noalloc")


class MoELayer:
    """Owns the outputs and the workspace for up to `max_tokens` tokens and runs
    route -> dispatch -> forward on the current stream.  With `stats=True` each
    route also fills `route_stats` (int32[4], as moe_route documents it)."""

    def __init__(self, cfg: MoEConfig, weights: Dict[str, torch.Tensor], w_router: torch.Tensor,
                 w_shared_gate: Optional[torch.Tensor] = None,
                 shared: Optional[Dict[str, torch.Tensor]] = None, max_tokens: int = 1,
                 device: str = "cuda", act_output: bool = False, stats: bool = False):
        self.cfg = cfg
        self.weights_dict, self.shared_dict = weights, shared
        self.weights = expert_weights_struct(cfg, weights, shared)
        self.w_router, self.w_shared_gate = w_router, w_shared_gate
        self.max_tokens = max_tokens
        E, K = cfg.n_routed_experts, cfg.num_experts_per_tok
        dev = torch.device(device)
        self.workspace = torch.empty(workspace_size(cfg, max_tokens), dtype=torch.uint8, device=dev)
        self.topk_ids = torch.empty(max_tokens, K, dtype=torch.int32, device=dev)
        self.topk_weights = torch.empty(max_tokens, K, dtype=torch.float32, device=dev)
        self.shared_gate = torch.empty(max_tokens, dtype=torch.float32, device=dev)
        # Routing statistics cost one extra single-block pass when there is no
        # expert budget, so they are kept only on request.
        self.route_stats = torch.zeros(4, dtype=torch.int32, device=dev) if stats else None
        self.counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.perm = torch.empty(max_tokens * K, dtype=torch.int32, device=dev)
        self.y = torch.empty(max_tokens, cfg.hidden_size, dtype=torch.float32, device=dev)
        # Optional copy of y in the activation dtype (written by the same pass).
        act = torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32
        self.y_act = torch.empty(max_tokens, cfg.hidden_size, dtype=act, device=dev) if act_output else None

    def views(self, T: int):
        K = self.cfg.num_experts_per_tok
        return dict(topk_ids=self.topk_ids[:T], topk_weights=self.topk_weights[:T],
                    shared_gate=self.shared_gate[:T], perm=self.perm[:T * K], y=self.y[:T],
                    y_act=None if self.y_act is None else self.y_act[:T])

    def route(self, x, logit_bias=None, stream=None):
        v = self.views(x.shape[0])
        sg = v["shared_gate"] if self.cfg.shared_expert_intermediate_size > 0 else None
        route(self.cfg, x, self.w_router, self.w_shared_gate, logit_bias, v["topk_ids"], v["topk_weights"],
              sg, self.route_stats, self.workspace, stream)

    def dispatch(self, T: int, stream=None):
        v = self.views(T)
        dispatch(self.cfg, v["topk_ids"], self.counts, self.offsets, v["perm"], self.workspace, stream)

    def forward(self, x, stream=None, half: Optional[str] = None):
        v = self.views(x.shape[0])
        sg = v["shared_gate"] if self.cfg.shared_expert_intermediate_size > 0 else None
        fn = {None: forward, "gate_up": forward_gate_up, "down": forward_down}[half]
        fn(self.cfg, x, v["topk_weights"], sg, self.counts, self.offsets, v["perm"], self.weights, v["y"],
           self.workspace, stream, v["y_act"])

    def __call__(self, x, logit_bias=None, stream=None) -> torch.Tensor:
        if x.shape[0] > self.max_tokens:
            raise ValueError("more tokens than the layer was sized for")
        self.route(x, logit_bias, stream)
        self.dispatch(x.shape[0], stream)
        self.forward(x, stream)
        return self.views(x.shape[0])["y"]
