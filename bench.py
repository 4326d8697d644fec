"""Benchmark of the routed MoE FFN forward on one MI355X.

One step = route -> dispatch -> forward (every kernel of the layer) over one
batch of synthetic tokens, inputs already resident in HBM.  The headline workload
is the largest configuration: the 256-expert top-8 layer (hidden 7168,
intermediate 2048, bf16) at T = 8192 tokens with a Zipf router skew of 1.5, the
shape of [DeepGEMM PR #381, "Validation" and "B200 performance"]; its gate/up
stage is priced against the bf16 MFMA peak.  The same line nests a decode record:
the 16 x 1024 top-2 drafter layer with its 2048-wide sigmoid-gated shared expert
at 32 concurrent 7-token blocks (T = 224) [SpecForge PR #943, "End-to-end serving
speed"], priced against the HBM peak.  Where a layer's weights are smaller than
~2 GB, several copies are cycled (one per step, like the layers of a model) so
that no step finds its weights in the 256 MB last-level cache.

Prints ONE JSON line (rank 0): tokens/s of the whole layer plus TFLOP/s, weight
GB/s, the roofline of the dominant kernel (timed with HIP events on the stream
the kernel runs on) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# Dense MFMA peaks by weight dtype; MXFP4 weights meet MXFP8 activations, a mixed
# fp8 x fp4 contraction, priced at the fp8 rate.
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8_e4m3_g128": 5000.0, "mxfp4": 5000.0, "f32": 157.3}

METRIC = "MoE layer tokens/s + TFLOP/s (prefill M) and weight HBM GB/s (decode M), 1 GPU"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="large",
                   choices=["drafter", "narrow", "large", "large_fp8", "tiny", "ep_rank",
                            "drafter_mxfp4", "narrow_mxfp4", "large_mxfp4", "drafter_fp8", "narrow_fp8"])
    p.add_argument("--tokens", type=int, default=None, help="T (default: the workload's bench size)")
    p.add_argument("--alpha", type=float, default=None, help="Zipf router skew for the large layers")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true", help="leave out the nested decode record")
    p.add_argument("--cpu-sample-tokens", type=int, default=None)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (the reference for HBM byte counters)")
    p.add_argument("--library-gemm", action="store_true",
                   help="only time torch.matmul (hipBLASLt) on dense bf16 GEMMs of the workload's expert shapes")
    return p.parse_args()


def workload(args):
    import workloads as W
    table = {
        "drafter": (W.DRAFTER, 1, 224, None),
        "narrow": (W.NARROW, 2, 224, None),
        "large": (W.LARGE, 3, 8192, 1.5),
        "large_fp8": (W.LARGE_FP8, 4, 8192, 1.5),
        "tiny": (W.TINY, 0, 64, None),
        "ep_rank": (W.EP_RANK, 5, 4096, 1.5),
        "drafter_mxfp4": (W.DRAFTER_MX4, 1, 224, None),
        "narrow_mxfp4": (W.NARROW_MX4, 2, 224, None),
        "large_mxfp4": (W.LARGE_MX4, 3, 512, 0.0),
        "drafter_fp8": (W.DRAFTER_FP8, 1, 224, None),
        "narrow_fp8": (W.NARROW_FP8, 2, 224, None),
    }
    shape, idx, T, alpha = table[args.workload]
    if args.tokens is not None:
        T = args.tokens
    if args.alpha is not None:
        alpha = args.alpha
    return shape, idx, T, alpha


def weight_bytes_per_elem(shape) -> float:
    # MXFP4: half a byte per element plus one E8M0 byte per 32.
    return {"f32": 4.0, "bf16": 2.0, "fp8_e4m3_g128": 1.0 + 4.0 / 128, "mxfp4": 0.5 + 1.0 / 32}[shape.weight_dtype]


def accounting(shape, T, counts, router=True):
    """Algorithmic FLOPs and bytes of one step (from the realised routing).
    `router` False: the step starts from given ids (no router GEMV)."""
    H, I, S, E = shape.hidden_size, shape.moe_intermediate_size, shape.shared_expert_intermediate_size, \
        shape.n_routed_experts
    slots = int(counts.sum())
    touched = int((counts > 0).sum())
    bw = weight_bytes_per_elem(shape)
    ba = 4.0 if shape.act_dtype == "f32" else 2.0
    flops = 2.0 * T * H * (E + (1 if S else 0)) * router + 6.0 * H * I * slots + 6.0 * T * H * S
    gate_up_w = touched * 2.0 * I * H * bw + 2.0 * S * H * bw
    down_w = touched * 1.0 * H * I * bw + 1.0 * H * S * bw
    router_w = (E + (1 if S else 0)) * H * ba * router
    weights = gate_up_w + down_w + router_w
    x_bytes = T * H * ba
    y_bytes = T * H * 4.0
    hbytes = 2.0 if shape.weight_dtype == "bf16" else 4.0
    h_elems = slots * I + T * S
    # Dominant kernel (gate/up + SwiGLU): its weights, x in, h out.
    gate_up_bytes = gate_up_w + x_bytes + h_elems * hbytes
    return dict(flops=flops, weight_bytes=weights, total_bytes=weights + x_bytes + y_bytes,
                gate_up_bytes=gate_up_bytes, touched=touched, slots=slots,
                gate_up_flops=4.0 * H * I * slots + 4.0 * T * H * S)


def layer_roofline(shape, a, ms_per_step):
    """The whole layer against its binding roofline: t_HBM = algorithmic bytes at
    8 TB/s, t_MFMA = algorithmic FLOPs at the weight dtype's dense peak; the
    binding one is the larger, and frac = that time / the measured step."""
    peak_tf = MFMA_PEAK_TFLOPS[shape.weight_dtype]
    t_hbm = a["total_bytes"] / (HBM_PEAK_GBPS * 1e9) * 1e3
    t_mfma = a["flops"] / (peak_tf * 1e12) * 1e3
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return {"bound": bound, "t_hbm_ms": round(t_hbm, 5), "t_mfma_ms": round(t_mfma, 5),
            "frac": round(max(t_hbm, t_mfma) / ms_per_step, 4)}


def gate_up_kernel(shape, T: int) -> str:
    """Name of the gate/up kernel(s) the library launches for this layer and T (the
    same rules as its launchers; used to label the roofline)."""
    if shape.weight_dtype == "f32":
        return "gate_up_f32_kernel"
    fp8 = shape.weight_dtype != "bf16"
    dt = {"bf16": "bf16", "fp8_e4m3_g128": "fp8", "mxfp4": "mxfp4"}[shape.weight_dtype]
    H, E, I, K, S = (shape.hidden_size, shape.n_routed_experts, shape.moe_intermediate_size,
                     shape.num_experts_per_tok, shape.shared_expert_intermediate_size)
    rho = T * K // E

    def stream(r):
        narrow = min(E, T * K) * (I // 64) < 3 * 256
        if r >= 48:
            cfg = "128, 256, 2" if dt == "mxfp4" and I % 128 == 0 and S % 128 == 0 else "128, 128, 2"
        elif r <= 12:
            cfg = "16, 128, 1"
        elif r <= 24:
            cfg = "32, 64, 2" if narrow else "32, 128, 1"
        else:
            cfg = "64, 64, 2" if narrow else "64, 128, 1"
        return f"stream_expert_kernel<GateUp, {cfg}, {dt}>"

    # Rows divided between the 256-row LDS-tiled kernel and the streaming kernel.
    if rho >= 16 and T * K * I >= 256 * 256 * 128:
        tall = {"bf16": "tiledpp_expert_kernel<GateUp> (bf16, 256x256)",
                "fp8": "tiled8pp_expert_kernel<GateUp> (fp8, 256x256)",
                "mxfp4": "tiledmx_expert_kernel<GateUp> (mxfp4, 256x256)"}[dt]
        if rho >= 192:
            # The streaming share divided by group: more than 64 rows left (if such
            # groups fill the GPU), and the rest.
            return (f"{tall} for groups of >= 128 rows + {stream(48)} for groups left with > 64 rows"
                    f" + {stream(47)} for the rest")
        return f"{tall} for groups of >= 128 rows + {stream(rho)} for the rest"
    return stream(rho)


def kernel_source_file(kernel_label: str) -> str:
    """HIP source files ('+'-joined) that hold the kernels named by a roofline label."""
    files = [f for key, f in (("tiled", "tile_gemm.hip"), ("stream", "stream_gemm.hip")) if key in kernel_label]
    return "+".join(files) if files else "experts.hip"


def library_source_hash(kernel_file: str = None) -> str:
    """sha256 over the HIP sources a stored counter reading depends on: the kernel's
    own file, the shared headers and the launch code (experts.hip, api.hip); all
    sources if no file is named."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "mixture_experts_layer_05_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*")))
    if kernel_file is not None:
        keep = set(kernel_file.split("+")) | {"experts.hip", "api.hip"}
        files = [f for f in files if f.endswith(".h") or os.path.basename(f) in keep]
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel: str, workload: str, kernel_file: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter summary
    (profiles/<kernel>_<workload>_traffic.md), or None if there is none or the
    sources it depends on changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != library_source_hash(kernel_file):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


CPU_BASELINE_SECONDS = 10.0


def cpu_baseline(shape, case_inputs, expert_cpu, shared_cpu, T, sample_tokens):
    """The CPU oracle as it stands, on a bounded sample: routing of every token plus
    the expert math of `sample_tokens` tokens; reported per token of the sample.
    expert_cpu / shared_cpu hand out host copies staged before the timing (the
    device-to-host copy of the weights is input staging, not oracle work)."""
    import numpy as np
    import threadpoolctl
    from oracle import moe as O
    toks = np.arange(min(sample_tokens, T))
    # The same pass repeated until at least CPU_BASELINE_SECONDS of timing (one
    # pass if it alone takes longer); the rate is over all passes.
    reps, t0 = 0, time.perf_counter()
    while True:
        O.moe_layer(case_inputs.x, case_inputs.w_router, case_inputs.w_shared_gate, case_inputs.logit_bias,
                    shape.num_experts_per_tok, shape.n_routed_experts, expert_cpu, shared_cpu,
                    shape.weight_dtype, bool(shape.norm_topk_prob), shape.expert_budget, toks)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_BASELINE_SECONDS:
            break
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    return {"value": reps * len(toks) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(toks)} of {T} tokens: routing of all {T} tokens + expert math of the "
                      f"first {len(toks)}, float64 numpy on the host (weights staged in host memory "
                      f"before timing); {reps} passes in {dt:.2f} s"}


def measure(args, shape, idx, T, alpha, steps, warmup):
    """Time `steps` steps of one workload; returns (JSON record, context for the CPU
    baseline)."""
    import numpy as np
    import torch
    import workloads as W
    import mixture_experts_layer_05_amd as moe

    dev = torch.device("cuda:0")
    seed = W.base_seed(idx, T)
    ep_rank = shape.name == W.EP_RANK.name
    cfg = moe.MoEConfig(shape.hidden_size, shape.n_routed_experts, shape.moe_intermediate_size,
                        shape.num_experts_per_tok, shape.shared_expert_intermediate_size,
                        shape.weight_dtype, shape.act_dtype, shape.norm_topk_prob, shape.expert_budget)

    # Weight copies: enough that consecutive steps never share cached weights.
    one = (shape.n_routed_experts * 3 * shape.hidden_size * shape.moe_intermediate_size
           + 3 * shape.hidden_size * shape.shared_expert_intermediate_size) * weight_bytes_per_elem(shape)
    n_copies = int(max(1, min(8, np.ceil(2.0e9 / one))))
    # ep_rank: the rank's inputs are the global layer's (x, router, Zipf bias).
    inp = W.layer_inputs(W.LARGE if ep_rank else shape, T, seed, alpha)
    layers = []
    for c in range(n_copies):
        wts = W.stacked_expert_weights(shape, seed + 7919 * c, "cuda")
        shw = W.shared_expert_weights(shape, seed + 7919 * c, "cuda")
        if ep_rank:   # the local layer's router is unused: routing is the global layer's
            wr = inp.w_router[:W.EP_RANK_LOCAL].to(dev)
        else:
            wr = W.router_weight(shape, seed + 7919 * c).to(dev) if c else inp.w_router.to(dev)
        wg = inp.w_shared_gate.to(dev) if inp.w_shared_gate is not None else None
        layers.append(moe.MoELayer(cfg, wts, wr, wg, shw, max_tokens=T))
    x = inp.x.to(dev)
    bias = inp.logit_bias.to(dev) if inp.logit_bias is not None else None
    stream = torch.cuda.current_stream()
    ep_slots = None
    if ep_rank:
        # Route the global layer once (every rank does this identically), keep the
        # slots of the busiest rank's experts [32r, 32r + 32) and time dispatch +
        # forward of that rank's share.
        g = W.LARGE
        gcfg = moe.MoEConfig(g.hidden_size, g.n_routed_experts, g.moe_intermediate_size,
                             g.num_experts_per_tok, 0, g.weight_dtype, g.act_dtype, g.norm_topk_prob, 0)
        gws = torch.empty(moe.workspace_size(gcfg, T), dtype=torch.uint8, device=dev)
        gids = torch.empty(T, g.num_experts_per_tok, dtype=torch.int32, device=dev)
        gw = torch.empty(T, g.num_experts_per_tok, dtype=torch.float32, device=dev)
        moe.route(gcfg, x, inp.w_router.to(dev), None, bias, gids, gw, None, None, gws)
        ep_slots = torch.bincount((gids // W.EP_RANK_LOCAL).flatten().long(), minlength=W.EP_RANKS)
        rank = int(ep_slots.argmax())
        lids = gids - rank * W.EP_RANK_LOCAL
        local = (lids >= 0) & (lids < W.EP_RANK_LOCAL)
        for L in layers:
            L.topk_ids[:T].copy_(torch.where(local, lids, torch.full_like(lids, -1)))
            L.topk_weights[:T].copy_(torch.where(local, gw, torch.zeros_like(gw)))
        torch.cuda.synchronize()
        ep_slots = {"rank": rank, "slots_per_rank": ep_slots.cpu().tolist()}

    def step(i, ev=None):
        L = layers[i % n_copies]
        if ev is not None:
            ev[0].record(stream)
        if not ep_rank:
            L.route(x, bias)
        L.dispatch(T)
        if ev is not None:
            ev[1].record(stream)
        L.forward(x, half="gate_up")
        if ev is not None:
            ev[2].record(stream)
        L.forward(x, half="down")
        if ev is not None:
            ev[3].record(stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # The timed steps: the layer alone (no event records between its launches).
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    # A second pass of as many steps with HIP events between the stages, on the
    # launching stream: per-stage times and the gate/up duration of the roofline.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    step_ev = np.array([e[0].elapsed_time(e[3]) for e in evs])
    gate_up_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    down_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    route_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))

    acc = [accounting(shape, T, L.counts.cpu().numpy(), router=not ep_rank) for L in layers]
    a = {k: float(np.mean([d[k] for d in acc])) for k in acc[0]}
    tokens_per_s = T / (ms_per_step * 1e-3)
    # Dominant kernel: gate/up + SwiGLU, against the roofline that binds it: its
    # algorithmic bytes at the HBM peak or its algorithmic FLOPs at the weight
    # dtype's dense MFMA peak, whichever takes longer.
    peak_tf = MFMA_PEAK_TFLOPS[shape.weight_dtype]
    t_hbm = a["gate_up_bytes"] / (HBM_PEAK_GBPS * 1e9)
    t_mfma = a["gate_up_flops"] / (peak_tf * 1e12)
    kernel = gate_up_kernel(shape, T)
    wl = args.workload if args is not None else "drafter"
    traffic = stored_traffic("gate_up", f"{wl}_T{T}", kernel_source_file(kernel))
    if t_mfma > t_hbm and shape.weight_dtype != "f32":
        achieved = a["gate_up_flops"] / (gate_up_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 1), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(achieved / peak_tf, 4), "traffic": traffic}
    else:
        achieved = a["gate_up_bytes"] / (gate_up_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic}
    rec = {
        "ms_per_step": round(ms_per_step, 5),
        "tokens_per_s": round(tokens_per_s, 1),
        "dtype": shape.weight_dtype,
        "config": {"workload": f"{shape.name} T={T}" + (f" alpha={alpha}" if alpha is not None else ""),
                   "tokens": T, "hidden": shape.hidden_size, "experts": shape.n_routed_experts,
                   "intermediate": shape.moe_intermediate_size, "topk": shape.num_experts_per_tok,
                   "shared": shape.shared_expert_intermediate_size, "budget": shape.expert_budget,
                   "weight_copies": n_copies},
        "tflops": round(a["flops"] / (ms_per_step * 1e-3) / 1e12, 3),
        "weight_gbps": round(a["weight_bytes"] / (ms_per_step * 1e-3) / 1e9, 1),
        "stage_ms": {"route_dispatch": round(route_ms, 5), "gate_up": round(gate_up_ms, 5),
                     "down": round(down_ms, 5)},
        "experts_touched": a["touched"],
        # Per-step GPU time (events around route .. combine), percentiles over the event pass.
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ev, q)), 5) for q in (10, 50, 90)],
        "roofline": roof,
        **({"ep": ep_slots} if ep_slots else {}),
        "layer_roofline": layer_roofline(shape, a, ms_per_step),
    }
    if shape.weight_dtype != "f32" and a["gate_up_flops"] / (gate_up_ms * 1e-3) / 1e12 > 0:
        rec["gate_up_tflops"] = round(a["gate_up_flops"] / (gate_up_ms * 1e-3) / 1e12, 2)
    return rec, {"inp": inp, "layer": layers[0], "ep_rank": ep_rank}


def dense_gemm_ms(M, N, K, reps=20):
    """Average time of torch.matmul (hipBLASLt) on a dense bf16 [M, K] x [K, N]
    product, with HIP events on torch's stream after 3 warm-up calls."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=gen)
    b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16, generator=gen)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    del a, b, c
    return e0.elapsed_time(e1) / reps


def library_gemm(shape, T, reps=20):
    """The vendor library's dense bf16 GEMM rate on this GPU for the layer's projection
    shapes: all T*K routed rows as one matrix, and one expert's worth of T rows.
    Context for the MFMA roofline (what a plain GEMM of the same size reaches here),
    not a measurement of this library."""
    H, I, K = shape.hidden_size, shape.moe_intermediate_size, shape.num_experts_per_tok
    for name, (M, N, Kd) in (("gate_up, T*K rows", (T * K, 2 * I, H)), ("down, T*K rows", (T * K, H, I)),
                             ("gate_up, T rows", (T, 2 * I, H)), ("down, T rows", (T, H, I))):
        ms = dense_gemm_ms(M, N, Kd, reps)
        print(json.dumps({"library_gemm": name, "M": M, "N": N, "K": Kd, "dtype": "bf16", "ms": round(ms, 4),
                          "tflops": round(2 * M * N * Kd / (ms * 1e-3) / 1e12, 1)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is not sharded "
              f"across GPUs (one GPU's share of an expert-parallel layer is the ep_rank workload).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    import mixture_experts_layer_05_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.lib()   # fail loudly if the HIP library is missing

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": 5}), flush=True)
        return

    shape, idx, T, alpha = workload(args)
    if args.library_gemm:
        library_gemm(shape, T)
        return
    print(f"[bench] {shape.name} T={T} alpha={alpha}: {args.steps} steps after {args.warmup}",
          file=sys.stderr, flush=True)
    rec, ctx = measure(args, shape, idx, T, alpha, args.steps, args.warmup)
    line = {
        "metric": METRIC,
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec["dtype"],
        "data": "synthetic (seeded; random-init weights)",
    }
    line.update({k: v for k, v in rec.items() if k not in ("ms_per_step", "tokens_per_s", "dtype")})
    if rec["roofline"]["bound"] == "mfma" and shape.weight_dtype == W.DT_BF16 and not ctx["ep_rank"]:
        # Context for the MFMA fraction: the vendor library's dense bf16 GEMM over the
        # same number of rows (all T*K routed rows as one matrix, no routing).
        M, N, Kd = T * shape.num_experts_per_tok, 2 * shape.moe_intermediate_size, shape.hidden_size
        lib_tf = 2 * M * N * Kd / (dense_gemm_ms(M, N, Kd) * 1e-3) / 1e12
        line["library_gemm"] = {"kind": "torch.matmul (hipBLASLt), dense bf16 [T*K, H] x [H, 2I]",
                                "tflops": round(lib_tf, 1), "frac_of_peak": round(lib_tf / rec["roofline"]["peak"], 4),
                                "gate_up_stage_vs_library": round(rec["gate_up_tflops"] / lib_tf, 4)}
    if not args.no_decode and args.workload == "large":
        # The decode record: the drafter layer at T = 224, HBM-bound.  Its steps are
        # ~0.2 ms, so it runs ten times the headline's step count.
        print("[bench] decode record: drafter T=224", file=sys.stderr, flush=True)
        drec, _ = measure(None, W.DRAFTER, 1, 224, None, 10 * args.steps, args.warmup)
        line["decode"] = {"ms_per_step": drec["ms_per_step"], "tokens_per_s": drec["tokens_per_s"],
                          "steps": 10 * args.steps, **{k: v for k, v in drec.items()
                                                       if k not in ("ms_per_step", "tokens_per_s")}}
    if not args.no_cpu_baseline and not ctx["ep_rank"]:
        print("[bench] CPU baseline (oracle)", file=sys.stderr, flush=True)
        L0, inp = ctx["layer"], ctx["inp"]
        sample = args.cpu_sample_tokens or min(T, 224 if shape.hidden_size <= 5120 else 4)
        # Stage the sample's experts in host memory before timing.
        ids = L0.topk_ids[:sample].cpu().numpy()
        host = {int(e): {k: v[int(e)].cpu() for k, v in L0.weights_dict.items()} for e in np.unique(ids)
                if e >= 0}
        expert_cpu = lambda e: host[e] if e in host else {k: v[e].cpu() for k, v in L0.weights_dict.items()}  # noqa: E731
        shared_cpu = None if L0.shared_dict is None else {k: v.cpu() for k, v in L0.shared_dict.items()}
        line["cpu_baseline"] = cpu_baseline(shape, inp, expert_cpu, shared_cpu, T, sample)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
