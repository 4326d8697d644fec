"""moe_forward_noalloc (the static-scratch forward) against moe_forward, through
the C ABI: bit-identical y and y_act on two calls in a row, the second with fewer
tokens, for bf16 and fp8 weights; a call too large for the scratch launches
nothing."""
import numpy as np
import pytest
import torch

import workloads as W
from tests import harness as Hn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [W.DRAFTER, W.DRAFTER_FP8, W.NARROW.with_(name="narrow_mxfp4_noalloc",
                                                                                   weight_dtype=W.DT_MXFP4)])
def test_noalloc_forward_matches_forward(shape):
    import mixture_experts_layer_05_amd as moe
    T0 = 224
    print(f"\n[case] noalloc {shape.name} T={T0} then 7", flush=True)
    case = Hn.make_case(shape, T0, W.base_seed(1, T0))
    cfg = Hn.config(shape)
    sg_w = None if case.inp.w_shared_gate is None else case.inp.w_shared_gate.cuda()
    layer = moe.MoELayer(cfg, case.weights, case.inp.w_router.cuda(), sg_w, case.shared, max_tokens=T0,
                         act_output=True)
    assert moe.workspace_size(cfg, T0) <= moe.NOALLOC_SCRATCH_BYTES
    x_all = case.inp.x.cuda()
    bias_all = None if case.inp.logit_bias is None else case.inp.logit_bias.cuda()
    for T in (T0, 7):                         # two calls in a row, the second smaller
        x = x_all[:T].contiguous()
        bias = None if bias_all is None else bias_all[:T].contiguous()
        layer.route(x, bias)
        layer.dispatch(T)
        v = layer.views(T)
        sg = v["shared_gate"] if shape.shared_expert_intermediate_size else None
        moe.forward(cfg, x, v["topk_weights"], sg, layer.counts, layer.offsets, v["perm"], layer.weights,
                    v["y"], layer.workspace, y_act=v["y_act"])
        torch.cuda.synchronize()
        y_ref, act_ref = v["y"].clone(), v["y_act"].clone()
        v["y"].fill_(float("nan"))
        v["y_act"].fill_(float("nan"))
        moe.forward_noalloc(cfg, x, v["topk_weights"], sg, layer.counts, layer.offsets, v["perm"],
                            layer.weights, v["y"], y_act=v["y_act"])
        torch.cuda.synchronize()
        assert torch.equal(v["y"], y_ref), f"T={T}: y differs from moe_forward"
        assert torch.equal(v["y_act"].view(torch.int16), act_ref.view(torch.int16)), f"T={T}: y_act differs"
        assert torch.isfinite(y_ref).all()
        print(f"[case] ok T={T} bit-identical to moe_forward", flush=True)


def test_noalloc_forward_rejects_calls_beyond_its_scratch():
    import mixture_experts_layer_05_amd as moe
    shape, T = W.DRAFTER, 4096
    case = Hn.make_case(shape, 8, 3)
    cfg = Hn.config(shape)
    assert moe.workspace_size(cfg, T) > moe.NOALLOC_SCRATCH_BYTES
    layer = moe.MoELayer(cfg, case.weights, case.inp.w_router.cuda(), case.inp.w_shared_gate.cuda(),
                         case.shared, max_tokens=T)
    x = torch.zeros(T, shape.hidden_size, dtype=torch.bfloat16, device="cuda")
    layer.route(x)
    layer.dispatch(T)
    layer.y.fill_(float("nan"))
    torch.cuda.synchronize()
    with pytest.raises(moe.MoEError) as ei:
        moe.forward_noalloc(cfg, x, layer.topk_weights, layer.shared_gate, layer.counts, layer.offsets,
                            layer.perm, layer.weights, layer.y)
    assert ei.value.status == -7
    torch.cuda.synchronize()
    assert torch.isnan(layer.y).all()       # nothing was launched
