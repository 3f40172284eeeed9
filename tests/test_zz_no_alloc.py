"""The allocation-free forward (vdn_forward_noalloc, static device scratch) against vdn_forward on
the same inputs: two calls in a row on one GPU, the second with a smaller input (another shape, so
the scratch still holds the first call's data where the second reads its tables and zero tiles),
then a third call of the first shape.  Same kernels, so the outputs are expected bit-identical; the
test also holds them to the bf16 bar against the CPU oracle."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import TOL, make_plan, rel_err, run_layer, to_device
from linear_video_attention_amd import vdn
from oracle import vdn_oracle as orc

pytestmark = pytest.mark.gpu

CASES = [
    # n_text, T, N, C, H, d, dtype, anchors: a larger bf16 case, then a smaller one with other
    # text and key-space lengths, then an fp32 case on the generic kernels
    (24, 11, 320, 3, 2, 128, "bf16", True),
    (7, 6, 72, 2, 1, 64, "bf16", False),
    (3, 5, 24, 2, 1, 32, "fp32", True),
]


def noalloc_forward(w, dev):
    out = torch.empty_like(dev["q"])
    vdn.vdn_forward_noalloc(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, dev["q"], dev["k"], dev["v"],
                            dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"], out)
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_plan_forward_on_consecutive_calls():
    for i, case in enumerate(CASES + CASES[:1]):
        n_text, T, N, C, H, d, dtype, anchors = case
        w = synth.custom(n_text, T, N, C, H, d, dtype, "sigmoid", anchors)
        inp = synth.make_inputs(w, seed=10 + i)
        dev = to_device(inp, w.dtype)
        got = noalloc_forward(w, dev)
        plan = make_plan(w)
        want = run_layer(plan, dev)
        plan.close()
        ref = orc.vdn_forward(inp, w.T, w.N, w.C, w.anchors)
        e_plan = rel_err(got.float().cpu().numpy(), want.float().cpu().numpy())
        e_orc = rel_err(got.float().cpu().numpy(), ref)
        print(f"call {i} {case}: vs vdn_forward {e_plan:.2e}, vs oracle {e_orc:.2e}", flush=True)
        assert e_plan <= TOL[w.dtype] and e_orc <= TOL[w.dtype]
        assert torch.equal(got, want), "same kernels on the same inputs: bit-identical"


def test_noalloc_rejects_large_and_bad_arguments():
    w = synth.WORKLOADS["768p"]
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vdn.VdnError) as ei:       # 0.63 GB of workspace: beyond the scratch
        vdn.vdn_forward_noalloc(w.T, w.N, w.C, w.n_text, w.H, w.d, True, "bf16", x, x, x, x, x, x, x, x)
    assert ei.value.status == vdn.VDN_ERR_TOO_LARGE
    w = synth.custom(4, 3, 32, 2, 1, 64, "bf16", "sigmoid", True)
    inp = synth.make_inputs(w)
    dev = to_device(inp, w.dtype)
    with pytest.raises(vdn.VdnError) as ei:       # out aliases q
        vdn.vdn_forward_noalloc(w.T, w.N, w.C, w.n_text, w.H, w.d, True, "bf16", dev["q"], dev["k"], dev["v"],
                                dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"], dev["q"])
    assert ei.value.status == vdn.VDN_ERR_INVALID_ARG
    with pytest.raises(vdn.VdnError) as ei:       # d outside {16, 32, 64, 128}
        vdn.vdn_forward_noalloc(w.T, w.N, w.C, w.n_text, w.H, 48, True, "bf16", dev["q"], dev["k"], dev["v"],
                                dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"], torch.empty_like(dev["q"]))
    assert ei.value.status == vdn.VDN_ERR_UNSUPPORTED
