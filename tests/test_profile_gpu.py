"""Per-stage timing through the C ABI (vdn_profile_enable / vdn_profile_read) on the MFMA, FP8 and
generic plans: every stage is timed, the first softmax launch alone takes no longer than the whole
softmax stage, the stages of a serial plan fit inside its total, and profiling changes no output."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

from linear_video_attention_amd.vdn import STAGES, Plan  # noqa: E402

from gpu_util import make_plan, run_layer, to_device  # noqa: E402


@pytest.mark.parametrize("kind", ["mfma", "fp8", "generic"])
def test_profile_stages(kind):
    w = synth.custom(64, 10, 256, 5, 2, 128, "bf16")
    inp = synth.make_inputs(w, seed=3)
    dev = to_device(inp, w.dtype)
    if kind == "fp8":
        plan = Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, fp8=True)
    else:
        plan = make_plan(w, generic=kind == "generic")
    ref = run_layer(plan, dev).clone()
    plan.profile_enable(3)
    for _ in range(3):
        out = run_layer(plan, dev)
    ms, calls = plan.profile_read()
    print(kind, {k: round(v / calls, 4) for k, v in ms.items()}, flush=True)
    assert calls == 3
    assert set(ms) == set(STAGES)
    assert all(v > 0 for v in ms.values()), ms
    assert ms["softmax_first"] <= ms["softmax"] * 1.001 + 1e-3
    parts = sum(ms[k] for k in ("prep", "vda_stats", "vda_scan", "softmax", "epilogue"))
    assert parts <= ms["total"] * 1.01 + 1e-3
    assert torch.equal(out, ref)
    plan.close()
