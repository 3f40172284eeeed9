"""Parity of the HIP backward pass (vdn_backward through the C ABI) with the reverse-mode oracle,
gradient by gradient.  Bar as for the forward: max |gpu - oracle| <= 1e-4 * RMS(oracle) for fp32
workloads and <= 2e-2 * RMS(oracle) for bf16 workloads (bf16 workloads store o_s in bf16 and run
the forward's linear branch on split-bf16 MFMA operands, both inside that bar)."""

import numpy as np
import pytest
import torch

import synth
from oracle import vdn_backward as bwd
from oracle import vdn_oracle as orc

pytestmark = pytest.mark.gpu

from gpu_util import TOL, make_plan, rel_err, to_device  # noqa: E402


def check_backward(w, seed=0, decay=False, generic=False, names=None):
    inp = synth.make_inputs(w, seed=seed, decay=decay)
    dout = np.random.default_rng(seed + 99).standard_normal((w.T * w.N, w.H, w.d)).astype(np.float32)
    if w.dtype == "bf16":
        dout = torch.from_numpy(dout).to(torch.bfloat16).float().numpy()
    plan = make_plan(w, generic=generic)
    dev = to_device(inp, w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = plan.backward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"],
                      torch.from_numpy(dout).cuda().to(tdt), alpha=dev["alpha"])
    torch.cuda.synchronize()
    ref = bwd.vdn_backward({k: np.asarray(v, np.float64) if isinstance(v, np.ndarray) else v for k, v in inp.items()},
                           dout.astype(np.float64), w.T, w.N, w.C, w.anchors)
    got = {k: v.cpu().numpy() for k, v in g.items()}
    if "text_kv" in got:
        got["text_k"], got["text_v"] = got.pop("text_kv")
    tol = TOL[w.dtype]
    errs = {}
    for name in (names or ref):
        if ref[name].size == 0:
            continue
        errs[name] = rel_err(got[name], ref[name])
    print(f"{w} decay={decay} generic={generic}: " + "  ".join(f"{k} {v:.1e}" for k, v in errs.items()), flush=True)
    for name, e in errs.items():
        assert e <= tol, (name, e)
    plan.close()


def test_backward_tiny_fp32():
    check_backward(synth.WORKLOADS["tiny"])


def test_backward_tiny_fp32_decay():
    check_backward(synth.WORKLOADS["tiny"], decay=True)


@pytest.mark.parametrize("generic", [False, True])
def test_backward_small_bf16(generic):
    check_backward(synth.WORKLOADS["small"], generic=generic)


BWD_RAGGED = [
    # n_text, T, N, C, H, d, dtype, anchors, decay
    (5, 9, 40, 2, 2, 64, "fp32", True, False),
    (0, 7, 24, 3, 1, 32, "fp32", False, False),
    (3, 1, 16, 5, 1, 64, "fp32", True, False),
    (7, 11, 72, 3, 2, 128, "bf16", True, True),
    (2, 6, 64, 1, 1, 128, "bf16", False, False),
    # more than one 128-row block per frame and of text rows, both ragged, on the d = 64 kernels
    (150, 6, 130, 2, 1, 64, "bf16", True, True),
]


@pytest.mark.parametrize("case", BWD_RAGGED, ids=lambda c: "x".join(str(x) for x in c))
def test_backward_ragged(case):
    n_text, T, N, C, H, d, dtype, anchors, decay = case
    check_backward(synth.custom(n_text, T, N, C, H, d, dtype, "sigmoid", anchors), seed=4, decay=decay)


def test_backward_768p_sampled_dq():
    """768p in the benchmark's configuration: dq of sampled rows (every frame's first and last
    token plus two random tokens per frame, all heads) against the row-wise oracle; every element
    of dbeta, dgate_w[1] and dproj_w[1] (the gradients that do not pass through the softmax
    branch: the merge's linear half and the linear branch's backward) against the full oracle;
    dk, dv and the softmax half of the weight gradients are checked for finiteness here and
    against the full oracle at the smaller shapes."""
    w = synth.WORKLOADS["768p"]
    inp = synth.make_inputs(w, seed=0)
    dout = np.random.default_rng(7).standard_normal((w.T * w.N, w.H, w.d)).astype(np.float32)
    dout = torch.from_numpy(dout).to(torch.bfloat16).float().numpy()
    plan = make_plan(w)
    dev = to_device(inp, w.dtype)
    g = plan.backward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"],
                      torch.from_numpy(dout).cuda().to(torch.bfloat16))
    torch.cuda.synchronize()
    rows = synth.sample_rows(w)
    got = g["q"][torch.from_numpy(rows).cuda()].cpu().numpy()
    got_beta = g["beta"].cpu().numpy()
    got_gw1 = g["gate_w"][1].cpu().numpy()
    got_pw1 = g["proj_w"][1].cpu().numpy()
    finite = all(bool(torch.isfinite(x).all()) for x in g.values())
    del dev, g
    plan.close()
    ref = bwd.dq_rows(inp, dout.astype(np.float64), w.T, w.N, w.C, w.anchors, rows)
    e = rel_err(got, ref)
    print(f"768p backward: dq of {len(rows)} sampled rows, err {e:.2e}", flush=True)
    assert finite
    assert e <= TOL[w.dtype]
    # linear half: do_l, dgate_w[1] and dproj_w[1] do not depend on o_s (zero here)
    print("768p backward: oracle linear branch ...", flush=True)
    o_l = orc.linear_branch(inp["q"], inp["k"], inp["v"], inp["beta"], inp["text_k"], inp["text_v"],
                            w.T, w.N, w.C, w.anchors)
    print("768p backward: oracle merge backward ...", flush=True)
    _, _, do_l, dgate, dproj = bwd.merge_backward(inp["q"], np.zeros_like(o_l), o_l, inp["gate_w"], inp["proj_w"],
                                                  dout.astype(np.float64))
    print("768p backward: oracle linear-branch backward ...", flush=True)
    dbeta = bwd.linear_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["text_k"], inp["text_v"],
                                w.T, w.N, w.C, w.anchors, do_l)[3]
    errs = {"beta": rel_err(got_beta, dbeta), "gate_w[1]": rel_err(got_gw1, dgate[1]),
            "proj_w[1]": rel_err(got_pw1, dproj[1])}
    print("768p backward, linear half: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for name, err in errs.items():
        assert err <= TOL[w.dtype], (name, err)


def test_backward_long_sampled_dq():
    """The long workload (180 frames of 1536 tokens, 5 heads) in the benchmark's launch
    configuration: dq of sampled rows (every frame's first and last token plus two random tokens
    per frame, all heads) against the row-wise oracle, and every gradient finite."""
    w = synth.WORKLOADS["long"]
    inp = synth.make_inputs(w, seed=0)
    dout = np.random.default_rng(9).standard_normal((w.T * w.N, w.H, w.d)).astype(np.float32)
    dout = torch.from_numpy(dout).to(torch.bfloat16).float().numpy()
    plan = make_plan(w)
    dev = to_device(inp, w.dtype)
    print("long backward on the GPU ...", flush=True)
    g = plan.backward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"],
                      torch.from_numpy(dout).cuda().to(torch.bfloat16))
    torch.cuda.synchronize()
    rows = synth.sample_rows(w)
    got = g["q"][torch.from_numpy(rows).cuda()].cpu().numpy()
    finite = all(bool(torch.isfinite(x).all()) for x in g.values())
    del dev, g
    plan.close()
    print("long backward: oracle dq rows ...", flush=True)
    ref = bwd.dq_rows(inp, dout.astype(np.float64), w.T, w.N, w.C, w.anchors, rows)
    e = rel_err(got, ref)
    print(f"long backward: dq of {len(rows)} sampled rows, err {e:.2e}", flush=True)
    assert finite
    assert e <= TOL[w.dtype]


@pytest.mark.parametrize("decay", [False, True])
def test_backward_after_forward_matches(decay):
    """vdn_backward_after_forward after a forward on the same inputs gives vdn_backward's gradients
    bit for bit (same kernels on the same intermediates); without a preceding forward, or with
    the decay gate given to only one of the two calls, it is an argument error."""
    from linear_video_attention_amd import vdn
    w = synth.custom(7, 11, 72, 3, 2, 128, "bf16", "sigmoid", True)
    inp = synth.make_inputs(w, seed=8, decay=decay)
    dev = to_device(inp, w.dtype)
    dout = torch.from_numpy(np.random.default_rng(5).standard_normal((w.T * w.N, w.H, w.d)).astype(np.float32))
    dout = dout.cuda().to(torch.bfloat16)
    args = (dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"], dout)
    plan = make_plan(w)
    with pytest.raises(vdn.VdnError) as ei:
        plan.backward(*args, alpha=dev["alpha"], after_forward=True)
    assert ei.value.status == -1
    ref = plan.backward(*args, alpha=dev["alpha"])
    plan.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"],
                 alpha=dev["alpha"])
    got = plan.backward(*args, alpha=dev["alpha"], after_forward=True)
    torch.cuda.synchronize()
    for name in ref:
        assert torch.equal(ref[name], got[name]), name
    if decay:
        with pytest.raises(vdn.VdnError) as ei:
            plan.backward(*args, after_forward=True)          # the forward had a decay gate
        assert ei.value.status == -1
    plan.close()
