"""Parity of the joint-sequence backward (vdn_backward_joint, and vdn_backward on plans with audio
tokens) with the reverse-mode oracle, gradient by gradient: audio keys are global softmax keys of
the video rows, and the text and audio query rows are one plain softmax over every key ("Video
DeltaNet speeds MiniMax H3 video generation 14.5x", summary).  Bar as for the other backward
tests: max |gpu - oracle| <= 1e-4 * RMS(oracle) for fp32 and <= 2e-2 * RMS(oracle) for bf16."""

import numpy as np
import pytest
import torch

import synth
from oracle import vdn_backward as bwd

pytestmark = pytest.mark.gpu

from gpu_util import TOL, make_plan, rel_err, to_device, weight_grad_storage_error  # noqa: E402


def _round(x, dtype):
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy() if dtype == "bf16" else x


def split_context(got, n_text):
    """The [2][n_ctx] context gradient as text_k, text_v, audio_k, audio_v."""
    ckv = got.pop("text_kv")
    got["text_k"], got["text_v"] = ckv[0][:n_text], ckv[1][:n_text]
    got["audio_k"], got["audio_v"] = ckv[0][n_text:], ckv[1][n_text:]


def split_weights(g):
    """gate_w and proj_w as their two matrices each, compared one by one."""
    for name in ("gate_w", "proj_w"):
        for m in range(2):
            g[f"{name}[{m}]"] = g[name][m]
        del g[name]
    return g


def rounding_sensitivity(x, dout, dctx, w, ctx_rows, trials=2, seed=5):
    """Largest relative change (max abs over the RMS) of every oracle gradient when every input is
    perturbed by up to 2^-24 of itself (the rounding of an fp32 input), over ``trials`` random
    perturbations: how much of an fp32 bar the problem's own conditioning already takes."""
    ref = split_weights(bwd.vdn_backward(x, dout, w.T, w.N, w.C, w.anchors, dctx_out=dctx if ctx_rows else None))
    rng = np.random.default_rng(seed)
    out = {name: 0.0 for name in ref}
    for _ in range(trials):
        xp = {k: v * (1.0 + 2.0 ** -24 * rng.uniform(-1.0, 1.0, v.shape)) for k, v in x.items()}
        g = split_weights(bwd.vdn_backward(xp, dout, w.T, w.N, w.C, w.anchors, dctx_out=dctx if ctx_rows else None))
        for name, r in ref.items():
            if r.size and np.any(r):
                out[name] = max(out[name], rel_err(g[name], r))
    return out


def check_joint_backward(w, n_audio, ctx_rows=True, seed=0, decay=False, generic=False, conditioning=False):
    """GPU gradients against the oracle's.  With ``conditioning`` (fp32 plans), each gradient may
    also differ by sqrt(2 d) times its sensitivity to rounding the inputs to fp32
    (``rounding_sensitivity``): fp32 sums of d terms gather rounding errors that grow like
    sqrt(d) 2^-24 in the random-rounding model, and an ill-conditioned step (the RMSNorm of a
    nearly empty linear memory's readout) amplifies them exactly as it amplifies input rounding."""
    inp = synth.make_inputs(w, seed=seed, decay=decay, n_audio=n_audio, ctx_rows=ctx_rows)
    n_ctx = w.n_text + n_audio
    rng = np.random.default_rng(seed + 99)
    dout = _round(rng.standard_normal((w.T * w.N, w.H, w.d)).astype(np.float32), w.dtype)
    dctx = _round(rng.standard_normal((n_ctx, w.H, w.d)).astype(np.float32), w.dtype)
    plan = make_plan(w, generic=generic, n_audio=n_audio)
    dev = to_device(inp, w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    print(f"joint backward {w} n_audio={n_audio} ctx_rows={ctx_rows} decay={decay} generic={generic}", flush=True)
    kw = {}
    if ctx_rows:
        kw = dict(ctx_q=dev["ctx_q"], dctx_out=torch.from_numpy(dctx).cuda().to(tdt))
    g = plan.backward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"],
                      torch.from_numpy(dout).cuda().to(tdt), alpha=dev["alpha"], **kw)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in g.items()}
    plan.close()
    if n_ctx > 0:
        split_context(got, w.n_text)
    x = {k: np.asarray(v, np.float64) for k, v in inp.items() if v is not None}
    if n_audio == 0:
        x.pop("audio_k", None)
        x.pop("audio_v", None)
    ref = bwd.vdn_backward(x, dout.astype(np.float64), w.T, w.N, w.C, w.anchors,
                           dctx_out=dctx.astype(np.float64) if ctx_rows else None)
    # the two gates' and the two projections' weight gradients are compared matrix by matrix
    split_weights(ref)
    split_weights(got)
    errs = {}
    for name, r in ref.items():
        if r.size == 0:
            continue
        # rows (tokens) whose reference gradient is exactly zero -- tokens that never reach the linear
        # memory, or a whole gradient when nothing does -- must be zero on the GPU too; the others
        # are held to the bar relative to their own RMS
        live = np.abs(r.reshape(r.shape[0], -1)).max(axis=1) > 0
        dead_err = float(np.abs(got[name][~live]).max()) if (~live).any() else 0.0
        errs[name] = max(rel_err(got[name][live], r[live]) if live.any() else 0.0, dead_err)
    # bf16 plans store o_s in bf16: the softmax-half weight gradients may differ by what that
    # storage alone makes (computed by the oracle) on top of the bar
    allow = weight_grad_storage_error(x, dout, w) if w.dtype == "bf16" else {}
    if conditioning and w.dtype == "fp32":
        sens = rounding_sensitivity(x, dout.astype(np.float64), dctx.astype(np.float64), w, ctx_rows)
        allow = {name: np.sqrt(2.0 * w.d) * v for name, v in sens.items()}
    print("   " + "  ".join(f"{k} {v:.1e}" for k, v in errs.items()) +
          "   allowance " + "  ".join(f"{k} {v:.1e}" for k, v in allow.items()), flush=True)
    assert {n for n, r in ref.items() if r.size} - {"audio_k", "audio_v"} <= set(got)
    for name, e in errs.items():
        assert e <= TOL[w.dtype] + allow.get(name, 0.0), (name, e)


JOINT_BWD = [
    # n_text, n_audio, T, N, C, H, d, dtype, anchors, decay, ctx_rows
    (3, 5, 7, 24, 2, 2, 32, "fp32", True, False, True),
    (0, 4, 6, 20, 1, 1, 16, "fp32", False, True, True),        # audio only, no text
    (2, 3, 5, 16, 5, 1, 64, "fp32", True, False, False),       # audio keys, no context rows
    (7, 9, 11, 72, 3, 2, 128, "bf16", True, True, True),
    (7, 9, 11, 72, 3, 2, 128, "bf16", True, False, False),
    (4, 0, 6, 64, 1, 1, 128, "bf16", False, False, True),      # context rows of a text-only plan
    # several 128-key blocks of global keys and several 64-row tiles of context rows, ragged, d = 64
    (70, 90, 6, 130, 2, 1, 64, "bf16", True, True, True),
    (0, 33, 7, 48, 2, 2, 128, "bf16", True, False, True),      # audio only on the matrix-core kernels
    (0, 5, 5, 48, 2, 1, 128, "bf16", True, False, True),       # no frame in the linear memory: dbeta = 0
]


@pytest.mark.parametrize("case", JOINT_BWD, ids=lambda c: "x".join(str(x) for x in c))
def test_joint_backward(case):
    n_text, n_audio, T, N, C, H, d, dtype, anchors, decay, ctx_rows = case
    w = synth.custom(n_text, T, N, C, H, d, dtype, "sigmoid", anchors)
    check_joint_backward(w, n_audio, ctx_rows=ctx_rows, seed=11, decay=decay)


def test_joint_backward_generic_bf16():
    check_joint_backward(synth.custom(5, 6, 40, 2, 2, 64, "bf16", "sigmoid", True), n_audio=7, seed=12,
                         generic=True)


def test_joint_backward_after_forward_matches():
    """On a plan with audio tokens, vdn_backward_after_forward after vdn_forward_joint gives
    vdn_backward's gradients bit for bit."""
    w = synth.custom(7, 11, 72, 3, 2, 128, "bf16", "sigmoid", True)
    n_audio = 9
    inp = synth.make_inputs(w, seed=8, n_audio=n_audio, ctx_rows=True)
    dev = to_device(inp, w.dtype)
    dout = torch.from_numpy(np.random.default_rng(5).standard_normal((w.T * w.N, w.H, w.d)).astype(np.float32))
    dout = dout.cuda().to(torch.bfloat16)
    args = (dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"], dout)
    plan = make_plan(w, n_audio=n_audio)
    ref = plan.backward(*args)
    plan.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"],
                 ctx_q=dev["ctx_q"])
    got = plan.backward(*args, after_forward=True)
    torch.cuda.synchronize()
    for name in ref:
        assert torch.equal(ref[name], got[name]), name
    plan.close()


def test_joint_backward_argument_errors():
    """Context-row pointers all or none."""
    from linear_video_attention_amd import vdn
    w = synth.custom(3, 4, 16, 2, 1, 128, "bf16", "sigmoid", True)
    n_audio = 2
    inp = synth.make_inputs(w, seed=2, n_audio=n_audio, ctx_rows=True)
    dev = to_device(inp, w.dtype)
    dout = torch.zeros((w.T * w.N, w.H, w.d), dtype=torch.bfloat16, device="cuda")
    dctx = torch.zeros((w.n_text + n_audio, w.H, w.d), dtype=torch.bfloat16, device="cuda")
    plan = make_plan(w, n_audio=n_audio)
    L = vdn.lib()
    f32 = dict(dtype=torch.float32, device="cuda")
    TN, H, d = w.T * w.N, w.H, w.d
    outs = [torch.empty((TN, H, d), **f32) for _ in range(3)] + [torch.empty((w.n_text + TN, H), **f32)]
    dcq = torch.empty((w.n_text + n_audio, H, d), **f32)
    dckv = torch.empty((2, w.n_text + n_audio, H, d), **f32)
    dw = [torch.empty((2, d, d), **f32) for _ in range(2)]
    p = lambda x: None if x is None else x.data_ptr()

    def call(cq, dco, dq_ctx):
        return L.vdn_backward_joint(plan.handle, p(dev["q"]), p(dev["k"]), p(dev["v"]), p(dev["beta"]), p(cq),
                                    p(dev["text_kv"]), None, p(dev["gate_w"]), p(dev["proj_w"]), p(dout), p(dco),
                                    *[p(x) for x in outs], p(dq_ctx), p(dckv), p(dw[0]), p(dw[1]), None, None)
    assert call(dev["ctx_q"], None, dcq) == -1
    assert call(None, dctx, None) == -1
    assert call(dev["ctx_q"], dctx, dev["ctx_q"]) == -1           # output aliases an input (and wrong dtype)
    assert call(dev["ctx_q"], dctx, dcq) == 0
    assert call(None, None, None) == 0
    torch.cuda.synchronize()
    plan.close()


def test_joint_backward_768p_sampled():
    """768p with 576 audio tokens and the text and audio query rows, in the benchmark's launch
    configuration: dq of sampled video rows against the row-wise oracle (audio keys included),
    the context rows' dq of every 16th context row against their own transpose (each row is
    independent), every gradient finite."""
    w = synth.WORKLOADS["768p"]
    n_audio = 576
    inp = synth.make_inputs(w, seed=0, n_audio=n_audio, ctx_rows=True)
    n_ctx = w.n_text + n_audio
    rng = np.random.default_rng(7)
    dout = _round(rng.standard_normal((w.T * w.N, w.H, w.d)).astype(np.float32), "bf16")
    dctx = _round(rng.standard_normal((n_ctx, w.H, w.d)).astype(np.float32), "bf16")
    plan = make_plan(w, n_audio=n_audio)
    dev = to_device(inp, w.dtype)
    print("768p joint backward on the GPU ...", flush=True)
    g = plan.backward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"],
                      torch.from_numpy(dout).cuda().to(torch.bfloat16), ctx_q=dev["ctx_q"],
                      dctx_out=torch.from_numpy(dctx).cuda().to(torch.bfloat16))
    torch.cuda.synchronize()
    rows = synth.sample_rows(w)
    crow = np.arange(0, n_ctx, 16)
    got = g["q"][torch.from_numpy(rows).cuda()].cpu().numpy()
    got_c = g["ctx_q"][torch.from_numpy(crow).cuda()].cpu().numpy()
    finite = all(bool(torch.isfinite(x).all()) for x in g.values())
    del dev, g
    plan.close()
    print("768p joint backward: oracle dq rows ...", flush=True)
    ref = bwd.dq_rows(inp, dout.astype(np.float64), w.T, w.N, w.C, w.anchors, rows)
    e = rel_err(got, ref)
    print(f"768p joint backward: dq of {len(rows)} sampled rows, err {e:.2e}", flush=True)
    keys = np.concatenate([inp["text_k"], inp["audio_k"], inp["k"]])
    vals = np.concatenate([inp["text_v"], inp["audio_v"], inp["v"]])
    ref_c = bwd.context_rows_backward(inp["ctx_q"][crow], keys, vals, dctx[crow].astype(np.float64))[0]
    e_c = rel_err(got_c, ref_c)
    print(f"768p joint backward: dq of {len(crow)} context rows, err {e_c:.2e}", flush=True)
    assert finite
    assert e <= TOL[w.dtype]
    assert e_c <= TOL[w.dtype]
