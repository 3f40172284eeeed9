"""Parity of the FP8 softmax variant (plans created with VDN_FLAG_FP8_SOFTMAX) with its CPU oracle
(``oracle/fp8_softmax.py``), through the C ABI.

* the packed E4M3 keys and values and the per-head scales are compared byte for byte with the
  oracle's rounding of the same inputs (integer work: bit-exact);
* o_s, out and the context rows are held to the bf16 bar, max |gpu - oracle| <= 2e-2 * RMS(oracle),
  against the FP8 oracle (the GPU stores o_s in bf16, inside that bar; the two sides round the same
  values, and a weight whose exponent lands within an fp32 rounding of an E4M3 midpoint may round
  the other way, which moves o_s by far less than the bar);
* every FP8 case is also held to the pages' exact softmax branch and exact layer (``exact_checks``:
  per-element envelopes and the RMS deviation derived from the FP8 rounding steps alone);
* the row-maximum offset (rows whose bound exceeds the limit), ragged tiles, no text, anchors off,
  one frame, decay, audio keys and context rows, and 768p on sampled rows in the bench's launch
  configuration.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import TOL, rel_err, softmax_out, to_device
from linear_video_attention_amd.vdn import VDN_BUF_K8, VDN_BUF_OS, VDN_BUF_SCALES8, VDN_BUF_V8, Plan
from oracle import fp8_softmax as f8
from oracle import vdn_oracle as orc

pytestmark = pytest.mark.gpu


def fp8_plan(w, n_audio=0):
    return Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, n_audio=n_audio, fp8=True)


def forward(plan, dev, ctx=False):
    res = plan.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"],
                       alpha=dev.get("alpha"), ctx_q=dev["ctx_q"] if ctx else None)
    torch.cuda.synchronize()
    return res


def ctx_keys_values(inp):
    ck, cv = inp["text_k"], inp["text_v"]
    if inp.get("audio_k") is not None:
        ck = np.concatenate([ck, inp["audio_k"]])
        cv = np.concatenate([cv, inp["audio_v"]])
    return ck, cv


def exact_checks(inp, w, got_os, got_out, rows=None, label=""):
    """The FP8 result against the pages' exact softmax branch (``vdn_oracle``), with envelopes
    derived from the FP8 rounding steps alone (``fp8_softmax.exact_deviation_bounds``), o_s being
    stored in bf16 (up to 2^-8 of its magnitude more):
    * every element of o_s within the worst-case envelope and within the probabilistic one
      (Hoeffding, tail 1e-12 per element);
    * the RMS deviation of o_s at most 1.25x the RMS predicted from the rounding steps;
    * every element of out within the bf16 bar of the exact layer plus the probabilistic envelope
      of o_s carried through the softmax gate and projection: sum_c |g_s,c| |Wp0[c, :]| env_c."""
    rows = np.arange(w.T * w.N) if rows is None else np.asarray(rows)
    o_ex, det, prob, rms = f8.softmax_branch_bounds(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], w.T,
                                                    w.N, w.C, w.anchors, rows, inp.get("audio_k"),
                                                    inp.get("audio_v"))
    err = np.abs(np.asarray(got_os, np.float64) - o_ex)
    store = 2.0 ** -8 * (np.abs(o_ex) + prob)
    pred = float(np.sqrt(np.mean(rms ** 2 + (2.0 ** -8 * o_ex) ** 2 / 3.0)))
    meas = float(np.sqrt(np.mean(err ** 2)))
    ref_out = orc.vdn_forward(inp, w.T, w.N, w.C, w.anchors, rows=rows)
    q = inp["q"][rows].astype(np.float64)
    g_s = 1.0 / (1.0 + np.exp(-(q @ inp["gate_w"][0].astype(np.float64))))
    carried = (np.abs(g_s) * prob) @ np.abs(inp["proj_w"][0].astype(np.float64))
    rms_out = float(np.sqrt(np.mean(ref_out ** 2)))
    err_out = np.abs(np.asarray(got_out, np.float64) - ref_out)
    rms_os = float(np.sqrt(np.mean(o_ex ** 2)))
    print(f"{label} vs exact: o_s max err {err.max() / rms_os:.3f} RMS (envelopes: worst case med "
          f"{np.median(det) / rms_os:.2f}, probabilistic med {np.median(prob) / rms_os:.3f} RMS; max err/prob "
          f"{np.max(err / (prob + store)):.2f}); RMS err {meas / rms_os:.4f} vs predicted {pred / rms_os:.4f}; "
          f"out max err/bar {np.max(err_out / (TOL['bf16'] * rms_out + carried)):.2f}", flush=True)
    assert np.all(err <= det + store)
    assert np.all(err <= prob + store)
    assert meas <= 1.25 * pred, (meas, pred)
    assert np.all(err_out <= TOL["bf16"] * rms_out + carried)


def check_fp8(w, seed=0, decay=False, n_audio=0, ctx_rows=False, q_scale=None):
    inp = synth.make_inputs(w, seed=seed, decay=decay, n_audio=n_audio, ctx_rows=ctx_rows)
    if q_scale is not None:          # the oracle must see the bf16 values the device holds
        q = torch.from_numpy((inp["q"] * q_scale[:, None, None]).astype(np.float32))
        inp["q"] = q.to(torch.bfloat16).float().numpy()
    plan = fp8_plan(w, n_audio=n_audio)
    dev = to_device(inp, w.dtype)
    res = forward(plan, dev, ctx=ctx_rows)
    out, ctx = res if ctx_rows else (res, None)
    got_os = softmax_out(plan)
    got_out = out.float().cpu().numpy()
    ref_out, inter = f8.vdn_forward_fp8(inp, w.T, w.N, w.C, w.anchors, with_intermediates=True)
    e_os, e_out = rel_err(got_os, inter["o_s"]), rel_err(got_out, ref_out)
    msg = f"{w} decay={decay} audio={n_audio}: o_s {e_os:.2e} out {e_out:.2e}"
    if ctx_rows:
        ref_c = f8.context_rows_fp8(inp, w.T, w.N)
        e_c = rel_err(ctx.float().cpu().numpy(), ref_c)
        msg += f" ctx {e_c:.2e}"
        assert e_c <= TOL["bf16"]
    print(msg, flush=True)
    assert e_os <= TOL["bf16"] and e_out <= TOL["bf16"]
    exact_checks(inp, w, got_os, got_out, label=str(w))
    plan.close()
    return inp, got_os, got_out


def test_fp8_packing_is_bit_exact():
    w = synth.custom(20, 5, 48, 2, 2, 128, "bf16", "sigmoid", True)
    inp = synth.make_inputs(w, seed=1, n_audio=7)
    plan = fp8_plan(w, n_audio=7)
    dev = to_device(inp, w.dtype)
    forward(plan, dev)
    k8 = plan.debug_buffer(VDN_BUF_K8).cpu()
    v8 = plan.debug_buffer(VDN_BUF_V8).cpu()
    sc = plan.debug_buffer(VDN_BUF_SCALES8).cpu().numpy()
    ck, cv = ctx_keys_values(inp)
    n_ctx = ck.shape[0]
    pad = (n_ctx + 63) // 64 * 64
    for h in range(w.H):
        keys = np.concatenate([ck[:, h], inp["k"][:, h]])
        vals = np.concatenate([cv[:, h], inp["v"][:, h]])
        s_k, s_v, _ = f8.head_scales(keys, vals)
        assert sc[h, 0] == s_k and sc[h, 1] == s_v, (h, sc[h], s_k, s_v)
        # decode the device bytes as E4M3 and compare with the oracle's rounding, key by key
        gk = k8[h].view(torch.float8_e4m3fn).double().numpy()
        gv = v8[h].view(torch.float8_e4m3fn).double().numpy()
        want_k = np.zeros_like(gk)
        want_v = np.zeros_like(gv)
        want_k[:n_ctx] = f8.e4m3(s_k * ck[:, h])
        want_k[pad:pad + w.T * w.N] = f8.e4m3(s_k * inp["k"][:, h])
        want_v[:, :n_ctx] = f8.e4m3(s_v * cv[:, h]).T
        want_v[:, pad:pad + w.T * w.N] = f8.e4m3(s_v * inp["v"][:, h]).T
        assert np.array_equal(gk, want_k), h
        assert np.array_equal(gv, want_v), h
    plan.close()


def test_fp8_small_matches_oracle():
    check_fp8(synth.custom(24, 9, 64, 3, 2, 128, "bf16", "sigmoid", True))


FP8_RAGGED = [
    # n_text, T, N, C, H, anchors: partial 128-key tiles, no text, anchors off, one frame,
    # one frame per chunk, a single chunk, more than one workgroup per frame
    (5, 7, 48, 2, 1, True),
    (0, 6, 80, 2, 2, True),
    (13, 8, 32, 3, 1, False),
    (3, 1, 64, 5, 1, True),
    (9, 5, 16, 1, 1, True),
    (40, 4, 96, 5, 1, True),
    (2, 3, 400, 2, 1, True),
]


@pytest.mark.parametrize("case", FP8_RAGGED, ids=lambda c: "x".join(str(x) for x in c))
def test_fp8_ragged_shapes(case):
    n_text, T, N, C, H, anchors = case
    check_fp8(synth.custom(n_text, T, N, C, H, 128, "bf16", "sigmoid", anchors), seed=2)


def test_fp8_decay_and_joint():
    w = synth.custom(12, 7, 48, 2, 2, 128, "bf16", "sigmoid", True)
    check_fp8(w, seed=3, decay=True, n_audio=21, ctx_rows=True)


def test_fp8_row_maximum_offset():
    """Queries scaled by 64 on every other row, so that the bound c |q| kmax (8.2) exceeds 4 there:
    those rows take the exact row maximum as the offset (the second launch), the others keep the
    bound, inside the same workgroups.

    These rows attend sharply (the weights span four binades and their sum is small), so one
    weight that rounds to the neighbouring E4M3 value moves o by up to ~4 % of the output's RMS.
    That happens when a weight's exponent lies within the score error of an E4M3 midpoint: the
    matrix cores' fp32 score sums are not exact (one measured weight: 2^-17.6 relative), which
    shifts the exponent by up to c 2^-16 sum|Q8 K8| / (s_q s_k).  The bar per row is the bf16 bar
    plus the effect of every weight that close to a midpoint (``ambiguous_rounding_effect``; zero
    on most rows)."""
    w = synth.custom(10, 6, 64, 2, 2, 128, "bf16", "sigmoid", True)
    scale = np.where(np.arange(w.T * w.N) % 2 == 0, 64.0, 1.0)
    inp = synth.make_inputs(w, seed=4)
    q = torch.from_numpy((inp["q"] * scale[:, None, None]).astype(np.float32))
    inp["q"] = q.to(torch.bfloat16).float().numpy()
    plan = fp8_plan(w)
    dev = to_device(inp, w.dtype)
    got_out = forward(plan, dev)
    got = softmax_out(plan)
    plan.close()
    ref = f8.softmax_branch_fp8(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], w.T, w.N, w.C,
                                w.anchors)
    rms = np.sqrt(np.mean(ref ** 2))
    allow = np.zeros((w.T * w.N, w.H))
    for h in range(w.H):
        keys_all = np.concatenate([inp["text_k"][:, h], inp["k"][:, h]])
        vals_all = np.concatenate([inp["text_v"][:, h], inp["v"][:, h]])
        scales = f8.head_scales(keys_all, vals_all)
        for t in range(w.T):
            kf = orc.key_frames(t, w.T, w.C, w.anchors)
            idx = np.concatenate([np.arange(f * w.N, (f + 1) * w.N) for f in kf])
            keys = np.concatenate([inp["text_k"][:, h], inp["k"][idx, h]])
            vals = np.concatenate([inp["text_v"][:, h], inp["v"][idx, h]])
            rows = slice(t * w.N, (t + 1) * w.N)
            allow[rows, h] = f8.ambiguous_rounding_effect(inp["q"][rows, h], keys, vals, *scales)
    err = np.abs(got - ref).max(axis=2)
    bar = TOL["bf16"] * rms + allow
    print(f"row-maximum offset: max err {err.max() / rms:.2e} RMS, plain bar exceeded on "
          f"{int((err > TOL['bf16'] * rms).sum())} of {err.size} rows, max err/bar {np.max(err / bar):.2f}", flush=True)
    assert np.all(err <= bar)
    # the bound rows of the same workgroups keep the plain bar
    assert err[1::2].max() <= TOL["bf16"] * rms
    exact_checks(inp, w, got, got_out.float().cpu().numpy(), label="row-maximum offset")


def test_fp8_768p_sampled_rows():
    """768p in the benchmark's launch configuration: sampled rows of out against the FP8 oracle."""
    w = synth.WORKLOADS["768p"]
    inp = synth.make_inputs(w, seed=0)
    plan = fp8_plan(w)
    dev = to_device(inp, w.dtype)
    out = forward(plan, dev)
    rows = synth.sample_rows(w)
    got = out[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    got_os = plan.debug_buffer(VDN_BUF_OS)[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    del dev, out
    ref, inter = f8.vdn_forward_fp8(inp, w.T, w.N, w.C, w.anchors, rows=rows, with_intermediates=True)
    e, e_os = rel_err(got, ref), rel_err(got_os, inter["o_s"])
    print(f"768p fp8: out err {e:.2e}, o_s err {e_os:.2e} ({len(rows)} rows)", flush=True)
    assert e <= TOL["bf16"] and e_os <= TOL["bf16"]
    exact_checks(inp, w, got_os, got, rows, label="768p fp8")
    plan.close()


@pytest.mark.parametrize("kind", ["fp8_softmax", "fp8_epilogue", "both"])
def test_fp8_backward_is_the_exact_layers(kind):
    """The backward of an FP8 plan (straight through its roundings) is the bf16 plan's backward at
    the same inputs, bit for bit (same kernels), for vdn_backward and, on a joint plan, for
    vdn_backward_joint; vdn_backward_after_forward rejects FP8 plans (VDN_ERR_UNSUPPORTED)."""
    from linear_video_attention_amd import vdn
    w = synth.custom(4, 5, 32, 2, 1, 128, "bf16", "sigmoid", True)
    n_audio = 3
    inp = synth.make_inputs(w, seed=6, n_audio=n_audio, ctx_rows=True)
    dev = to_device(inp, w.dtype)
    rng = np.random.default_rng(8)
    dout = torch.from_numpy(rng.standard_normal((w.T * w.N, w.H, w.d)).astype(np.float32)).cuda().to(torch.bfloat16)
    dctx = torch.from_numpy(rng.standard_normal((w.n_text + n_audio, w.H, w.d)).astype(np.float32))
    dctx = dctx.cuda().to(torch.bfloat16)
    args = (dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"], dout)
    exact = Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, n_audio=n_audio)
    ref = exact.backward(*args)
    ref_j = exact.backward(*args, ctx_q=dev["ctx_q"], dctx_out=dctx)
    plan = Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, n_audio=n_audio,
                fp8=kind != "fp8_epilogue", fp8_epilogue=kind != "fp8_softmax")
    plan.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"])
    with pytest.raises(vdn.VdnError) as ei:
        plan.backward(*args, after_forward=True)
    assert ei.value.status == -2
    got = plan.backward(*args)
    got_j = plan.backward(*args, ctx_q=dev["ctx_q"], dctx_out=dctx)
    torch.cuda.synchronize()
    for r, g in ((ref, got), (ref_j, got_j)):
        assert set(r) == set(g)
        for name in r:
            assert torch.equal(r[name], g[name]), (kind, name)
    plan.close()
    exact.close()
