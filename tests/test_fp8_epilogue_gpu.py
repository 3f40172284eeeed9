"""MXFP8 epilogue (VDN_FLAG_FP8_EPILOGUE) against its definition and against the exact epilogue.

The epilogue alone runs through vdn_debug_epilogue on seeded inputs -- q, o_s (bf16), a chunk-state
buffer (fp32), the weights -- that the oracle takes unchanged, so:
  * GPU vs the definition (oracle/mxfp8.epilogue_mx), element by element: within the allowance
    for E4M3 elements the GPU may round the other way (its gate sums, sigmoid and readout are
    computed values; the readout's error bound 2^-15 sum_k |S_jk q_k| follows from the split-bf16
    states and fp32 accumulation) plus half a bf16 ulp of storage;
  * GPU vs the exact epilogue (vdn_oracle.merge): within the worst-case envelope of the E4M3
    roundings (epilogue_mx_deviation_bound) plus the same allowance and storage.
The whole layer with the MXFP8 epilogue is compared with the exact layer within that envelope
plus the bf16 bar of the rest of the layer."""

import numpy as np
import pytest
import torch

import synth
from oracle import mxfp8 as mx
from oracle import vdn_oracle as orc

pytestmark = pytest.mark.gpu

from linear_video_attention_amd import vdn  # noqa: E402
from linear_video_attention_amd.vdn import Plan  # noqa: E402

from gpu_util import bf16_half_ulp, run_layer, to_device  # noqa: E402


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


def epilogue_inputs(T, N, C, H, seed, grid=False):
    """Seeded q (L2-normalised), o_s (bf16, N(0, 0.3^2)), states ([2, Nc+1, H, d, d] fp32 with
    entries N(0, 1/d): readouts of unit scale), weights N(0, 1/d); all bf16-rounded where bf16.
    grid=True: q on multiples of 2^-7 in (-1, 1) (scaled N(0, 1/d) * 4) and state entries on
    multiples of 2^-6 with |S_fwd + S_rev| <= 1, so that every partial sum of the readout is a
    multiple of 2^-13 below 2^7: exact in fp32, with an exact split-bf16 state (low part 0)."""
    d = 128
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T * N, H, d), dtype=np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    o_s = rng.standard_normal((T * N, H, d), dtype=np.float32) * 0.3
    nc = (T + C - 1) // C
    states = (rng.standard_normal((2, nc + 1, H, d, d), dtype=np.float32) / np.sqrt(d)).astype(np.float32)
    if grid:
        q = np.clip(np.round(q * 4 * 128), -127, 127).astype(np.float32) / 128
        states = np.clip(np.round(states * 64), -32, 32).astype(np.float32) / 64
    gw = rng.standard_normal((2, d, d), dtype=np.float32) / np.sqrt(d)
    pw = rng.standard_normal((2, d, d), dtype=np.float32) / np.sqrt(d)
    t = {k: bf16(v) for k, v in (("q", q), ("o_s", o_s), ("gate_w", gw), ("proj_w", pw))}
    f = {k: v.float().numpy().astype(np.float64) for k, v in t.items()}
    f["states"] = states.astype(np.float64)
    t["states"] = torch.from_numpy(states)
    return t, f


def readout_window(f, T, N, C, anchors):
    """Bound on the GPU readout's error: 2^-15 sum_k |S_jk| |q_k| (split-bf16 states, fp32 sums)."""
    s = f["states"]
    sabs = np.stack([np.abs(s[0] + s[1]), np.zeros_like(s[0])])
    return 2.0 ** -15 * mx.readout(sabs, np.abs(f["q"]), T, N, C, anchors)


def run_debug(T, N, C, H, seed, rows=None, fp8=True, grid=False):
    t, f = epilogue_inputs(T, N, C, H, seed, grid)
    plan = Plan(T, N, C, 8, H, 128, True, "bf16", fp8_epilogue=fp8)
    dev = {k: v.to("cuda").contiguous() for k, v in t.items()}
    out = plan.debug_epilogue(dev["q"], dev["o_s"], dev["states"], dev["gate_w"], dev["proj_w"])
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    plan.close()
    if rows is not None:
        got = got[rows]
    o_l = mx.readout(f["states"], f["q"], T, N, C, True)
    win = np.zeros_like(o_l) if grid else readout_window(f, T, N, C, True)
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    return got, {k: sel(f[k]) for k in ("q", "o_s")}, sel(o_l), sel(win), f["gate_w"], f["proj_w"]


def check_mx(got, f, o_l, win, gw, pw, label):
    q, o_s = f["q"], f["o_s"]
    ref = mx.epilogue_mx(q, o_s, o_l, gw, pw)
    exact = orc.merge(q, o_s, o_l, gw, pw)
    allow = mx.epilogue_mx_allowance(q, o_s, o_l, win, gw, pw)
    store = bf16_half_ulp(got)
    rms = np.sqrt(np.mean(exact ** 2))
    err_def = np.abs(got - ref)
    ratio = err_def / (allow + store + 1e-300)
    env = mx.epilogue_mx_deviation_bound(q, o_s, o_l, gw, pw)
    err_ex = np.abs(got - exact)
    print(f"{label}: vs definition max {err_def.max() / rms:.3e} RMS (max ratio to allowance+storage "
          f"{ratio.max():.3f}; allowance nonzero beyond rel terms at {np.mean(allow > 1e-4 * rms):.4%}); "
          f"vs exact RMS {np.sqrt(np.mean(err_ex ** 2)) / rms:.4f}, max {err_ex.max() / rms:.4f}, "
          f"max ratio to envelope {(err_ex / (env + allow + store)).max():.3f}", flush=True)
    assert np.all(np.isfinite(got))
    assert np.all(err_def <= allow + store), label
    assert np.all(err_ex <= env + allow + store), label
    # the GPU deviates from the exact epilogue like the definition does
    dev_def = np.sqrt(np.mean((ref - exact) ** 2))
    assert abs(np.sqrt(np.mean(err_ex ** 2)) - dev_def) <= 0.1 * dev_def + 2e-3 * rms, label


@pytest.mark.parametrize("T,N,C,H,seed", [(7, 64, 3, 2, 0), (5, 48, 2, 1, 1), (4, 100, 5, 3, 2)])
def test_mx_epilogue_matches_definition(T, N, C, H, seed):
    """Small shapes, ragged token tiles (48 and 100 tokens per frame), boundary frames."""
    got, f, o_l, win, gw, pw = run_debug(T, N, C, H, seed)
    check_mx(got, f, o_l, win, gw, pw, f"T={T} N={N} C={C} H={H}")


@pytest.mark.parametrize("T,N,C,H,seed", [(7, 64, 3, 2, 7), (3, 200, 2, 2, 8)])
def test_mx_epilogue_matches_definition_exact_readout(T, N, C, H, seed):
    """Grid inputs on which the GPU readout is exact: the allowance keeps only the gate-sum and
    sigmoid terms, so almost every element must match the definition to bf16 storage."""
    got, f, o_l, win, gw, pw = run_debug(T, N, C, H, seed, grid=True)
    check_mx(got, f, o_l, win, gw, pw, f"grid T={T} N={N} C={C} H={H}")


def test_mx_epilogue_768p_shape_sampled_rows():
    """The 768p launch shape (75 frames x 1536 tokens, 5 heads) on 4096 sampled token rows."""
    T, N, C, H = 75, 1536, 5, 5
    rows = np.sort(np.random.default_rng(11).choice(T * N, 4096, replace=False))
    got, f, o_l, win, gw, pw = run_debug(T, N, C, H, 3, rows=rows)
    check_mx(got, f, o_l, win, gw, pw, "768p sampled")


def test_bf16_debug_epilogue_matches_exact():
    """The same entry point on a bf16 plan: the exact epilogue within the bf16 bar."""
    T, N, C, H = 6, 80, 3, 2
    got, f, o_l, win, gw, pw = run_debug(T, N, C, H, 4, fp8=False)
    exact = orc.merge(f["q"], f["o_s"], o_l, gw, pw)
    rms = np.sqrt(np.mean(exact ** 2))
    e = np.abs(got - exact).max() / rms
    print(f"bf16 debug epilogue: {e:.3e} RMS", flush=True)
    assert e <= 2e-2


def test_layer_with_mx_epilogue_near_exact():
    """The whole layer (bf16 softmax and linear branches, MXFP8 epilogue) against the exact layer:
    the E4M3 envelope of the epilogue at the exact intermediates plus the bf16 bar."""
    w = synth.custom(16, 10, 128, 5, 2, 128, "bf16")
    inp = synth.make_inputs(w, seed=5)
    plan = Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, fp8_epilogue=True)
    assert plan.kernel_kind(vdn.VDN_STAGE_EPILOGUE) == 2
    out = run_layer(plan, to_device(inp, w.dtype)).float().cpu().numpy().astype(np.float64)
    plan.close()
    ref, mids = orc.vdn_forward(inp, w.T, w.N, w.C, w.anchors, with_intermediates=True)
    f = {k: np.asarray(inp[k], np.float64) for k in ("q", "gate_w", "proj_w")}
    q = f["q"]
    o_s = np.asarray(mids["o_s"], np.float64)
    o_l = np.asarray(mids["o_l"], np.float64)
    env = mx.epilogue_mx_deviation_bound(q, o_s, o_l, f["gate_w"], f["proj_w"])
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(out - ref)
    dev_def = np.sqrt(np.mean((mx.epilogue_mx(q, o_s, o_l, f["gate_w"], f["proj_w"]) - ref) ** 2)) / rms
    print(f"layer with MXFP8 epilogue: RMS {np.sqrt(np.mean(err ** 2)) / rms:.4f} (definition {dev_def:.4f}), "
          f"max ratio to envelope+bar {(err / (env + 2e-2 * rms)).max():.3f}", flush=True)
    assert np.all(np.isfinite(out))
    assert np.all(err <= env + 2e-2 * rms)
    assert np.sqrt(np.mean(err ** 2)) / rms <= 1.2 * dev_def + 5e-3


def test_fp8_softmax_and_mx_epilogue_together():
    """Both FP8 paths in one plan: finite, and the layer within the two envelopes' scale of the
    exact one (the FP8 softmax's own deviation is checked by its tests)."""
    w = synth.custom(16, 10, 128, 5, 2, 128, "bf16")
    inp = synth.make_inputs(w, seed=6)
    plan = Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, fp8=True, fp8_epilogue=True)
    assert plan.kernel_kind(vdn.VDN_STAGE_SOFTMAX) == 2 and plan.kernel_kind(vdn.VDN_STAGE_EPILOGUE) == 2
    out = run_layer(plan, to_device(inp, w.dtype)).float().cpu().numpy().astype(np.float64)
    plan.close()
    ref = orc.vdn_forward(inp, w.T, w.N, w.C, w.anchors)
    rms = np.sqrt(np.mean(ref ** 2))
    e = np.sqrt(np.mean((out - ref) ** 2)) / rms
    print(f"FP8 softmax + MXFP8 epilogue: RMS deviation {e:.4f}", flush=True)
    assert np.all(np.isfinite(out)) and e <= 0.1


def test_debug_epilogue_argument_errors():
    T, N, C, H = 4, 32, 2, 1
    t, _ = epilogue_inputs(T, N, C, H, 0)
    dev = {k: v.to("cuda").contiguous() for k, v in t.items()}
    plan = Plan(T, N, C, 8, H, 128, True, "bf16", fp8_epilogue=True)
    L = vdn.lib()
    args = [dev[k].data_ptr() for k in ("q", "o_s")] + [dev["states"].data_ptr(), dev["gate_w"].data_ptr(),
                                                       dev["proj_w"].data_ptr()]
    # out on top of o_s, on top of q, and a null pointer
    assert L.vdn_debug_epilogue(plan.handle, *args, dev["o_s"].data_ptr(), None) == vdn.VDN_ERR_INVALID_ARG
    assert L.vdn_debug_epilogue(plan.handle, *args, dev["q"].data_ptr(), None) == vdn.VDN_ERR_INVALID_ARG
    assert L.vdn_debug_epilogue(plan.handle, *args, None, None) == vdn.VDN_ERR_INVALID_ARG
    plan.close()
    gplan = Plan(T, N, C, 8, H, 128, True, "bf16", generic=True)
    out = torch.empty_like(dev["q"])
    assert L.vdn_debug_epilogue(gplan.handle, *args, out.data_ptr(), None) == vdn.VDN_ERR_UNSUPPORTED
    gplan.close()
