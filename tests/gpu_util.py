"""Helpers for the GPU tests: move seeded inputs to the device and run the layer through the C ABI."""

from __future__ import annotations

import numpy as np
import torch

from linear_video_attention_amd.vdn import VDN_BUF_OS, VDN_BUF_STATES, Plan

TOL = {"fp32": 1e-4, "bf16": 2e-2}   # max |gpu - oracle| <= TOL * RMS(oracle)


def to_device(inp: dict, dtype: str) -> dict:
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = {}
    for key in ("q", "k", "v", "gate_w", "proj_w"):
        dev[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to("cuda").to(tdt).contiguous()
    dev["beta"] = torch.from_numpy(np.ascontiguousarray(inp["beta"])).to("cuda").float().contiguous()
    ck, cv = inp["text_k"], inp["text_v"]
    if inp.get("audio_k") is not None:                  # context tokens: text rows, then audio
        ck = np.concatenate([ck, inp["audio_k"]])
        cv = np.concatenate([cv, inp["audio_v"]])
    if ck.shape[0] > 0:
        tkv = np.stack([ck, cv])
        dev["text_kv"] = torch.from_numpy(np.ascontiguousarray(tkv)).to("cuda").to(tdt).contiguous()
    else:
        dev["text_kv"] = None
    dev["ctx_q"] = None
    if inp.get("ctx_q") is not None:
        dev["ctx_q"] = torch.from_numpy(np.ascontiguousarray(inp["ctx_q"])).to("cuda").to(tdt).contiguous()
    dev["alpha"] = None
    if inp.get("alpha") is not None:
        dev["alpha"] = torch.from_numpy(np.ascontiguousarray(inp["alpha"])).to("cuda").float().contiguous()
    return dev


def make_plan(w, generic=False, n_audio=0) -> Plan:
    return Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, generic=generic, n_audio=n_audio)


def run_joint(plan: Plan, dev: dict):
    """The joint forward: (video rows out, context rows out)."""
    out, ctx = plan.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"],
                            dev["proj_w"], alpha=dev.get("alpha"), ctx_q=dev["ctx_q"])
    torch.cuda.synchronize()
    return out, ctx


def run_layer(plan: Plan, dev: dict, out=None):
    out = plan.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["text_kv"], dev["gate_w"], dev["proj_w"], out,
                       alpha=dev.get("alpha"))
    torch.cuda.synchronize()
    return out


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / rms)


def combined_states(plan: Plan) -> np.ndarray:
    """GPU readout state per query frame: S_fwd[c] + S_rev[c], slot Nc (= S0) for boundary frames."""
    st = plan.debug_buffer(VDN_BUF_STATES).double().cpu().numpy()
    res = np.zeros((plan.T, plan.H, plan.d, plan.d))
    for t in range(plan.T):
        bnd = plan.anchors and t in (0, plan.T - 1)
        slot = plan.Nc if bnd else t // plan.C
        res[t] = st[0, slot] + st[1, slot]
    return res


def softmax_out(plan: Plan) -> np.ndarray:
    return plan.debug_buffer(VDN_BUF_OS).float().cpu().numpy()


def oracle_layer_rows(inp: dict, w, rows=None, workers: int = 8, softmax_fn=None):
    """The oracle's layer output (and o_s) for the given video rows (every row when None).

    The same functions as ``vdn_oracle.vdn_forward``: the softmax branch frame by frame, here
    spread over a thread pool (numpy releases the GIL in its matrix products and exponentials, and
    each worker's BLAS is held to two threads), then the linear branch and the merge.
    ``softmax_fn(rows)`` replaces the exact softmax branch (the FP8 definition)."""
    import concurrent.futures

    import threadpoolctl

    from oracle import vdn_oracle as orc
    rows = np.arange(w.T * w.N) if rows is None else np.asarray(rows)
    frames = rows // w.N
    groups = [np.nonzero(frames == t)[0] for t in np.unique(frames)]
    if softmax_fn is None:
        def softmax_fn(r):
            return orc.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], w.T, w.N, w.C,
                                      w.anchors, r, inp.get("audio_k"), inp.get("audio_v"))
    o_s = np.zeros((len(rows), w.H, w.d))
    with threadpoolctl.threadpool_limits(2):
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            for sel, res in zip(groups, ex.map(lambda g: softmax_fn(rows[g]), groups)):
                o_s[sel] = res
        o_l = orc.linear_branch(inp["q"], inp["k"], inp["v"], inp["beta"], inp["text_k"], inp["text_v"], w.T, w.N,
                                w.C, w.anchors, rows, alpha=inp.get("alpha"))
    out = orc.merge(inp["q"][rows], o_s, o_l, inp["gate_w"], inp["proj_w"])
    return out, o_s


def describe_error(got, ref) -> str:
    """Max |got - ref| / RMS(ref), where it occurs (|ref| / RMS there), and the largest error left
    after subtracting half a bf16 unit of |ref| (the rounding of a stored bf16 value)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    err = np.abs(got - ref)
    i = int(np.argmax(err))
    ax = np.abs(ref)
    half_ulp = np.where(ax > 0, 2.0 ** (np.floor(np.log2(np.maximum(ax, 1e-30))) - 8), 0.0)
    return (f"max err {err.flat[i] / rms:.3e} RMS at |ref| = {ax.flat[i] / rms:.2f} RMS; max |ref| "
            f"{ax.max() / rms:.2f} RMS; beyond bf16 storage {np.max(err - half_ulp) / rms:.3e} RMS")


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place of |x| (8 significant bits): the largest move of storing
    x in bf16 (round to nearest)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(ax, 1e-30)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def weight_grad_storage_error(inp: dict, dout, w) -> dict:
    """The part of the softmax-half weight gradients (gate_w[0], proj_w[0]) that storing o_s in bf16
    alone makes, as a fraction of each one's RMS: the oracle's merge backward with o_s rounded to
    bf16 against the same with o_s exact.  Both gradients sum x_s = sigmoid(q Wg0) * o_s over
    every row, so where the attention is near uniform (rows of a frame with nearly the same o_s)
    the storage roundings add up coherently."""
    from oracle import vdn_backward as bwd
    from oracle import vdn_oracle as orc
    x = {k: np.asarray(v, np.float64) for k, v in inp.items() if v is not None}
    audio = {}
    if x.get("audio_k") is not None and x["audio_k"].shape[0] > 0:
        audio = dict(audio_k=x["audio_k"], audio_v=x["audio_v"])
    o_s = orc.softmax_branch(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.T, w.N, w.C, w.anchors,
                             dtype=np.float64, **audio)
    o_l = orc.linear_branch(x["q"], x["k"], x["v"], x["beta"], x["text_k"], x["text_v"], w.T, w.N, w.C,
                            w.anchors, alpha=x.get("alpha"))
    stored = torch.from_numpy(o_s.astype(np.float32)).to(torch.bfloat16).double().numpy()
    dout = np.asarray(dout, np.float64)
    _, _, _, dg, dp = bwd.merge_backward(x["q"], o_s, o_l, x["gate_w"], x["proj_w"], dout)
    _, _, _, dg16, dp16 = bwd.merge_backward(x["q"], stored, o_l, x["gate_w"], x["proj_w"], dout)
    return {"gate_w[0]": rel_err(dg16[0], dg[0]), "proj_w[0]": rel_err(dp16[0], dp[0])}
