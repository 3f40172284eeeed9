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
