"""The allowance of the GPU suite's large-score fallback test, pinned on the CPU: with queries
scaled by 600 the exact softmax branch is nearly one-hot (max |o_s| ~ 7.6 RMS), and merely
storing that exact result in bf16 (what the layer's o_s buffer holds) already uses more than 90 %
of the plain 2e-2 RMS bar, leaving the kernel's own arithmetic almost nothing; the half-ulp
allowance the test grants is exactly the storage rounding and nothing more."""

import numpy as np
import torch

import synth
from gpu_util import TOL, bf16_half_ulp, rel_err, weight_grad_storage_error
from oracle import vdn_oracle as orc


def fallback_case():
    w = synth.custom(8, 6, 256, 2, 2, 128, "bf16", "sigmoid", True)
    inp = synth.make_inputs(w, seed=4)
    inp["q"] = torch.from_numpy(inp["q"] * np.float32(600.0)).to(torch.bfloat16).float().numpy()
    return w, inp


def test_fallback_storage_allowance():
    w, inp = fallback_case()
    ref = orc.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], w.T, w.N, w.C, w.anchors)
    ref = ref.astype(np.float64)
    stored = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.abs(ref).max() / rms > 6.0                 # nearly one-hot rows
    assert rel_err(stored, ref) > 0.9 * TOL["bf16"]       # the exact result, stored, uses > 90 % of the bar
    excess = np.max(np.abs(stored - ref) - bf16_half_ulp(ref)) / rms
    assert excess <= 1e-9                                # the allowance is the storage rounding
    # and it is not larger than needed: some element's storage error is within 1 % of its allowance
    ratio = np.abs(stored - ref) / np.maximum(bf16_half_ulp(ref), 1e-300)
    assert ratio.max() >= 0.99


def test_weight_gradient_storage_allowance():
    """The joint backward test's shape with an empty linear memory (no text, 5 audio tokens, 5
    frames of 48 tokens): attention is near uniform, so every row of a frame has nearly the same
    o_s, and storing the exact o_s in bf16 alone moves dproj_w[0] and dgate_w[0] by more than
    90 % of the plain bar.  The allowance the GPU test adds is this storage effect, computed by
    the oracle, and it stays below the plain bar on this and on a regular joint shape."""
    w = synth.custom(0, 5, 48, 2, 1, 128, "bf16", "sigmoid", True)
    inp = synth.make_inputs(w, seed=11, n_audio=5, ctx_rows=True)
    dout = np.random.default_rng(110).standard_normal((w.T * w.N, w.H, w.d))
    allow = weight_grad_storage_error(inp, dout, w)
    assert allow["proj_w[0]"] > 0.9 * TOL["bf16"] and allow["gate_w[0]"] > 0.9 * TOL["bf16"], allow
    # the allowance stays below the plain bar itself: at most a doubled bar for these gradients
    assert max(allow.values()) < TOL["bf16"], allow
    w2 = synth.custom(7, 11, 72, 3, 2, 128, "bf16", "sigmoid", True)
    inp2 = synth.make_inputs(w2, seed=11, n_audio=9, ctx_rows=True)
    dout2 = np.random.default_rng(110).standard_normal((w2.T * w2.N, w2.H, w2.d))
    allow2 = weight_grad_storage_error(inp2, dout2, w2)
    assert 0.0 < max(allow2.values()) < TOL["bf16"], allow2
