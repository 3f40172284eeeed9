"""The allowance of the GPU suite's large-score fallback test, pinned on the CPU: with queries
scaled by 600 the exact softmax branch is nearly one-hot (max |o_s| ~ 7.6 RMS), and merely
storing that exact result in bf16 (what the layer's o_s buffer holds) already uses more than 90 %
of the plain 2e-2 RMS bar, leaving the kernel's own arithmetic almost nothing; the half-ulp
allowance the test grants is exactly the storage rounding and nothing more."""

import numpy as np
import torch

import synth
from gpu_util import TOL, bf16_half_ulp, rel_err
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
