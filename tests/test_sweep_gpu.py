"""A seeded sweep over small shapes: forward and backward of the whole layer against the oracle in
every combination the plans accept -- fp32 and bf16, d = 16 to 128, ragged frames, one to twelve
frames, chunk sizes larger than the sequence, with and without text, audio, context rows, anchors
and the decay gate (kernel families chosen by the plan).  Bars as elsewhere: 1e-4 RMS for fp32,
2e-2 RMS for bf16 (plus the oracle-computed bf16 storage effect on the softmax-half weight
gradients); the fp32 gradients may also differ by sqrt(2 d) times their measured sensitivity to
rounding the inputs to fp32, since some drawn shapes leave the linear memory nearly empty and its
RMSNorm ill-conditioned."""

import numpy as np
import pytest
import torch

import synth
from oracle import vdn_oracle as orc

pytestmark = pytest.mark.gpu

from gpu_util import TOL, make_plan, rel_err, run_joint, run_layer, to_device  # noqa: E402
from test_backward_joint_gpu import check_joint_backward  # noqa: E402


def sweep_cases(n=20, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([16, 32, 64, 128]))
        dtype = "bf16" if rng.random() < 0.6 else "fp32"
        cases.append(dict(d=d, dtype=dtype, N=int(rng.choice([8, 16, 24, 40, 72, 130])),
                          T=int(rng.integers(1, 13)), C=int(rng.integers(1, 6)), H=int(rng.integers(1, 4)),
                          n_text=int(rng.choice([0, 1, 5, 70])), n_audio=int(rng.choice([0, 0, 3, 40])),
                          anchors=bool(rng.random() < 0.7), decay=bool(rng.random() < 0.4),
                          ctx=bool(rng.random() < 0.7)))
    return cases


CASES = sweep_cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{T}x{N}x{C}x{H}x{d}x{dtype}_t{n_text}a{n_audio}".format(**c))
def test_sweep(case):
    c = case
    w = synth.custom(c["n_text"], c["T"], c["N"], c["C"], c["H"], c["d"], c["dtype"], "sigmoid", c["anchors"])
    n_ctx = c["n_text"] + c["n_audio"]
    ctx_rows = c["ctx"] and n_ctx > 0
    seed = 31 + CASES.index(case)
    print(f"sweep {c}", flush=True)
    # forward: the video rows' output and, with context rows, theirs
    inp = synth.make_inputs(w, seed=seed, decay=c["decay"], n_audio=c["n_audio"], ctx_rows=ctx_rows)
    plan = make_plan(w, n_audio=c["n_audio"])
    dev = to_device(inp, w.dtype)
    if ctx_rows:
        out, ctx = run_joint(plan, dev)
    else:
        out, ctx = run_layer(plan, dev), None
    plan.close()
    x = dict(inp)
    if c["n_audio"] == 0:
        x.pop("audio_k", None)
        x.pop("audio_v", None)
    e_out = rel_err(out.float().cpu().numpy(), orc.vdn_forward(x, w.T, w.N, w.C, w.anchors))
    e_ctx = rel_err(ctx.float().cpu().numpy(), orc.context_rows(x, w.T, w.N)) if ctx_rows else 0.0
    print(f"   forward: out {e_out:.2e}  ctx {e_ctx:.2e}", flush=True)
    assert e_out <= TOL[w.dtype] and e_ctx <= TOL[w.dtype], (e_out, e_ctx)
    # backward: every gradient
    check_joint_backward(w, c["n_audio"], ctx_rows=ctx_rows, seed=seed, decay=c["decay"], conditioning=True)
