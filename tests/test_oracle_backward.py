"""The backward-pass oracle against autograd and finite differences (no GPU)."""

import pytest

import pins
from oracle import vdn_backward as bwd


@pytest.mark.parametrize("pin", [pins.pin_backward_autograd, pins.pin_backward_finite_differences,
                                 pins.pin_joint_backward_autograd, pins.pin_joint_backward_finite_differences],
                         ids=lambda f: f.__name__)
def test_pin(pin):
    pin(bwd)


import importlib.util
import math
import os

import numpy as np

BWD_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "vdn_backward.py")


def fresh_backward():
    spec = importlib.util.spec_from_file_location("vdn_backward_mutant", BWD_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def m_softmax_no_rowsum(b):
    """The rowsum(P dP) term of the softmax Jacobian dropped."""
    orig_exp = np.exp

    def softmax_backward(q, k, v, text_k, text_v, T, N, C, anchors, do_s):
        import math
        TN, H, d = q.shape
        tau = 1.0 / math.sqrt(d)
        n_text = text_k.shape[0]
        dq = np.zeros((TN, H, d)); dk = np.zeros((TN, H, d)); dv = np.zeros((TN, H, d))
        dtk = np.zeros((n_text, H, d)); dtv = np.zeros((n_text, H, d))
        for t in range(T):
            rows = np.arange(t * N, (t + 1) * N)
            kf = b.orc.key_frames(t, T, C, anchors)
            idx = np.concatenate([np.arange(f * N, (f + 1) * N) for f in kf])
            for h in range(H):
                qh = q[rows, h].astype(np.float64)
                keys = np.concatenate([text_k[:, h], k[idx, h]]).astype(np.float64)
                vals = np.concatenate([text_v[:, h], v[idx, h]]).astype(np.float64)
                s = tau * (qh @ keys.T)
                p = orig_exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                do = do_s[rows, h].astype(np.float64)
                ds = p * (do @ vals.T)
                dq[rows, h] += tau * (ds @ keys)
                dkeys, dvals = tau * (ds.T @ qh), p.T @ do
                dtk[:, h] += dkeys[:n_text]; dtv[:, h] += dvals[:n_text]
                dk[idx, h] += dkeys[n_text:]; dv[idx, h] += dvals[n_text:]
        return dq, dk, dv, dtk, dtv
    b.softmax_backward = softmax_backward


def m_text_full_weight(b):
    """Text token gradients taken at full write strength instead of beta/2."""
    orig = b.frame_stats_backward
    b.frame_stats_backward = lambda kf, vf, bf, da, db, weight_scale=1.0: orig(kf, vf, bf, da, db, 1.0)


def m_gram_gradient_sign(b):
    """dA taken as +M dM M (the inverse's derivative with the wrong sign)."""
    orig = b.frame_stats_backward
    b.frame_stats_backward = lambda kf, vf, bf, da, db, weight_scale=1.0: orig(kf, vf, bf, -da, db, weight_scale)


def m_rms_no_projection(b):
    """The RMSNorm Jacobian reduced to 1/rho (its projection term dropped)."""
    orig = b.merge_backward

    def merge_backward(q, o_s, o_l, gate_w, proj_w, dout, eps=b.orc.RMS_EPS):
        dq, do_s, do_l, dgate, dproj = orig(q, o_s, o_l, gate_w, proj_w, dout, eps)
        o_l = np.asarray(o_l, np.float64)
        rho = np.sqrt(np.mean(o_l * o_l, axis=-1, keepdims=True) + eps)
        r = o_l / rho
        dr = do_l * rho + r * np.mean(r * (do_l * rho), axis=-1, keepdims=True)  # undo, then drop
        return dq, do_s, dr / rho, dgate, dproj
    b.merge_backward = merge_backward


def m_context_rows_no_rowsum(b):
    """The context rows' softmax Jacobian without its rowsum(P dP) term."""
    import math

    def context_rows_backward(ctx_q, keys, vals, do_ctx):
        n_ctx, H, d = ctx_q.shape
        tau = 1.0 / math.sqrt(d)
        dq = np.zeros((n_ctx, H, d)); dkeys = np.zeros(keys.shape); dvals = np.zeros(vals.shape)
        for h in range(H):
            s = tau * (ctx_q[:, h] @ keys[:, h].T)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            ds = p * (do_ctx[:, h] @ vals[:, h].T)
            dq[:, h] = tau * (ds @ keys[:, h])
            dkeys[:, h] = tau * (ds.T @ ctx_q[:, h])
            dvals[:, h] = p.T @ do_ctx[:, h]
        return dq, dkeys, dvals
    b.context_rows_backward = context_rows_backward


def m_context_key_grad_unscaled(b):
    """The context rows' key gradient taken without the softmax scale tau."""
    orig = b.context_rows_backward

    def context_rows_backward(ctx_q, keys, vals, do_ctx):
        dq, dkeys, dvals = orig(ctx_q, keys, vals, do_ctx)
        return dq, dkeys * math.sqrt(ctx_q.shape[-1]), dvals
    b.context_rows_backward = context_rows_backward


def m_audio_keys_left_out(b):
    """The video rows' softmax transpose run over the text keys only (audio keys forgotten)."""
    orig = b.softmax_backward

    def softmax_backward(q, k, v, text_k, text_v, T, N, C, anchors, do_s, audio_k=None, audio_v=None):
        dq, dk, dv, dgk, dgv = orig(q, k, v, text_k, text_v, T, N, C, anchors, do_s)
        if audio_k is not None:
            dgk = np.concatenate([dgk, np.zeros(audio_k.shape)])
            dgv = np.concatenate([dgv, np.zeros(audio_v.shape)])
        return dq, dk, dv, dgk, dgv
    b.softmax_backward = softmax_backward


BWD_MUTANTS = [
    (m_context_rows_no_rowsum, pins.pin_joint_backward_autograd),
    (m_context_key_grad_unscaled, pins.pin_joint_backward_finite_differences),
    (m_audio_keys_left_out, pins.pin_joint_backward_autograd),
    (m_softmax_no_rowsum, pins.pin_backward_autograd),
    (m_text_full_weight, pins.pin_backward_autograd),
    (m_gram_gradient_sign, pins.pin_backward_finite_differences),
    (m_rms_no_projection, pins.pin_backward_finite_differences),
]


@pytest.mark.parametrize("mutate,pin", BWD_MUTANTS, ids=[m.__name__ for m, _ in BWD_MUTANTS])
def test_backward_mutant_is_caught(mutate, pin):
    b = fresh_backward()
    pin(b)
    mutate(b)
    with pytest.raises(AssertionError):
        pin(b)


def test_dq_rows_equals_full_backward():
    """The row-wise dq (used for full-size sampled checks) equals the full reverse-mode dq."""
    rng = np.random.default_rng(60)
    T, N, C, n_text, H, d = 9, 3, 2, 2, 2, 6
    inp = pins._bwd_inputs(T, N, n_text, H, d, False, 61)
    dout = rng.standard_normal((T * N, H, d))
    full = bwd.vdn_backward(inp, dout, T, N, C, True)["q"]
    rows = np.array([0, 4, 13, T * N - 1])
    assert np.allclose(bwd.dq_rows(inp, dout, T, N, C, True, rows), full[rows], rtol=1e-10, atol=1e-12)
