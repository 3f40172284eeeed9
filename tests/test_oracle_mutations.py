"""Planted mistakes in a private copy of the CPU oracle must each fail a pin.

Every mutant is a fresh copy of the oracle module with one function replaced by a plausible
wrong version (a dropped term, a wrong sign, a transposed operand, an off-by-one window, a wrong
scan order, ...).  The named pin must reject it; otherwise the pins would not guard the oracle.
All of this runs on the CPU.
"""

import importlib.util
import os

import numpy as np
import pytest

import pins

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "vdn_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("vdn_oracle_mutant", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def m_drop_sbar(o):
    def frame_update(s_bar, a, b):
        d = a.shape[0]
        return np.linalg.solve((np.eye(d) + a).T, b.T).T
    o.frame_update = frame_update


def m_minus_gram(o):
    def frame_update(s_bar, a, b):
        d = a.shape[0]
        return np.linalg.solve((np.eye(d) - a).T, (s_bar + b).T).T
    o.frame_update = frame_update


def m_write_transposed(o):
    orig = o.frame_stats

    def frame_stats(kf, vf, bf):
        a, b = orig(kf, vf, bf)
        return a, b.T
    o.frame_stats = frame_stats


def m_gram_unweighted(o):
    orig = o.frame_stats

    def frame_stats(kf, vf, bf):
        _, b = orig(kf, vf, bf)
        kf = np.asarray(kf, np.float64)
        return kf.T @ kf, b
    o.frame_stats = frame_stats


def m_forward_window_off_by_one(o):
    orig = o.frame_sets

    def frame_sets(t, T, C, anchors):
        w, anc, f, r = orig(t, T, C, anchors)
        bset = o.boundary_set(T, anchors)
        if t not in bset:
            c = t // C
            f = [x for x in range(T) if x not in bset and x // C <= c - 1]
        return w, anc, f, r
    o.frame_sets = frame_sets


def m_reverse_scan_increasing(o):
    def head_states(k, v, beta, text_k, text_v, h, T, N, C, anchors, text_mode="half_beta", alpha=None):
        n_text = text_k.shape[0]
        s0 = o.text_state(text_k[:, h], text_v[:, h], beta[:n_text, h], text_mode)
        order = o.scan_order(T, anchors)
        stats = {f: o.frame_stats(k[f * N:(f + 1) * N, h], v[f * N:(f + 1) * N, h],
                                  beta[n_text + f * N:n_text + (f + 1) * N, h]) for f in order}
        fwd = [s0]
        for f in order:
            fwd.append(o.frame_update(fwd[-1], *stats[f]))
        per = []
        for t in range(T):
            _, _, ff, rr = o.frame_sets(t, T, C, anchors)
            s = s0
            for f in rr:                                # wrong: farthest frame written last
                s = o.frame_update(s, *stats[f])
            per.append((fwd[len(ff)], s))
        return s0, per
    o.head_states = head_states


def m_text_full_beta(o):
    def text_state(tk, tv, tb, text_mode="half_beta"):
        d = tk.shape[-1]
        if tk.shape[0] == 0:
            return np.zeros((d, d))
        return o.frame_update(np.zeros((d, d)), *o.frame_stats(tk, tv, tb))
    o.text_state = text_state


def m_gate_transposed(o):
    def merge(q, o_s, o_l, gate_w, proj_w, eps=o.RMS_EPS):
        gw = np.asarray(gate_w, np.float64)
        pw = np.asarray(proj_w, np.float64)
        q = np.asarray(q, np.float64)
        g_s = o.sigmoid(q @ gw[0].T)
        g_l = o.sigmoid(q @ gw[1].T)
        return (g_s * o_s) @ pw[0] + (g_l * o.rms_norm(np.asarray(o_l, np.float64), eps)) @ pw[1]
    o.merge = merge


def m_no_rmsnorm(o):
    def merge(q, o_s, o_l, gate_w, proj_w, eps=o.RMS_EPS):
        gw = np.asarray(gate_w, np.float64)
        pw = np.asarray(proj_w, np.float64)
        q = np.asarray(q, np.float64)
        return (o.sigmoid(q @ gw[0]) * o_s) @ pw[0] + (o.sigmoid(q @ gw[1]) * o_l) @ pw[1]
    o.merge = merge


def m_softmax_ignores_anchors(o):
    def key_frames(t, T, C, anchors):
        return sorted(o.frame_sets(t, T, C, anchors)[0])
    o.key_frames = key_frames


def m_softmax_scale(o):
    def softmax_rows(qr, keys, vals, dtype=np.float32):
        s = (qr.astype(np.float32) @ keys.astype(np.float32).T) / np.float32(qr.shape[-1])
        p = np.exp(s - s.max(axis=1, keepdims=True))
        return (p @ vals.astype(np.float32)) / p.sum(axis=1, keepdims=True)
    o.softmax_rows = softmax_rows


def m_softmax_no_text(o):
    orig = o.softmax_branch

    def softmax_branch(q, k, v, text_k, text_v, T, N, C, anchors, rows=None, audio_k=None, audio_v=None,
                       dtype=np.float32):
        return orig(q, k, v, text_k[:0], text_v[:0], T, N, C, anchors, rows, audio_k, audio_v, dtype)
    o.softmax_branch = softmax_branch


def m_boundary_reads_states(o):
    orig = o.frame_sets

    def frame_sets(t, T, C, anchors):
        w, anc, f, r = orig(t, T, C, anchors)
        if anchors and t in (0, T - 1):
            c = t // C
            bset = o.boundary_set(T, anchors)
            f = [x for x in range(T) if x not in bset and x // C <= c - 2]
            r = [x for x in range(T) if x not in bset and x // C >= c + 2]
        return w, anc, f, r
    o.frame_sets = frame_sets


def m_decay_dropped(o):
    o.decay = lambda s, alpha_f: s


def m_decay_on_rows(o):
    def decay(s, alpha_f):
        if alpha_f is None:
            return s
        return np.asarray(alpha_f, np.float64)[:, None] * s
    o.decay = decay


def m_decay_after_solve(o):
    orig_update = o.frame_update
    pending = {}

    def decay(s, alpha_f):
        pending["alpha"] = alpha_f           # remember it; apply it to the solved state instead
        return s

    def frame_update(s_bar, a, b):
        out = orig_update(s_bar, a, b)
        alpha_f = pending.pop("alpha", None)
        return out if alpha_f is None else out * np.asarray(alpha_f, np.float64)[None, :]
    o.decay = decay
    o.frame_update = frame_update


def m_decay_reverse_uses_next_frame(o):
    orig = o.head_states

    def head_states(k, v, beta, text_k, text_v, h, T, N, C, anchors, text_mode="half_beta", alpha=None):
        if alpha is None:
            return orig(k, v, beta, text_k, text_v, h, T, N, C, anchors, text_mode)
        # forward pass unchanged, reverse pass with alpha shifted by one frame
        s0, fwd_only = orig(k, v, beta, text_k, text_v, h, T, N, C, anchors, text_mode, alpha)
        shifted = np.concatenate([alpha[1:], alpha[-1:]])
        _, rev_only = orig(k, v, beta, text_k, text_v, h, T, N, C, anchors, text_mode, shifted)
        return s0, [(fwd_only[t][0], rev_only[t][1]) for t in range(T)]
    o.head_states = head_states


def m_audio_written_to_linear(o):
    """Audio tokens treated as more prompt: appended to the text for both branches, so they are
    also written into the linear memory at initialisation (unit write strength)."""
    orig = o.vdn_forward

    def vdn_forward(inp, T, N, C, anchors=True, rows=None, text_mode="half_beta", with_intermediates=False):
        if inp.get("audio_k") is None:
            return orig(inp, T, N, C, anchors, rows, text_mode, with_intermediates)
        n_text, n_audio, H = inp["text_k"].shape[0], inp["audio_k"].shape[0], inp["q"].shape[1]
        mod = {key: val for key, val in inp.items() if key not in ("audio_k", "audio_v")}
        mod["text_k"] = np.concatenate([inp["text_k"], inp["audio_k"]])
        mod["text_v"] = np.concatenate([inp["text_v"], inp["audio_v"]])
        mod["beta"] = np.concatenate([inp["beta"][:n_text], np.ones((n_audio, H), np.float32), inp["beta"][n_text:]])
        return orig(mod, T, N, C, anchors, rows, text_mode, with_intermediates)
    o.vdn_forward = vdn_forward


def m_audio_dropped_from_softmax(o):
    orig = o.softmax_branch

    def softmax_branch(q, k, v, text_k, text_v, T, N, C, anchors, rows=None, audio_k=None, audio_v=None,
                       dtype=np.float32):
        return orig(q, k, v, text_k, text_v, T, N, C, anchors, rows, dtype=dtype)
    o.softmax_branch = softmax_branch


def m_context_rows_context_only(o):
    """Text and audio queries attend only to the text and audio tokens."""
    def context_rows(inp, T, N):
        cq = inp["ctx_q"]
        out = np.zeros(cq.shape, np.float32)
        for h in range(cq.shape[1]):
            keys = np.concatenate([inp["text_k"][:, h], inp["audio_k"][:, h]])
            vals = np.concatenate([inp["text_v"][:, h], inp["audio_v"][:, h]])
            out[:, h] = o.softmax_rows(cq[:, h], keys, vals)
        return out
    o.context_rows = context_rows


def m_context_rows_unscaled(o):
    """The 1/sqrt(d) score scale forgotten on the text and audio query rows."""
    orig = o.context_rows

    def context_rows(inp, T, N):
        mod = dict(inp)
        mod["ctx_q"] = inp["ctx_q"] * np.float32(np.sqrt(inp["ctx_q"].shape[-1]))
        return orig(mod, T, N)
    o.context_rows = context_rows


MUTANTS = [
    (m_drop_sbar, pins.pin_objective_minimum),
    (m_minus_gram, pins.pin_spectrum),
    (m_write_transposed, pins.pin_sherman_morrison),
    (m_gram_unweighted, pins.pin_objective_minimum),
    (m_forward_window_off_by_one, pins.pin_golden_frame_sets),
    (m_reverse_scan_increasing, pins.pin_bruteforce),
    (m_text_full_beta, pins.pin_text_once),
    (m_gate_transposed, pins.pin_gate_closed_forms),
    (m_no_rmsnorm, pins.pin_gate_closed_forms),
    (m_softmax_ignores_anchors, pins.pin_uniform_keys_visibility),
    (m_softmax_scale, pins.pin_bruteforce),
    (m_softmax_no_text, pins.pin_uniform_keys_visibility),
    (m_boundary_reads_states, pins.pin_partition),
    (m_decay_dropped, pins.pin_decay_zero),
    (m_decay_on_rows, pins.pin_decay_columns),
    (m_decay_after_solve, pins.pin_decay_columns),
    (m_decay_reverse_uses_next_frame, pins.pin_decay_columns),
    (m_audio_written_to_linear, pins.pin_audio_softmax_only),
    (m_audio_dropped_from_softmax, pins.pin_golden_attention_map),
    (m_context_rows_context_only, pins.pin_context_rows_sdpa),
    (m_context_rows_unscaled, pins.pin_context_rows_sdpa),
]


@pytest.mark.parametrize("mutate,pin", MUTANTS, ids=[m.__name__ for m, _ in MUTANTS])
def test_mutant_is_caught(mutate, pin):
    o = fresh_oracle()
    pin(o)                       # the unmodified copy passes
    mutate(o)
    with pytest.raises(AssertionError):
        pin(o)
