"""Brute-force CPU oracle for tiny VDN layers.

TEST INFRASTRUCTURE ONLY (same rules as ``vdn_oracle``: only tests, the smoke check and the
benchmark's CPU-baseline leg may use it; it shares nothing with the GPU path).

It is written independently of ``vdn_oracle`` so the two can check each other:

* the softmax branch uses a dense (T*N) x (n_text + T*N) boolean mask built token by token from
  the visibility rule of [VDN] "Local Softmax and Long-Range Linear Memory" (chunk distance at most
  one, boundary anchors in both directions, text always visible) and a masked dense softmax;
* every frame update is obtained by minimising the frame objective of [VDN] "From independent
  token updates to one frame-wise solve" -- a beta-weighted least-squares fit of the reads
  S k_u ~ v_u plus the proximity term ||S - S_bar||_F^2 -- with a generic least-squares routine on
  the stacked system, never through the closed form;
* each query frame's forward and reverse states are rebuilt from the text state in fresh loops
  over the frames the rule assigns to it (no reuse between query frames);
* with a decay gate alpha ``[T, H, d]`` the proximity target of frame f is the inherited state
  times the diagonal matrix of alpha_f (a matrix product here);
* with audio tokens and text/audio query rows ([GLN] "Video DeltaNet speeds MiniMax H3 video
  generation 14.5x": every interaction involving text or audio stays softmax attention), the
  whole sequence [text, audio, video] gets one dense mask built entry by entry from a per-token
  kind: a text or audio query sees every token, a text or audio key is seen by every query,
  video-video pairs follow the frame rule; audio never enters the linear memory.

[VDN] = "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models" (openvdn.github.io).
"""

from __future__ import annotations

import math

import numpy as np


def visible(i_frame: int, j_frame: int, T: int, C: int, anchors: bool) -> bool:
    """Softmax visibility of a key in frame j_frame for a query in frame i_frame."""
    if abs(i_frame // C - j_frame // C) <= 1:
        return True
    if anchors and (j_frame in (0, T - 1) or i_frame in (0, T - 1)):
        return True
    return False


def dense_mask(T, N, n_text, C, anchors) -> np.ndarray:
    m = np.zeros((T * N, n_text + T * N), bool)
    m[:, :n_text] = True
    for i in range(T * N):
        for j in range(T * N):
            m[i, n_text + j] = visible(i // N, j // N, T, C, anchors)
    return m


def token_kinds(n_text, n_audio, T, N):
    """Kind and frame of every token of the joint sequence [text, audio, video]."""
    kinds = ["text"] * n_text + ["audio"] * n_audio + ["video"] * (T * N)
    frames = [-1] * (n_text + n_audio) + [j // N for j in range(T * N)]
    return kinds, frames


def joint_mask(n_text, n_audio, T, N, C, anchors) -> np.ndarray:
    """Softmax visibility over the joint sequence, query x key."""
    kinds, frames = token_kinds(n_text, n_audio, T, N)
    L = len(kinds)
    m = np.zeros((L, L), bool)
    for i in range(L):
        for j in range(L):
            if kinds[i] != "video" or kinds[j] != "video":
                m[i, j] = True
            else:
                m[i, j] = visible(frames[i], frames[j], T, C, anchors)
    return m


def joint_softmax_dense(inp, T, N, C, anchors):
    """Softmax output of every token of the joint sequence [text, audio, video] under joint_mask;
    the text and audio queries are ``inp["ctx_q"]`` (text rows first)."""
    n_text = inp["text_k"].shape[0]
    has_audio = inp.get("audio_k") is not None
    n_audio = inp["audio_k"].shape[0] if has_audio else 0
    def seq(text, audio, video):
        return np.concatenate([inp[text]] + ([inp[audio]] if has_audio else []) + [inp[video]], axis=0)
    ctx_q = inp.get("ctx_q")
    if ctx_q is None:                                  # no context rows wanted: placeholder queries
        ctx_q = np.zeros((n_text + n_audio,) + inp["q"].shape[1:], np.float32)
    qs = np.concatenate([ctx_q, inp["q"]], axis=0)
    ks = seq("text_k", "audio_k", "k")
    vs = seq("text_v", "audio_v", "v")
    mask = joint_mask(n_text, n_audio, T, N, C, anchors)
    d = qs.shape[-1]
    out = np.zeros(qs.shape, np.float32)
    for h in range(qs.shape[1]):
        s = (qs[:, h].astype(np.float32) @ ks[:, h].astype(np.float32).T) / np.float32(math.sqrt(d))
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h] = (p @ vs[:, h].astype(np.float32)) / p.sum(axis=1, keepdims=True)
    return out


def softmax_dense(q, k, v, text_k, text_v, T, N, C, anchors) -> np.ndarray:
    TN, H, d = q.shape
    n_text = text_k.shape[0]
    mask = dense_mask(T, N, n_text, C, anchors)
    out = np.zeros(q.shape, np.float32)
    for h in range(H):
        keys = np.concatenate([text_k[:, h], k[:, h]]).astype(np.float32)
        vals = np.concatenate([text_v[:, h], v[:, h]]).astype(np.float32)
        s = (q[:, h].astype(np.float32) @ keys.T) / np.float32(math.sqrt(d))
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h] = (p @ vals) / p.sum(axis=1, keepdims=True)
    return out


def lstsq_update(s_bar, keys, vals, weights):
    """argmin_S 1/2 sum_u w_u ||S k_u - v_u||^2 + 1/2 ||S - S_bar||_F^2 by least squares.

    Row r of S only meets row r of the targets, so each row is the least-squares solution of the
    stacked system [sqrt(w) * K ; I] s_r = [sqrt(w) * V[:, r] ; s_bar[r]].
    """
    d = s_bar.shape[0]
    sw = np.sqrt(np.asarray(weights, np.float64))[:, None]
    lhs = np.concatenate([sw * np.asarray(keys, np.float64), np.eye(d)])
    rhs = np.concatenate([sw * np.asarray(vals, np.float64), s_bar.T])
    sol, *_ = np.linalg.lstsq(lhs, rhs, rcond=None)
    return sol.T


def linear_dense(q, k, v, beta, text_k, text_v, T, N, C, anchors, alpha=None):
    TN, H, d = q.shape
    def inherited(s, f, h):
        return s if alpha is None else s @ np.diag(np.asarray(alpha[f, h], np.float64))
    n_text = text_k.shape[0]
    out = np.zeros(q.shape)
    bset = (0, T - 1) if anchors else ()
    for h in range(H):
        s_text = lstsq_update(np.zeros((d, d)), text_k[:, h], text_v[:, h], 0.5 * beta[:n_text, h])
        for t in range(T):
            c = t // C
            fwd = np.array(s_text)
            rev = np.array(s_text)
            if t not in bset:
                for f in range(T):                       # frames before the window, nearest last
                    if f not in bset and f // C < c - 1:
                        sl = slice(f * N, (f + 1) * N)
                        fwd = lstsq_update(inherited(fwd, f, h), k[sl, h], v[sl, h],
                                           beta[n_text + f * N:n_text + (f + 1) * N, h])
                for f in range(T - 1, -1, -1):           # frames after the window, nearest last
                    if f not in bset and f // C > c + 1:
                        sl = slice(f * N, (f + 1) * N)
                        rev = lstsq_update(inherited(rev, f, h), k[sl, h], v[sl, h],
                                           beta[n_text + f * N:n_text + (f + 1) * N, h])
            for n in range(N):
                i = t * N + n
                out[i, h] = fwd @ q[i, h] + rev @ q[i, h]
    return out


def context_dense(inp, T, N, C, anchors=True):
    """The text and audio query rows of the joint softmax, ``[n_text + n_audio, H, d]``."""
    return joint_softmax_dense(inp, T, N, C, anchors)[:inp["ctx_q"].shape[0]]


def layer_dense(inp, T, N, C, anchors=True, eps=1e-6):
    q = inp["q"]
    if inp.get("audio_k") is not None:
        o_s = joint_softmax_dense(inp, T, N, C, anchors)[-q.shape[0]:]
    else:
        o_s = softmax_dense(q, inp["k"], inp["v"], inp["text_k"], inp["text_v"], T, N, C, anchors)
    o_l = linear_dense(q, inp["k"], inp["v"], inp["beta"], inp["text_k"], inp["text_v"], T, N, C, anchors,
                       inp.get("alpha"))
    q64 = q.astype(np.float64)
    gw = inp["gate_w"].astype(np.float64)
    pw = inp["proj_w"].astype(np.float64)
    out = np.zeros(q.shape)
    for i in range(q.shape[0]):
        for h in range(q.shape[1]):
            x = q64[i, h]
            g_soft = 1.0 / (1.0 + np.exp(-(x @ gw[0])))
            g_lin = 1.0 / (1.0 + np.exp(-(x @ gw[1])))
            ol = o_l[i, h]
            normed = ol / math.sqrt(float(np.dot(ol, ol)) / ol.size + eps)
            out[i, h] = (g_soft * o_s[i, h]) @ pw[0] + (g_lin * normed) @ pw[1]
    return out, o_s, o_l
