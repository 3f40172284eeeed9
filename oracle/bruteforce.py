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
  times the diagonal matrix of alpha_f (a matrix product here).

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


def layer_dense(inp, T, N, C, anchors=True, eps=1e-6):
    q = inp["q"]
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
