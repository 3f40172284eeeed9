"""CPU oracle for the forward pass of the Video DeltaNet (VDN) hybrid video-video attention layer.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain definition that the GPU path is checked
against.  Only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import or call it.  It imports nothing from the GPU package, and the GPU package
imports nothing from here.

Sources (cited by page title and section; no other document is used):

* [VDN] "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models" (openvdn.github.io).
  Sections: "Local Softmax and Long-Range Linear Memory", "Gating the Softmax and Linear Branch
  Outputs", "Video Delta Attention: A Frame-Wise Solution" with its sub-part "From independent
  token updates to one frame-wise solve" (and the review of the token-wise rule before it, which
  defines the channel-wise decay of the inherited state), "Stability of the Inherited State".
* [FTP] "Faster Than It Plays: Video DeltaNet Generates 14 Seconds of 768p Video in 11 Seconds"
  (ai-blog.deepmagic.app), section "Two branches instead of one", which prints the closed-form
  frame update S_t = (S_bar + B)(I + A)^-1 in text.
* [GLN] "Video DeltaNet speeds MiniMax H3 video generation 14.5x" (glonce.com), its summary and
  key facts: the hybrid attention replaces only video-to-video interactions; every interaction
  with a text or audio token keeps the model's full softmax attention.

Precision: the softmax branch is computed in float32 with float32 accumulation; the text
initialisation, the per-frame solves, the two state scans, the readout and the merge are computed
in float64.  Inputs are taken as given (for bfloat16 workloads: the bf16-rounded values, upcast).

Layouts (token-major, head inside the token): q, k, v ``[T*N, H, d]``; text_k, text_v
``[n_text, H, d]``; beta ``[n_text + T*N, H]`` with the text rows first; gate_w and proj_w
``[2, d, d]`` stored [in][out] (y = x @ W), index 0 for the softmax branch and 1 for the linear
branch.

Readings of points the pages leave open (each one is also listed in the design notes):

* softmax scale tau = 1/sqrt(d); one normaliser over text, window and anchor keys together;
* text is written into each direction's state by one joint frame-wise solve from the zero state
  with every text weight halved (beta/2) -- ``text_mode="half_beta"``; the alternative reading
  (solve at full beta, then halve the state) is kept as ``text_mode="half_state"``;
* boundary query frames read only the text part of the linear memory (both scans empty), so no
  video frame reaches them twice;
* decay: none by default (alpha == 1, the inherited state is the previous state); with an alpha
  argument ``[T, H, d]``, writing frame f first decays the inherited state channel-wise,
  S_bar = S Diag(alpha_f), in either scan direction (the same alpha_f for both); the text
  initialisation starts from the zero state and is unaffected;
* the linear-branch output is RMS-normalised over d with eps = 1e-6 and unit weight, gated by
  sigmoid(q @ W_gate[1]); the softmax branch is gated by sigmoid(q @ W_gate[0]); each gated
  branch goes through its own projection and the two are summed (no residual);
* audio tokens (optional ``audio_k``, ``audio_v`` ``[n_audio, H, d]``): global keys of the
  softmax branch exactly like the text keys (same normaliser), never written into the linear
  memory (only the text prompt initialises it);
* text and audio query rows (optional ``ctx_q`` ``[n_text + n_audio, H, d]``, text rows first):
  one plain softmax over every token (text, audio and all video tokens), fp32; the result is the
  attention output before any projection (the model's own output projection applies to it, as
  it did before the hybrid layer).
"""

from __future__ import annotations

import math

import numpy as np

RMS_EPS = 1e-6


# ----------------------------------------------------------------------------------------------
# Frame bookkeeping.  [VDN] "Local Softmax and Long-Range Linear Memory": frames are grouped into
# chunks of C consecutive latent frames; a chunk sees itself and its two neighbouring chunks; the
# first and last frames are anchors that every frame sees and that see every frame; the forward
# linear state covers the frames before the window, the reverse state the frames after it, and
# neither covers window or boundary frames.
# ----------------------------------------------------------------------------------------------

def boundary_set(T: int, anchors: bool) -> list[int]:
    """The boundary (anchor) frames: the first and the last frame when anchors are on."""
    if not anchors:
        return []
    return sorted({0, T - 1})


def frame_sets(t: int, T: int, C: int, anchors: bool):
    """Return (W, Anc, F, R) for query frame ``t`` as sorted lists of frame indices.

    W: window frames (chunk distance at most one); Anc: anchor frames outside the window (for a
    boundary query frame: every frame outside the window); F: frames summarised by the forward
    state; R: frames summarised by the reverse state.
    """
    c = t // C
    bset = boundary_set(T, anchors)
    window = [f for f in range(T) if abs(f // C - c) <= 1]
    if t in bset:
        anc = [f for f in range(T) if f not in window]
        return window, anc, [], []
    anc = [f for f in bset if f not in window]
    fwd = [f for f in range(T) if f not in bset and f // C <= c - 2]
    rev = [f for f in range(T) if f not in bset and f // C >= c + 2]
    return window, anc, fwd, rev


# ----------------------------------------------------------------------------------------------
# Softmax branch.  [VDN] "Local Softmax and Long-Range Linear Memory": text tokens stay visible to
# every frame; the softmax attends to text, window and anchor keys.  Exact softmax, fp32.
# ----------------------------------------------------------------------------------------------

def softmax_rows(qr: np.ndarray, keys: np.ndarray, vals: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Exact softmax attention of query rows ``qr`` [m, d] over keys/values [n, d], in ``dtype``
    (fp32 by default; fp64 for derivative checks)."""
    d = qr.shape[-1]
    tau = dtype(1.0 / math.sqrt(d))
    s = (qr.astype(dtype) @ keys.astype(dtype).T) * tau
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s, dtype=dtype)
    return (p @ vals.astype(dtype)) / p.sum(axis=1, keepdims=True, dtype=dtype)


def key_frames(t: int, T: int, C: int, anchors: bool) -> list[int]:
    window, anc, _, _ = frame_sets(t, T, C, anchors)
    return sorted(window + anc)


def softmax_branch(q, k, v, text_k, text_v, T, N, C, anchors, rows=None, audio_k=None,
                   audio_v=None, dtype=np.float32) -> np.ndarray:
    """o_s for every video token (``rows=None``) or for the given token indices; float32.

    Global keys are the text tokens and, when given, the audio tokens ([GLN]: interactions with
    audio stay in the softmax).  Returns an array shaped like ``q`` (``rows=None``) or
    ``[len(rows), H, d]``.
    """
    if audio_k is not None:
        text_k = np.concatenate([text_k, audio_k], axis=0)
        text_v = np.concatenate([text_v, audio_v], axis=0)
    TN, H, d = q.shape
    assert TN == T * N
    rows = np.arange(TN) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), H, d), dtype)
    frames_of_rows = rows // N
    for t in np.unique(frames_of_rows):
        sel = np.nonzero(frames_of_rows == t)[0]
        kf = key_frames(int(t), T, C, anchors)
        idx = np.concatenate([np.arange(f * N, (f + 1) * N) for f in kf])
        for h in range(H):
            keys = np.concatenate([text_k[:, h], k[idx, h]], axis=0)
            vals = np.concatenate([text_v[:, h], v[idx, h]], axis=0)
            out[sel, h] = softmax_rows(q[rows[sel], h], keys, vals, dtype)
    return out


# ----------------------------------------------------------------------------------------------
# Video Delta Attention.  [VDN] "Video Delta Attention: A Frame-Wise Solution" / "From independent
# token updates to one frame-wise solve"; [FTP] "Two branches instead of one".
# The frame's tokens jointly minimise  1/2 sum_u beta_u ||S k_u - v_u||^2 + 1/2 ||S - S_bar||_F^2,
# whose stationarity condition is S (I + A) = S_bar + B with A = K^T Diag(beta) K and
# B = V^T Diag(beta) K, so S = (S_bar + B)(I + A)^-1.  All fp64.
# ----------------------------------------------------------------------------------------------

def frame_stats(kf: np.ndarray, vf: np.ndarray, bf: np.ndarray):
    """Weighted key Gram A = sum_u b_u k_u k_u^T and write matrix B = sum_u b_u v_u k_u^T."""
    kf = np.asarray(kf, np.float64)
    vf = np.asarray(vf, np.float64)
    bf = np.asarray(bf, np.float64)
    a = kf.T @ (bf[:, None] * kf)
    b = vf.T @ (bf[:, None] * kf)
    return a, b


def decay(s: np.ndarray, alpha_f) -> np.ndarray:
    """The inherited state S_bar = S Diag(alpha_f): key channel j (column j) scaled by alpha_f[j]
    ([VDN] "Video Delta Attention: A Frame-Wise Solution", the channel-wise decay gate)."""
    if alpha_f is None:
        return s
    return s * np.asarray(alpha_f, np.float64)[None, :]


def frame_update(s_bar: np.ndarray, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Closed-form frame update S = (S_bar + B)(I + A)^-1, via a linear solve (no inverse)."""
    d = a.shape[0]
    rhs = s_bar + b
    # S (I + A) = rhs  <=>  (I + A)^T S^T = rhs^T
    return np.linalg.solve((np.eye(d) + a).T, rhs.T).T


def text_state(tk: np.ndarray, tv: np.ndarray, tb: np.ndarray, text_mode: str = "half_beta"):
    """Initial state of each direction from the text tokens of one head.

    [VDN] "Local Softmax and Long-Range Linear Memory": the prompt is written once, at
    initialisation, into both the forward and the reverse state through the delta rule, each at
    one half, so that the two readouts together carry the text once.
    """
    d = tk.shape[-1]
    zero = np.zeros((d, d))
    if tk.shape[0] == 0:
        return zero
    if text_mode == "half_beta":
        a, b = frame_stats(tk, tv, 0.5 * np.asarray(tb, np.float64))
        return frame_update(zero, a, b)
    if text_mode == "half_state":
        a, b = frame_stats(tk, tv, tb)
        return 0.5 * frame_update(zero, a, b)
    raise ValueError(text_mode)


def scan_order(T: int, anchors: bool) -> list[int]:
    """Frames written into the linear memory, in forward order (boundary frames excluded)."""
    bset = boundary_set(T, anchors)
    return [f for f in range(T) if f not in bset]


def head_states(k, v, beta, text_k, text_v, h, T, N, C, anchors, text_mode="half_beta", alpha=None):
    """For one head: S0 and, for every query frame t, (S_fwd(t), S_rev(t)) in fp64.

    S_fwd(t) is the forward state after exactly the frames F(t) in increasing order; S_rev(t) is
    the reverse state after exactly R(t) in decreasing order (nearest frame written last).  With
    ``alpha`` ([T, H, d]), writing frame f updates decay(S, alpha[f, h]) instead of S.
    """
    alpha_of = (lambda f: None) if alpha is None else (lambda f: alpha[f, h])
    n_text = text_k.shape[0]
    s0 = text_state(text_k[:, h], text_v[:, h], beta[:n_text, h], text_mode)
    order = scan_order(T, anchors)
    stats = {}
    for f in order:
        sl = slice(f * N, (f + 1) * N)
        stats[f] = frame_stats(k[sl, h], v[sl, h], beta[n_text + f * N:n_text + (f + 1) * N, h])
    # prefix states of the forward scan and of the reverse scan
    fwd_prefix = [s0]
    for f in order:
        fwd_prefix.append(frame_update(decay(fwd_prefix[-1], alpha_of(f)), *stats[f]))
    rev_prefix = [s0]
    for f in reversed(order):
        rev_prefix.append(frame_update(decay(rev_prefix[-1], alpha_of(f)), *stats[f]))
    per_frame = []
    for t in range(T):
        _, _, fwd, rev = frame_sets(t, T, C, anchors)
        assert fwd == order[:len(fwd)], "forward set must be a prefix of the scan order"
        assert rev[::-1] == order[::-1][:len(rev)], "reverse set must be a suffix of the scan order"
        per_frame.append((fwd_prefix[len(fwd)], rev_prefix[len(rev)]))
    return s0, per_frame


def linear_branch(q, k, v, beta, text_k, text_v, T, N, C, anchors, rows=None,
                  text_mode="half_beta", return_states=False, alpha=None):
    """o_l = (S_fwd(t) + S_rev(t)) q for each video token; fp64."""
    TN, H, d = q.shape
    rows = np.arange(TN) if rows is None else np.asarray(rows)
    o_l = np.zeros((len(rows), H, d))
    states = []
    for h in range(H):
        s0, per_frame = head_states(k, v, beta, text_k, text_v, h, T, N, C, anchors, text_mode, alpha)
        states.append((s0, per_frame))
        for j, i in enumerate(rows):
            sf, sr = per_frame[i // N]
            o_l[j, h] = (sf + sr) @ np.asarray(q[i, h], np.float64)
    if return_states:
        return o_l, states
    return o_l


# ----------------------------------------------------------------------------------------------
# Merge.  [VDN] "Gating the Softmax and Linear Branch Outputs": each branch gets a content-dependent
# sigmoid gate and its own output projection; the linear branch is RMS-normalised before its gate;
# both projected branches are added.  fp64.
# ----------------------------------------------------------------------------------------------

def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def rms_norm(x, eps=RMS_EPS):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def merge(q, o_s, o_l, gate_w, proj_w, eps=RMS_EPS):
    q = np.asarray(q, np.float64)
    gw = np.asarray(gate_w, np.float64)
    pw = np.asarray(proj_w, np.float64)
    g_s = sigmoid(q @ gw[0])
    g_l = sigmoid(q @ gw[1])
    r = rms_norm(np.asarray(o_l, np.float64), eps)
    return (g_s * np.asarray(o_s, np.float64)) @ pw[0] + (g_l * r) @ pw[1]


# ----------------------------------------------------------------------------------------------
# The whole layer.
# ----------------------------------------------------------------------------------------------

def vdn_forward(inp: dict, T, N, C, anchors=True, rows=None, text_mode="half_beta",
                with_intermediates=False, softmax_dtype=np.float32):
    """Layer output ``out`` [len(rows) or T*N, H, d] (fp64) from the inputs dict.

    ``inp`` holds float32 arrays: q, k, v, text_k, text_v, beta, gate_w, proj_w, and optionally
    alpha ``[T, H, d]`` (the decay gate; absent = no decay) and audio_k, audio_v
    ``[n_audio, H, d]`` (global softmax keys; absent = none).  Video query rows only; the text
    and audio query rows are ``context_rows``.
    """
    q, k, v = inp["q"], inp["k"], inp["v"]
    tk, tv = inp["text_k"], inp["text_v"]
    beta = inp["beta"]
    rows_arr = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    o_s = softmax_branch(q, k, v, tk, tv, T, N, C, anchors, rows_arr, inp.get("audio_k"), inp.get("audio_v"),
                         softmax_dtype)
    o_l = linear_branch(q, k, v, beta, tk, tv, T, N, C, anchors, rows_arr, text_mode,
                        alpha=inp.get("alpha"))
    out = merge(q[rows_arr], o_s, o_l, inp["gate_w"], inp["proj_w"])
    if with_intermediates:
        return out, {"o_s": o_s, "o_l": o_l}
    return out


def context_rows(inp: dict, T, N, dtype=np.float32) -> np.ndarray:
    """Text and audio query rows ``[n_text + n_audio, H, d]`` (in ``dtype``: fp32 by default, fp64
    for derivative checks).

    [GLN]: interactions that involve a text or audio token keep the full softmax attention, so a
    text or audio query attends to every token of the sequence (text, audio and every video
    frame) under one softmax, with the layer's scale 1/sqrt(d).
    """
    cq = inp["ctx_q"]
    H = cq.shape[1]
    parts_k = [inp["text_k"]] + ([inp["audio_k"]] if inp.get("audio_k") is not None else []) + [inp["k"]]
    parts_v = [inp["text_v"]] + ([inp["audio_v"]] if inp.get("audio_v") is not None else []) + [inp["v"]]
    assert inp["k"].shape[0] == T * N
    out = np.zeros(cq.shape, dtype)
    for h in range(H):
        keys = np.concatenate([p[:, h] for p in parts_k], axis=0)
        vals = np.concatenate([p[:, h] for p in parts_v], axis=0)
        out[:, h] = softmax_rows(cq[:, h], keys, vals, dtype)
    return out


def chunk_states(inp: dict, T, N, C, anchors=True, text_mode="half_beta"):
    """Per query frame t and head h the combined readout state S_fwd(t) + S_rev(t); [T, H, d, d]."""
    q = inp["q"]
    H, d = q.shape[1], q.shape[2]
    res = np.zeros((T, H, d, d))
    for h in range(H):
        _, per_frame = head_states(inp["k"], inp["v"], inp["beta"], inp["text_k"], inp["text_v"],
                                   h, T, N, C, anchors, text_mode, inp.get("alpha"))
        for t in range(T):
            res[t, h] = per_frame[t][0] + per_frame[t][1]
    return res
