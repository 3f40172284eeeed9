"""CPU oracle for the backward pass (reverse mode) of the VDN hybrid video-video attention layer.

TEST INFRASTRUCTURE ONLY (same rules as ``vdn_oracle``: only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; it shares nothing with the GPU path).

Given the layer inputs and the gradient ``dout`` of a scalar loss with respect to the layer output
``out`` (video rows), it returns the gradients with respect to every input: q, k, v, beta, the
text keys and values, the gate and projection weights, and (with a decay gate) alpha.  Each step
below is the transpose of the corresponding step of the forward definition in ``vdn_oracle``
(which cites the pages), written out in float64:

* merge ([VDN] "Gating the Softmax and Linear Branch Outputs"): out = (g_s * o_s) Wp0 +
  (g_l * r) Wp1, g = sigmoid(q Wg), r = o_l / sqrt(mean(o_l^2) + eps);
* softmax branch ([VDN] "Local Softmax and Long-Range Linear Memory"): o = P V with
  P = softmax(tau q K^T) over each query frame's key set; dP = do V^T, dS = P (dP - rowsum(P dP)),
  dq = tau dS K, dK = tau dS^T q, dV = P^T do;
* linear branch ([VDN] "Video Delta Attention: A Frame-Wise Solution"; [FTP] "Two branches
  instead of one"): every frame step Z' = (Z Diag(alpha_f) + B_f) M_f with M_f = (I + A_f)^-1,
  A_f = sum beta k k^T, B_f = sum beta v k^T; readout o_l = (Z_fwd + Z_rev) q.  Transposed:
  with R = Z Diag(alpha) + B,  dR = dZ' M^T,  dM = R^T dZ',  dA = -M^T dM M^T,  dB = dR,
  dZ += dR Diag(alpha),  dalpha_j += (Z^T dR)_jj;  and per token  dk = beta (dA + dA^T) k +
  beta dB^T v,  dv = beta dB k,  dbeta = k^T dA k + v^T dB k (text tokens at beta/2).

[VDN] = "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models" (openvdn.github.io);
[FTP] = "Faster Than It Plays: Video DeltaNet Generates 14 Seconds of 768p Video in 11 Seconds"
(ai-blog.deepmagic.app).

Joint sequences ([GLN] = "Video DeltaNet speeds MiniMax H3 video generation 14.5x", summary: every
interaction with a text or audio token keeps the full softmax attention): audio keys are global
softmax keys of the video rows beside the text keys, so their gradients come from the same softmax
transpose; the text and audio query rows are one plain softmax over every key, whose transpose is
the same three products (``context_rows_backward``).  Audio tokens never enter the linear memory.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import vdn_oracle as orc


def merge_backward(q, o_s, o_l, gate_w, proj_w, dout, eps=orc.RMS_EPS):
    """Gradients of the merge: (dq from the gates, do_s, do_l, dgate_w, dproj_w); rows of any
    leading shape [..., d]."""
    q = np.asarray(q, np.float64)
    o_s = np.asarray(o_s, np.float64)
    o_l = np.asarray(o_l, np.float64)
    dout = np.asarray(dout, np.float64)
    gw = np.asarray(gate_w, np.float64)
    pw = np.asarray(proj_w, np.float64)
    d = q.shape[-1]
    g_s = orc.sigmoid(q @ gw[0])
    g_l = orc.sigmoid(q @ gw[1])
    rho = np.sqrt(np.mean(o_l * o_l, axis=-1, keepdims=True) + eps)
    r = o_l / rho
    x_s, x_l = g_s * o_s, g_l * r
    flat = lambda x: x.reshape(-1, d)
    dproj = np.stack([flat(x_s).T @ flat(dout), flat(x_l).T @ flat(dout)])
    dx_s, dx_l = dout @ pw[0].T, dout @ pw[1].T
    do_s = dx_s * g_s
    dz_s = dx_s * o_s * g_s * (1.0 - g_s)
    dr = dx_l * g_l
    dz_l = dx_l * r * g_l * (1.0 - g_l)
    # r = o_l / rho(o_l):  d o_l = (dr - r mean(r dr)) / rho
    do_l = (dr - r * np.mean(r * dr, axis=-1, keepdims=True)) / rho
    dgate = np.stack([flat(q).T @ flat(dz_s), flat(q).T @ flat(dz_l)])
    dq = dz_s @ gw[0].T + dz_l @ gw[1].T
    return dq, do_s, do_l, dgate, dproj


def softmax_backward(q, k, v, text_k, text_v, T, N, C, anchors, do_s, audio_k=None, audio_v=None):
    """Gradients of the video rows' softmax branch: (dq, dk, dv, dglobal_k, dglobal_v), float64.

    The global keys are the text tokens followed, when given, by the audio tokens (as in
    ``vdn_oracle.softmax_branch``); dglobal_k and dglobal_v are ordered the same way."""
    if audio_k is not None:
        text_k = np.concatenate([text_k, audio_k], axis=0)
        text_v = np.concatenate([text_v, audio_v], axis=0)
    TN, H, d = q.shape
    tau = 1.0 / math.sqrt(d)
    n_text = text_k.shape[0]
    dq = np.zeros((TN, H, d))
    dk = np.zeros((TN, H, d))
    dv = np.zeros((TN, H, d))
    dtk = np.zeros((n_text, H, d))
    dtv = np.zeros((n_text, H, d))
    for t in range(T):
        rows = np.arange(t * N, (t + 1) * N)
        kf = orc.key_frames(t, T, C, anchors)
        idx = np.concatenate([np.arange(f * N, (f + 1) * N) for f in kf])
        for h in range(H):
            qh = np.asarray(q[rows, h], np.float64)
            keys = np.concatenate([text_k[:, h], k[idx, h]]).astype(np.float64)
            vals = np.concatenate([text_v[:, h], v[idx, h]]).astype(np.float64)
            s = tau * (qh @ keys.T)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            do = np.asarray(do_s[rows, h], np.float64)
            dp = do @ vals.T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[rows, h] += tau * (ds @ keys)
            dkeys = tau * (ds.T @ qh)
            dvals = p.T @ do
            dtk[:, h] += dkeys[:n_text]
            dtv[:, h] += dvals[:n_text]
            dk[idx, h] += dkeys[n_text:]
            dv[idx, h] += dvals[n_text:]
    return dq, dk, dv, dtk, dtv


def context_rows_backward(ctx_q, keys, vals, do_ctx):
    """Gradients of the text and audio query rows: (dctx_q, dkeys, dvals), float64.

    Each context row is one plain softmax over every key of the sequence ([GLN]), o = P V with
    P = softmax(tau q K^T); its transpose is dS = P (dP - rowsum(P dP)) with dP = do V^T, and
    dq = tau dS K, dK = tau dS^T q, dV = P^T do.  ``keys``, ``vals`` are [L, H, d] in the
    sequence's order (text, audio, video)."""
    n_ctx, H, d = ctx_q.shape
    tau = 1.0 / math.sqrt(d)
    dq = np.zeros((n_ctx, H, d))
    dkeys = np.zeros(keys.shape)
    dvals = np.zeros(vals.shape)
    for h in range(H):
        qh = np.asarray(ctx_q[:, h], np.float64)
        kh = np.asarray(keys[:, h], np.float64)
        vh = np.asarray(vals[:, h], np.float64)
        s = tau * (qh @ kh.T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        do = np.asarray(do_ctx[:, h], np.float64)
        dp = do @ vh.T
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        dq[:, h] = tau * (ds @ kh)
        dkeys[:, h] = tau * (ds.T @ qh)
        dvals[:, h] = p.T @ do
    return dq, dkeys, dvals


def frame_stats_backward(kf, vf, bf, da, db, weight_scale=1.0):
    """Token gradients of A = sum w k k^T, B = sum w v k^T with w = weight_scale * beta, given dA,
    dB: (dk, dv, dbeta)."""
    kf = np.asarray(kf, np.float64)
    vf = np.asarray(vf, np.float64)
    w = weight_scale * np.asarray(bf, np.float64)
    dsym = da + da.T
    dk = w[:, None] * (kf @ dsym.T) + w[:, None] * (vf @ db)          # (dA + dA^T) k + dB^T v
    dv = w[:, None] * (kf @ db.T)                                     # dB k
    dbeta = weight_scale * (np.einsum("ui,ij,uj->u", kf, da, kf) + np.einsum("ui,ij,uj->u", vf, db, kf))
    return dk, dv, dbeta


def linear_backward(q, k, v, beta, text_k, text_v, T, N, C, anchors, do_l, alpha=None):
    """Gradients of the linear branch: (dq, dk, dv, dbeta, dtext_k, dtext_v, dalpha), float64."""
    TN, H, d = q.shape
    n_text = text_k.shape[0]
    dq = np.zeros((TN, H, d))
    dk = np.zeros((TN, H, d))
    dv = np.zeros((TN, H, d))
    dbeta = np.zeros(beta.shape)
    dtk = np.zeros((n_text, H, d))
    dtv = np.zeros((n_text, H, d))
    dalpha = None if alpha is None else np.zeros(alpha.shape)
    order = orc.scan_order(T, anchors)
    eye = np.eye(d)
    for h in range(H):
        # forward recomputation: per-frame stats, inverses and prefix states of both scans
        stats = {}
        for f in order:
            sl = slice(f * N, (f + 1) * N)
            stats[f] = orc.frame_stats(k[sl, h], v[sl, h], beta[n_text + f * N:n_text + (f + 1) * N, h])
        minv = {f: np.linalg.inv(eye + stats[f][0]) for f in order}
        a_of = (lambda f: np.ones(d)) if alpha is None else (lambda f: np.asarray(alpha[f, h], np.float64))
        if n_text > 0:
            a0, b0 = orc.frame_stats(text_k[:, h], text_v[:, h], 0.5 * np.asarray(beta[:n_text, h], np.float64))
            m0 = np.linalg.inv(eye + a0)
            s0 = b0 @ m0
        else:
            s0 = np.zeros((d, d))
        scans = {}
        for name, seq in (("fwd", order), ("rev", order[::-1])):
            z = [s0]
            for f in seq:
                z.append((z[-1] * a_of(f)[None, :] + stats[f][1]) @ minv[f])
            scans[name] = (seq, z)
        # readout: o_l = (Z_fwd[|F(t)|] + Z_rev[|R(t)|]) q
        dz = {name: [np.zeros((d, d)) for _ in scans[name][1]] for name in scans}
        for t in range(T):
            _, _, fset, rset = orc.frame_sets(t, T, C, anchors)
            rows = slice(t * N, (t + 1) * N)
            qh = np.asarray(q[rows, h], np.float64)
            dl = np.asarray(do_l[rows, h], np.float64)
            zsum = scans["fwd"][1][len(fset)] + scans["rev"][1][len(rset)]
            dq[rows, h] += dl @ zsum
            g = dl.T @ qh                       # sum_i do_l_i q_i^T
            dz["fwd"][len(fset)] += g
            dz["rev"][len(rset)] += g
        # transposed scans: per-frame dA, dB (both directions), dalpha
        da = {f: np.zeros((d, d)) for f in order}
        db = {f: np.zeros((d, d)) for f in order}
        ds0 = np.zeros((d, d))
        for name in scans:
            seq, z = scans[name]
            adj = [x.copy() for x in dz[name]]
            for m in range(len(seq), 0, -1):
                f = seq[m - 1]
                af = a_of(f)
                rhs = z[m - 1] * af[None, :] + stats[f][1]
                drhs = adj[m] @ minv[f].T
                dm = rhs.T @ adj[m]
                da[f] += -minv[f].T @ dm @ minv[f].T
                db[f] += drhs
                adj[m - 1] += drhs * af[None, :]
                if dalpha is not None:
                    dalpha[f, h] += np.sum(z[m - 1] * drhs, axis=0)
            ds0 += adj[0]
        for f in order:
            sl = slice(f * N, (f + 1) * N)
            gk, gv, gb = frame_stats_backward(k[sl, h], v[sl, h], beta[n_text + f * N:n_text + (f + 1) * N, h],
                                              da[f], db[f])
            dk[sl, h] += gk
            dv[sl, h] += gv
            dbeta[n_text + f * N:n_text + (f + 1) * N, h] += gb
        if n_text > 0:
            # S0 = (0 + B0) M0 at half write strength
            db0 = ds0 @ m0.T
            dm0 = b0.T @ ds0
            da0 = -m0.T @ dm0 @ m0.T
            gk, gv, gb = frame_stats_backward(text_k[:, h], text_v[:, h], beta[:n_text, h], da0, db0, 0.5)
            dtk[:, h] += gk
            dtv[:, h] += gv
            dbeta[:n_text, h] += gb
    return dq, dk, dv, dbeta, dtk, dtv, dalpha


def vdn_backward(inp: dict, dout, T, N, C, anchors=True, dctx_out=None):
    """All input gradients of the layer for the output gradient ``dout`` [T*N, H, d] (float64).

    Returns a dict with q, k, v, beta, text_k, text_v, gate_w, proj_w and, when ``inp`` has a decay
    gate, alpha.  With audio tokens (``audio_k``, ``audio_v`` in ``inp``) it also holds audio_k and
    audio_v.  ``dctx_out`` [n_text + n_audio, H, d] is the gradient of the text and audio query
    rows' output (``vdn_oracle.context_rows`` of ``inp["ctx_q"]``); when given, their transpose is
    added and the dict also holds ctx_q."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    tk, tv, beta = inp["text_k"], inp["text_v"], inp["beta"]
    alpha = inp.get("alpha")
    n_text = tk.shape[0]
    audio = {}
    if inp.get("audio_k") is not None:
        audio = dict(audio_k=inp["audio_k"], audio_v=inp["audio_v"])
    o_s = orc.softmax_branch(q, k, v, tk, tv, T, N, C, anchors, dtype=np.float64, **audio)
    o_l = orc.linear_branch(q, k, v, beta, tk, tv, T, N, C, anchors, alpha=alpha)
    dq_m, do_s, do_l, dgate, dproj = merge_backward(q, o_s, o_l, inp["gate_w"], inp["proj_w"], dout)
    dq_s, dk_s, dv_s, dgk_s, dgv_s = softmax_backward(q, k, v, tk, tv, T, N, C, anchors, do_s, **audio)
    dq_l, dk_l, dv_l, dbeta, dtk_l, dtv_l, dalpha = linear_backward(q, k, v, beta, tk, tv, T, N, C, anchors,
                                                                   do_l, alpha)
    grads = dict(q=dq_m + dq_s + dq_l, k=dk_s + dk_l, v=dv_s + dv_l, beta=dbeta, text_k=dgk_s[:n_text] + dtk_l,
                 text_v=dgv_s[:n_text] + dtv_l, gate_w=dgate, proj_w=dproj)
    if audio:
        grads["audio_k"] = dgk_s[n_text:]
        grads["audio_v"] = dgv_s[n_text:]
    if alpha is not None:
        grads["alpha"] = dalpha
    if dctx_out is not None:
        parts_k = [tk] + ([audio["audio_k"]] if audio else []) + [k]
        parts_v = [tv] + ([audio["audio_v"]] if audio else []) + [v]
        dcq, dka, dva = context_rows_backward(inp["ctx_q"], np.concatenate(parts_k), np.concatenate(parts_v),
                                              dctx_out)
        n_ctx = dcq.shape[0]
        grads["ctx_q"] = dcq
        grads["text_k"] = grads["text_k"] + dka[:n_text]
        grads["text_v"] = grads["text_v"] + dva[:n_text]
        if audio:
            grads["audio_k"] = grads["audio_k"] + dka[n_text:n_ctx]
            grads["audio_v"] = grads["audio_v"] + dva[n_text:n_ctx]
        grads["k"] = grads["k"] + dka[n_ctx:]
        grads["v"] = grads["v"] + dva[n_ctx:]
    return grads


def dq_rows(inp: dict, dout, T, N, C, anchors, rows):
    """dq of the given video rows only (float64 [len(rows), H, d]): the merge, softmax and readout
    parts of ``vdn_backward``'s dq, evaluated row by row (each needs only its own key set and the
    two states of its frame), so that it stays cheap at full size."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    tk, tv, beta = inp["text_k"], inp["text_v"], inp["beta"]
    if inp.get("audio_k") is not None:          # global softmax keys: text, then audio
        gk = np.concatenate([tk, inp["audio_k"]])
        gv = np.concatenate([tv, inp["audio_v"]])
    else:
        gk, gv = tk, tv
    TN, H, d = q.shape
    tau = 1.0 / math.sqrt(d)
    rows = np.asarray(rows)
    out = np.zeros((len(rows), H, d))
    for h in range(H):
        _, per_frame = orc.head_states(k, v, beta, tk, tv, h, T, N, C, anchors, alpha=inp.get("alpha"))
        for j, i in enumerate(rows):
            t = int(i) // N
            kf = orc.key_frames(t, T, C, anchors)
            idx = np.concatenate([np.arange(f * N, (f + 1) * N) for f in kf])
            keys = np.concatenate([gk[:, h], k[idx, h]]).astype(np.float64)
            vals = np.concatenate([gv[:, h], v[idx, h]]).astype(np.float64)
            qi = np.asarray(q[i, h], np.float64)
            s = tau * (keys @ qi)
            p = np.exp(s - s.max())
            p /= p.sum()
            o_s = p @ vals
            zsum = per_frame[t][0] + per_frame[t][1]
            o_l = zsum @ qi
            dq_m, do_s, do_l, _, _ = merge_backward(qi[None], o_s[None], o_l[None], inp["gate_w"], inp["proj_w"],
                                                    np.asarray(dout[i, h], np.float64)[None])
            dp = vals @ do_s[0]
            ds = p * (dp - np.sum(p * dp))
            out[j, h] = dq_m[0] + tau * (ds @ keys) + do_l[0] @ zsum
    return out
