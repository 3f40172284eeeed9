"""CPU oracle of the FP8 variant of the VDN softmax branch.

TEST INFRASTRUCTURE ONLY (same rules as ``vdn_oracle``: only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; it shares nothing with the GPU path).

The pages run the layer with FP8 arithmetic in production ([VDN] "Adapting the Pretrained H3
backbone": optimized kernels plus FP8 cut the per-block latency further) but do not say which
roundings the FP8 path makes.  This module is the definition used here, written so that every
rounding is a stated, deterministic step; the window, anchors, global keys and the one softmax per
query are those of the exact branch ([VDN] "Local Softmax and Long-Range Linear Memory";
``vdn_oracle.softmax_branch``).

Number format: OCP FP8 E4M3 (one sign bit, four exponent bits with bias 7, three mantissa bits,
no infinities; largest finite value 448, subnormal spacing 2^-9), rounding to nearest with ties to
even; values beyond 448 saturate (the scales below keep every operand inside the range).

Definition, per head h, for a video query row q with key set J (global keys, window, anchors):

* power-of-two scales: scale(m) = 2^(8 - e) for a largest magnitude m = f 2^e, f in [0.5, 1)
  (scale(0) = 1), so the scaled values stay below 256.  s_k = scale(max |k|) and s_v =
  scale(max |v|) over every key and value of the head (global and video);
* the query enters multiplied by c = log2(e) / sqrt(d), so that scores come out in log2 units:
  s_q = scale(max |c q|) per query row, Q8 = e4m3(s_q c q); K8 = e4m3(s_k k), V8 = e4m3(s_v v);
* scores x_j = <Q8, K8_j> / (s_q s_k) (exact);
* exponent offset: with the bound b = c |q| kmax (kmax the largest key norm of the head, |q| the
  query's norm), m = b when b <= 4, else m = max_{j in J} x_j.  (Any offset gives the exact
  softmax; after rounding it matters, so it is part of the definition.  With b <= 4 every row's
  largest term 2^(8 + x - m) is at least 1.)
* P8_j = e4m3(2^(8 + x_j - m));
* o = sum_j P8_j V8_j / (s_v sum_j P8_j).

The normaliser sums the same rounded weights that multiply the values, so o is a convex
combination of the dequantised values.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import vdn_oracle as orc

E4M3_MAX = 448.0
OFFSET_BOUND_LIMIT = 4.0      # log2 units: larger bounds use the row maximum as the offset
P_SHIFT = 8.0                 # the weights are rounded as 2^8 p


def e4m3(x) -> np.ndarray:
    """Round to the nearest OCP E4M3 value (ties to even), saturating at +-448; float64 result."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                        # a = f 2^ex with f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                 # binade of a; below 2^-6 the subnormal spacing
    step = np.ldexp(1.0, (e - 3).astype(np.int64))  # three mantissa bits
    r = np.round(a / step) * step              # numpy rounds halves to even
    r = np.minimum(r, E4M3_MAX)
    return np.where(np.isnan(x), np.nan, np.copysign(r, x))


def pow2_scale(max_abs: float) -> float:
    """2^(8 - e) for max_abs = f 2^e, f in [0.5, 1); 1 for zero."""
    if max_abs == 0.0:
        return 1.0
    _, e = math.frexp(float(max_abs))
    return math.ldexp(1.0, 8 - e)


def head_scales(keys_all: np.ndarray, vals_all: np.ndarray):
    """(s_k, s_v, kmax) of one head from all of its keys and values [n, d]."""
    keys_all = np.asarray(keys_all, np.float64)
    vals_all = np.asarray(vals_all, np.float64)
    s_k = pow2_scale(np.abs(keys_all).max()) if keys_all.size else 1.0
    s_v = pow2_scale(np.abs(vals_all).max()) if vals_all.size else 1.0
    kmax = float(np.sqrt((keys_all ** 2).sum(axis=1)).max()) if keys_all.size else 0.0
    return s_k, s_v, kmax


def softmax_rows_fp8(qr, keys, vals, s_k, s_v, kmax) -> np.ndarray:
    """FP8 softmax attention of query rows ``qr`` [m, d] over ``keys``, ``vals`` [n, d] with the
    head's scales; float64 result."""
    return softmax_rows_rounded(qr, e4m3(s_k * np.asarray(keys, np.float64)),
                                e4m3(s_v * np.asarray(vals, np.float64)), s_k, s_v, kmax)


def softmax_rows_rounded(qr, k8, v8, s_k, s_v, kmax) -> np.ndarray:
    """As ``softmax_rows_fp8`` for keys and values already rounded (k8 = e4m3(s_k k), v8 likewise)."""
    qr = np.asarray(qr, np.float64)
    d = qr.shape[-1]
    c = math.log2(math.e) / math.sqrt(d)
    out = np.zeros(qr.shape)
    for i, q in enumerate(qr):
        s_q = pow2_scale(np.abs(c * q).max())
        x = (k8 @ e4m3(s_q * c * q)) / (s_q * s_k)
        b = c * math.sqrt(float(q @ q)) * kmax
        m = b if b <= OFFSET_BOUND_LIMIT else x.max()
        p8 = e4m3(np.exp2(P_SHIFT + x - m))
        out[i] = (p8 @ v8) / (s_v * p8.sum())
    return out


def ambiguous_rounding_effect(qr, keys, vals, s_k, s_v, kmax, rel_score_err=2.0 ** -16) -> np.ndarray:
    """Per query row, how far o may move when the scores carry a relative error: a weight P8_j can
    round to the other side of an E4M3 midpoint only if its exponent 8 + x_j - m lies within
    delta_j = rel_score_err sum_i |Q8_i K8_ji| / (s_q s_k) (+ a float32 rounding of the
    exponent) of the midpoint's exponent; each such weight moves o by at most one E4M3 step times
    max |V8_j / s_v - o| / sum P8.  Returns the sum over those weights (zero for most rows).  Used
    to compare with hardware whose fp32 score sums are not exact."""
    qr = np.asarray(qr, np.float64)
    d = qr.shape[-1]
    c = math.log2(math.e) / math.sqrt(d)
    k8 = e4m3(s_k * np.asarray(keys, np.float64))
    v8 = e4m3(s_v * np.asarray(vals, np.float64)) / s_v
    res = np.zeros(len(qr))
    for i, q in enumerate(qr):
        s_q = pow2_scale(np.abs(c * q).max())
        q8 = e4m3(s_q * c * q)
        x = (k8 @ q8) / (s_q * s_k)
        b = c * math.sqrt(float(q @ q)) * kmax
        m = b if b <= OFFSET_BOUND_LIMIT else x.max()
        arg = P_SHIFT + x - m
        p8 = e4m3(np.exp2(arg))
        o = (p8 @ v8) / p8.sum()
        delta = rel_score_err * (np.abs(k8) @ np.abs(q8)) / (s_q * s_k) + 2.0 ** -20 * (np.abs(arg) + P_SHIFT)
        if m != b:
            delta = delta + rel_score_err * np.max(np.abs(k8) @ np.abs(q8)) / (s_q * s_k)  # the row maximum too
        p = np.exp2(arg)
        _, ex = np.frexp(p)
        e = np.maximum(ex - 1, -6)
        step = np.ldexp(1.0, e - 3)
        mid = (np.floor(p / step) + 0.5) * step                   # midpoint above the value's floor
        near = np.minimum(np.abs(np.log2(p / mid)), np.abs(np.log2(p / np.maximum(mid - step, 2.0 ** -12))))
        amb = near < delta
        res[i] = np.sum(2 * step[amb] * np.abs(v8[amb] - o).max(axis=1)) / p8.sum()
    return res


def softmax_branch_fp8(q, k, v, text_k, text_v, T, N, C, anchors, rows=None, audio_k=None, audio_v=None):
    """o_s of the FP8 variant for every video token (``rows=None``) or the given token indices."""
    if audio_k is not None:
        text_k = np.concatenate([text_k, audio_k], axis=0)
        text_v = np.concatenate([text_v, audio_v], axis=0)
    TN, H, d = q.shape
    assert TN == T * N
    n_g = text_k.shape[0]
    rows = np.arange(TN) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), H, d))
    frames_of_rows = rows // N
    for h in range(H):
        keys_all = np.concatenate([text_k[:, h], k[:, h]]).astype(np.float64)
        vals_all = np.concatenate([text_v[:, h], v[:, h]]).astype(np.float64)
        s_k, s_v, kmax = head_scales(keys_all, vals_all)
        k8, v8 = e4m3(s_k * keys_all), e4m3(s_v * vals_all)       # every key rounded once
        for t in np.unique(frames_of_rows):
            sel = np.nonzero(frames_of_rows == t)[0]
            kf = orc.key_frames(int(t), T, C, anchors)
            idx = np.concatenate([np.arange(n_g)] + [n_g + np.arange(f * N, (f + 1) * N) for f in kf])
            out[sel, h] = softmax_rows_rounded(q[rows[sel], h], k8[idx], v8[idx], s_k, s_v, kmax)
    return out


def context_rows_fp8(inp: dict, T, N) -> np.ndarray:
    """Text and audio query rows of the FP8 variant: every key of the sequence, one softmax."""
    cq = inp["ctx_q"]
    H = cq.shape[1]
    parts_k = [inp["text_k"]] + ([inp["audio_k"]] if inp.get("audio_k") is not None else []) + [inp["k"]]
    parts_v = [inp["text_v"]] + ([inp["audio_v"]] if inp.get("audio_v") is not None else []) + [inp["v"]]
    assert inp["k"].shape[0] == T * N
    out = np.zeros(cq.shape)
    for h in range(H):
        keys = np.concatenate([p[:, h] for p in parts_k], axis=0)
        vals = np.concatenate([p[:, h] for p in parts_v], axis=0)
        out[:, h] = softmax_rows_fp8(cq[:, h], keys, vals, *head_scales(keys, vals))
    return out


def vdn_forward_fp8(inp: dict, T, N, C, anchors=True, rows=None, with_intermediates=False):
    """The layer with the FP8 softmax branch; the linear branch and the merge are the exact ones
    of ``vdn_oracle`` (float64)."""
    q = inp["q"]
    rows_arr = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    o_s = softmax_branch_fp8(q, inp["k"], inp["v"], inp["text_k"], inp["text_v"], T, N, C, anchors, rows_arr,
                             inp.get("audio_k"), inp.get("audio_v"))
    o_l = orc.linear_branch(q, inp["k"], inp["v"], inp["beta"], inp["text_k"], inp["text_v"], T, N, C, anchors,
                            rows_arr, alpha=inp.get("alpha"))
    out = orc.merge(q[rows_arr], o_s, o_l, inp["gate_w"], inp["proj_w"])
    if with_intermediates:
        return out, {"o_s": o_s, "o_l": o_l}
    return out


# ----------------------------------------------------------------------------------------------
# How far the FP8 definition may lie from the exact softmax ([VDN] "Local Softmax and Long-Range
# Linear Memory"; ``vdn_oracle.softmax_rows``), from nothing but its rounding steps.  Used to hold
# the FP8 kernel to the pages' exact branch as well as to the definition above.
# ----------------------------------------------------------------------------------------------

E4M3_REL = 2.0 ** -4          # a rounding to E4M3 moves a normal value by at most 2^-4 of itself
E4M3_ABS = 2.0 ** -10         # ... and a value below 2^-6 by at most half the spacing 2^-9


def e4m3_half_step(y) -> np.ndarray:
    """The largest move of a rounding to E4M3 near |y|: half the spacing, 2^(e-4) in the binade
    [2^e, 2^(e+1)) for |y| >= 2^-6, 2^-10 below."""
    a = np.abs(np.asarray(y, np.float64))
    _, ex = np.frexp(a)
    hs = np.ldexp(1.0, (ex - 1 - 4).astype(np.int64))
    return np.where(a < 2.0 ** -6, E4M3_ABS, hs)


def exact_deviation_bounds(qr, keys, vals, s_k, s_v, kmax, tail=1e-12, block=128):
    """Per query row and channel: the exact softmax o (float64) and three envelopes of
    |o_fp8 - o|, where o_fp8 is any result computed with the roundings of this module's
    definition -- query, keys, values and weights rounded to E4M3 with the scales above, scores
    summed from the rounded operands, one normaliser over the rounded weights -- whatever the
    order of the sums.  Returns ``(o, det, prob, rms)``, each ``[m, d]``.

    Derivation (per row; x_j = c <q, k_j> in log2 units, c = log2(e)/sqrt(d), p_j = 2^(8 + x_j - m)):

    * scores: Q8_i = s_q c q_i + e_i, K8_ji = s_k k_ji + f_ji with |e_i| <= E_i = h(s_q c q_i),
      |f_ji| <= F_ji = h(s_k k_ji) (h = ``e4m3_half_step``), so |x~_j - x_j| <= eta_j =
      sum_i E_i |k_ji| / s_q + |c q_i| F_ji / s_k + E_i F_ji / (s_q s_k), plus 2^-17 sum_i
      |Q8_i K8_ji| / (s_q s_k) for the float32 sums and 2^-18 (|m| + 8) for the exponent's
      float32 arithmetic;
    * weights: P8_j = e4m3(2^(8 + x~_j - m)) lies in [p_j r_j - 2^-10, p_j u_j + 2^-10] with
      u_j = 2^eta_j (1 + 2^-4), r_j = 2^-eta_j - 2^-4 2^eta_j, so |P8_j - p_j| <= p_j a_j + 2^-10
      with a_j = u_j - 1;
    * values: |V8_jc / s_v - v_jc| <= g_jc = h(s_v v_jc) / s_v;
    * since sum_j p_j (v_j - o) = 0,
      o_fp8 - o = [sum_j (P8_j - p_j)(v_j - o) + sum_j P8_j (V8_j / s_v - v_j)] / sum_j P8_j,
      with sum_j P8_j >= Z = sum_j (p_j r_j - 2^-10).

    ``det`` = [sum_j (p_j a_j + 2^-10)(|v_jc| + |o_c|) + sum_j (p_j u_j + 2^-10) g_jc] / Z holds
    for every input (worst case: every move aligned).  The offset m only scales p; the bound is
    largest for the largest offset the row can take (m = c |q| kmax when that is <= 4, else
    max x + max eta), which is the one used.

    ``rms`` is the predicted root-mean-square deviation when each rounding error is uniform over
    its half step and independent of the others (keys and values drawn independently), to first
    order in the score error: the score error has variance sum_i [(c q_i)^2 F_ji^2 / s_k^2 +
    k_ji^2 E_i^2 / s_q^2] / 3 (log2 units), each weight the relative variance
    (ln 2)^2 var(x~_j) + (h(p_j) / p_j)^2 / 3, each value the variance g_jc^2 / 3, combined as
    [sum_j p_j^2 var_w (v_jc - o_c)^2 + sum_j p_j^2 g_jc^2 / 3] / (sum_j p_j)^2.

    ``prob`` = sqrt(6 ln(2 / tail)) rms: under the same model the deviation is a sum of independent
    zero-mean terms, each confined to +-sqrt(3) times its standard deviation, so Hoeffding's
    inequality bounds it by ``prob`` except with probability ``tail``.
    """
    qr = np.asarray(qr, np.float64)
    keys = np.asarray(keys, np.float64)
    vals = np.asarray(vals, np.float64)
    m_rows, d = qr.shape
    c = math.log2(math.e) / math.sqrt(d)
    ln2 = math.log(2.0)
    ak = np.abs(keys)
    F = e4m3_half_step(s_k * keys)                     # [n, d], scaled units
    g = e4m3_half_step(s_v * vals) / s_v               # [n, d], value units
    V, V2 = vals, vals * vals
    lam = math.sqrt(6.0 * math.log(2.0 / tail))
    o_all, det_all, prob_all, rms_all = (np.zeros((m_rows, d)) for _ in range(4))
    for r0 in range(0, m_rows, block):
        q = qr[r0:r0 + block]
        cq = c * q
        s_q = np.array([pow2_scale(np.abs(row).max()) for row in cq])[:, None]
        E = e4m3_half_step(s_q * cq)                   # [b, d]
        acq = np.abs(cq)
        eta = (E @ ak.T) / s_q + (acq @ F.T) / s_k + (E @ F.T) / (s_q * s_k)
        eta += 2.0 ** -17 * (((s_q * acq + E) @ (s_k * ak + F).T) / (s_q * s_k))
        x = cq @ keys.T                                # exact scores, log2 units
        b = c * np.sqrt((q * q).sum(axis=1)) * kmax
        m = np.where(b <= OFFSET_BOUND_LIMIT, b, x.max(axis=1) + eta.max(axis=1))[:, None]
        eta += 2.0 ** -18 * (np.abs(m) + P_SHIFT)
        p = np.exp2(P_SHIFT + x - m)
        u = np.exp2(eta) * (1.0 + E4M3_REL)
        r = np.exp2(-eta) - E4M3_REL * np.exp2(eta)
        W1 = p * (u - 1.0) + E4M3_ABS
        W2 = p * u + E4M3_ABS
        Z = (p * r - E4M3_ABS).sum(axis=1, keepdims=True)
        assert np.all(Z > 0), "rounding envelope of the normaliser reaches zero"
        o = (p @ V) / p.sum(axis=1, keepdims=True)
        det = (W1 @ np.abs(V) + np.abs(o) * W1.sum(axis=1, keepdims=True) + W2 @ g) / Z
        var_x = ((acq * acq) @ (F * F).T / s_k ** 2 + (E * E) @ (keys * keys).T / s_q ** 2) / 3.0
        var_w = ln2 * ln2 * var_x + (e4m3_half_step(p) / p) ** 2 / 3.0
        P2w = p * p * var_w
        dev2w = P2w @ V2 - 2.0 * o * (P2w @ V) + o * o * P2w.sum(axis=1, keepdims=True)
        var = (np.maximum(dev2w, 0.0) + (p * p) @ (g * g) / 3.0) / p.sum(axis=1, keepdims=True) ** 2
        sl = slice(r0, r0 + len(q))
        o_all[sl], det_all[sl], prob_all[sl], rms_all[sl] = o, det, lam * np.sqrt(var), np.sqrt(var)
    return o_all, det_all, prob_all, rms_all


def softmax_branch_bounds(q, k, v, text_k, text_v, T, N, C, anchors, rows=None, audio_k=None, audio_v=None,
                          tail=1e-12):
    """``exact_deviation_bounds`` for the video rows of the softmax branch (every row, or the given
    token indices), with each head's scales; returns ``(o, det, prob, rms)`` shaped
    ``[len(rows), H, d]``."""
    if audio_k is not None:
        text_k = np.concatenate([text_k, audio_k], axis=0)
        text_v = np.concatenate([text_v, audio_v], axis=0)
    TN, H, d = q.shape
    rows = np.arange(TN) if rows is None else np.asarray(rows)
    res = [np.zeros((len(rows), H, d)) for _ in range(4)]
    frames_of_rows = rows // N
    for h in range(H):
        keys_all = np.concatenate([text_k[:, h], k[:, h]]).astype(np.float64)
        vals_all = np.concatenate([text_v[:, h], v[:, h]]).astype(np.float64)
        s_k, s_v, kmax = head_scales(keys_all, vals_all)
        n_g = text_k.shape[0]
        for t in np.unique(frames_of_rows):
            sel = np.nonzero(frames_of_rows == t)[0]
            kf = orc.key_frames(int(t), T, C, anchors)
            idx = np.concatenate([np.arange(n_g)] + [n_g + np.arange(f * N, (f + 1) * N) for f in kf])
            out = exact_deviation_bounds(q[rows[sel], h], keys_all[idx], vals_all[idx], s_k, s_v, kmax, tail)
            for a, b in zip(res, out):
                a[sel, h] = b
    return tuple(res)
