"""Pins of the CPU oracle: checks against facts the pages and mathematics fix.

Each pin takes the oracle module as an argument so that ``test_oracle_mutations`` can run the
same pin against a deliberately broken copy of the oracle and see it fail.  A pin raises
``AssertionError`` when the oracle disagrees with the fact it encodes.

[VDN] = "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models" (openvdn.github.io).
"""

from __future__ import annotations

import math
import os

import numpy as np
import scipy.linalg

from oracle import bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def frame_objective(s, s_bar, keys, vals, beta):
    """The frame objective of [VDN] "From independent token updates to one frame-wise solve":
    beta-weighted squared read errors plus the proximity term, each with a factor 1/2."""
    err = keys @ s.T - vals                      # row u: S k_u - v_u
    return 0.5 * float(np.sum(beta[:, None] * err * err)) + 0.5 * float(np.sum((s - s_bar) ** 2))


# --------------------------------------------------------------------------------------------
# VDA frame update pins
# --------------------------------------------------------------------------------------------

def pin_objective_minimum(orc, seed=0):
    """P1: the update minimises the frame objective: zero directional derivatives (central
    differences), no random perturbation decreases it, and a generic least-squares solve of the
    stacked system gives the same state."""
    rng = _rng(seed)
    U, d = 12, 8
    keys = _unit(rng.standard_normal((U, d)))
    vals = rng.standard_normal((U, d))
    beta = rng.random(U)
    s_bar = rng.standard_normal((d, d))
    a, b = orc.frame_stats(keys, vals, beta)
    s = orc.frame_update(s_bar, a, b)
    j0 = frame_objective(s, s_bar, keys, vals, beta)
    eps = 1e-5
    scale = 0.0
    for _ in range(8):
        delta = rng.standard_normal((d, d))
        g = (frame_objective(s + eps * delta, s_bar, keys, vals, beta)
             - frame_objective(s - eps * delta, s_bar, keys, vals, beta)) / (2 * eps)
        g_bar = (frame_objective(s_bar + eps * delta, s_bar, keys, vals, beta)
                 - frame_objective(s_bar - eps * delta, s_bar, keys, vals, beta)) / (2 * eps)
        scale = max(scale, abs(g_bar))
        assert abs(g) < 1e-6 * max(1.0, scale), f"directional derivative {g} not zero"
        assert frame_objective(s + 1e-3 * delta, s_bar, keys, vals, beta) > j0
    ref = bruteforce.lstsq_update(s_bar, keys, vals, beta)
    assert np.allclose(s, ref, rtol=1e-10, atol=1e-10), "closed form differs from least squares"


def pin_sherman_morrison(orc, seed=1):
    """P2: one token (U=1) reduces to the classical delta-rule step with the effective rate
    beta/(1 + beta ||k||^2) (Sherman-Morrison on I + beta k k^T); [VDN] "Video Delta Attention"."""
    rng = _rng(seed)
    d = 6
    for trial in range(4):
        k = rng.standard_normal(d) * (1.0 if trial % 2 else 1.7)   # also non-unit keys
        v = rng.standard_normal(d)
        beta = float(rng.random()) * 1.5
        s_bar = rng.standard_normal((d, d))
        a, b = orc.frame_stats(k[None], v[None], np.array([beta]))
        s = orc.frame_update(s_bar, a, b)
        c = beta / (1.0 + beta * float(k @ k))
        expect = s_bar - c * np.outer(s_bar @ k - v, k)
        assert np.allclose(s, expect, rtol=1e-12, atol=1e-12)


def pin_repeated_keys(orc, seed=2):
    """P3: every token of the frame uses the same unit key with a shared rate: the state's read on
    that key becomes (S_bar k + U beta v_mean) / (1 + U beta) -- repeated evidence accumulates."""
    rng = _rng(seed)
    U, d = 9, 7
    k = _unit(rng.standard_normal(d))
    vals = rng.standard_normal((U, d))
    beta = 0.35
    s_bar = rng.standard_normal((d, d))
    a, b = orc.frame_stats(np.tile(k, (U, 1)), vals, np.full(U, beta))
    s = orc.frame_update(s_bar, a, b)
    vmean = vals.mean(axis=0)
    assert np.allclose(s @ k, (s_bar @ k + U * beta * vmean) / (1 + U * beta), atol=1e-12)
    z = rng.standard_normal(d)
    z -= (z @ k) * k                                   # a direction no token addressed
    assert np.allclose(s @ z, s_bar @ z, atol=1e-12)


def pin_orthonormal_keys(orc, seed=3):
    """P4: orthonormal keys: each token's read becomes (S_bar k_u + beta v_u)/(1 + beta), with no
    penalty from the other tokens."""
    rng = _rng(seed)
    d, U = 8, 5
    qmat, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = qmat[:, :U].T
    vals = rng.standard_normal((U, d))
    beta = 0.6
    s_bar = rng.standard_normal((d, d))
    a, b = orc.frame_stats(keys, vals, np.full(U, beta))
    s = orc.frame_update(s_bar, a, b)
    for u in range(U):
        assert np.allclose(s @ keys[u], (s_bar @ keys[u] + beta * vals[u]) / (1 + beta), atol=1e-12)


def _transition_matrix(orc, a):
    """Matrix of the linear map S_bar -> S_bar (I + A)^-1 (the frame update with B = 0): its
    image of the identity."""
    d = a.shape[0]
    return orc.frame_update(np.eye(d), a, np.zeros((d, d)))


def pin_spectrum(orc, seed=4):
    """P5: the inherited-state transition has eigenvalues 1/(1 + lambda_i(A)) in (0, 1] and
    operator norm at most one, for any A >= 0 ([VDN] "Stability of the Inherited State")."""
    rng = _rng(seed)
    d, U = 6, 40
    keys = _unit(rng.standard_normal((1, d)) + 0.05 * rng.standard_normal((U, d)))  # crowded
    a, _ = orc.frame_stats(keys, np.zeros((U, d)), rng.random(U))
    lam = np.linalg.eigvalsh(a)
    assert lam.max() > 2.0                          # the additive rule would expand here
    m = _transition_matrix(orc, a)
    ev = np.sort(np.linalg.eigvals(m).real)
    assert np.allclose(ev, np.sort(1.0 / (1.0 + lam)), atol=1e-10)
    assert np.linalg.norm(m, 2) <= 1.0 + 1e-12


def pin_contraction(orc, seed=5):
    """P6: the frame update is non-expansive: ||f(X) - f(Y)||_F <= ||X - Y||_F."""
    rng = _rng(seed)
    d, U = 8, 64
    for crowd in (0.02, 1.0):
        keys = _unit(rng.standard_normal((1, d)) + crowd * rng.standard_normal((U, d)))
        vals = rng.standard_normal((U, d))
        a, b = orc.frame_stats(keys, vals, rng.random(U))
        for _ in range(5):
            x, y = rng.standard_normal((2, d, d)) * 3
            fx, fy = orc.frame_update(x, a, b), orc.frame_update(y, a, b)
            assert np.linalg.norm(fx - fy) <= np.linalg.norm(x - y) * (1 + 1e-12)


def pin_neumann(orc, seed=6):
    """P7: for a Gram matrix of spectral radius < 1 the update equals the Neumann-series form
    (S_bar + B)(I - A + A^2 - ...) ([VDN] "Correlation-Aware Frame Updates")."""
    rng = _rng(seed)
    d, U = 6, 4
    keys = _unit(rng.standard_normal((U, d)))
    vals = rng.standard_normal((U, d))
    beta = 0.2 * rng.random(U)
    s_bar = rng.standard_normal((d, d))
    a, b = orc.frame_stats(keys, vals, beta)
    assert max(abs(np.linalg.eigvalsh(a))) < 0.5
    series = np.zeros((d, d))
    term = np.eye(d)
    for _ in range(80):
        series += term
        term = -term @ a
    assert np.allclose(orc.frame_update(s_bar, a, b), (s_bar + b) @ series, atol=1e-12)


def pin_cho_solve(orc, seed=7):
    """P9: the update agrees with a Cholesky-based solve from another library routine."""
    rng = _rng(seed)
    d, U = 16, 100
    keys = _unit(rng.standard_normal((U, d)))
    vals = rng.standard_normal((U, d))
    beta = rng.random(U)
    s_bar = rng.standard_normal((d, d))
    a, b = orc.frame_stats(keys, vals, beta)
    fac = scipy.linalg.cho_factor(np.eye(d) + a)
    ref = scipy.linalg.cho_solve(fac, (s_bar + b).T).T
    assert np.allclose(orc.frame_update(s_bar, a, b), ref, rtol=1e-11, atol=1e-11)


# --------------------------------------------------------------------------------------------
# Frame-set and state-bookkeeping pins
# --------------------------------------------------------------------------------------------

def _parse_set(tok):
    tok = tok.strip()
    if tok == "-":
        return []
    out = []
    for part in tok.split(","):
        if "-" in part:
            lo, hi = part.split("-")
            out.extend(range(int(lo), int(hi) + 1))
        else:
            out.append(int(part))
    return out


def golden_frame_sets():
    rows = {}
    with open(os.path.join(GOLDEN, "frame_sets_T16_C2.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split("|")
            rows[int(parts[0])] = tuple(_parse_set(p) for p in parts[1:])
    return rows


def pin_golden_frame_sets(orc):
    """The hand-derived frame sets of the 16-frame, chunk-2 visualisation workload."""
    gold = golden_frame_sets()
    assert len(gold) == 16
    for t, (w, anc, f, r) in gold.items():
        got = orc.frame_sets(t, 16, 2, True)
        assert [list(x) for x in got] == [w, anc, f, r], (t, got)


def pin_partition(orc):
    """P10: W, Anc, F and R partition all frames for every query frame (the two linear regions
    are disjoint and exclude window and boundary frames, so no frame is counted twice)."""
    for anchors in (True, False):
        for C in (1, 2, 3, 5):
            for T in list(range(1, 26)) + [37, 59]:
                for t in range(T):
                    w, anc, f, r = orc.frame_sets(t, T, C, anchors)
                    allf = sorted(w + anc + f + r)
                    assert allf == list(range(T)), (T, C, anchors, t)
                    if anchors:
                        assert not ({0, T - 1} & set(f + r))
                        assert {0, T - 1} <= set(w + anc)


def pin_uniform_keys_visibility(orc):
    """With identical keys the softmax is uniform over the visible keys, so a frame-indicator value
    per key reveals each query's visible set; it must match the golden frame sets (text plus
    window plus anchors)."""
    T, N, C, H, d = 16, 3, 2, 1, 20
    n_text = 2
    q = np.zeros((T * N, H, d), np.float32)
    q[..., 0] = 1
    k = np.zeros_like(q)
    k[..., 0] = 1
    v = np.zeros_like(q)
    for f in range(T):
        v[f * N:(f + 1) * N, 0, f] = 1.0
    tk = np.zeros((n_text, H, d), np.float32)
    tk[..., 0] = 1
    tv = np.zeros((n_text, H, d), np.float32)
    tv[..., 16] = 1.0
    o = orc.softmax_branch(q, k, v, tk, tv, T, N, C, True)
    gold = golden_frame_sets()
    for t in range(T):
        w, anc, _, _ = gold[t]
        vis = sorted(w + anc)
        nkeys = n_text + N * len(vis)
        expect = np.zeros(d)
        expect[vis] = N / nkeys
        expect[16] = n_text / nkeys
        for n in range(N):
            assert np.allclose(o[t * N + n, 0], expect, atol=1e-6), t


def pin_beta_zero(orc, seed=8):
    """P8: with every video write strength zero the states keep the text state: o_l = 2 S0 q."""
    rng = _rng(seed)
    T, N, C, H, d, n_text = 11, 3, 2, 2, 5, 4
    q = rng.standard_normal((T * N, H, d))
    k = _unit(rng.standard_normal((T * N, H, d)))
    v = rng.standard_normal((T * N, H, d))
    tk = _unit(rng.standard_normal((n_text, H, d)))
    tv = rng.standard_normal((n_text, H, d))
    beta = rng.random((n_text + T * N, H))
    beta[n_text:] = 0.0
    o_l = orc.linear_branch(q, k, v, beta, tk, tv, T, N, C, True)
    for h in range(H):
        s0 = bruteforce.lstsq_update(np.zeros((d, d)), tk[:, h], tv[:, h], 0.5 * beta[:n_text, h])
        assert np.allclose(o_l[:, h], q[:, h] @ (2 * s0).T, atol=1e-10)


def pin_text_once(orc, seed=9):
    """P11: text enters only through the initial states, each at half strength, so that in the
    small-beta limit the two readouts together carry the text write B_text exactly once."""
    rng = _rng(seed)
    n_text, d = 6, 5
    tk = _unit(rng.standard_normal((n_text, d)))
    tv = rng.standard_normal((n_text, d))
    tb = rng.random(n_text)
    b_text = (tv * tb[:, None]).T @ tk
    for eps in (1e-4, 1e-6):
        s0 = orc.text_state(tk, tv, eps * tb)
        assert np.allclose((s0 + s0) / eps, b_text, atol=10 * eps * np.abs(b_text).max() * n_text)
    # no text -> zero initial state
    assert np.allclose(orc.text_state(tk[:0], tv[:0], tb[:0]), 0)


def pin_boundary_text_only(orc, seed=10):
    """Boundary query frames see every frame through the softmax, so their linear readout holds
    only the text: o_l = 2 S0 q for frames 0 and T-1."""
    rng = _rng(seed)
    T, N, C, H, d, n_text = 9, 2, 2, 1, 4, 3
    q = rng.standard_normal((T * N, H, d))
    k = _unit(rng.standard_normal((T * N, H, d)))
    v = rng.standard_normal((T * N, H, d))
    tk = _unit(rng.standard_normal((n_text, H, d)))
    tv = rng.standard_normal((n_text, H, d))
    beta = rng.random((n_text + T * N, H))
    o_l = orc.linear_branch(q, k, v, beta, tk, tv, T, N, C, True)
    s0 = bruteforce.lstsq_update(np.zeros((d, d)), tk[:, 0], tv[:, 0], 0.5 * beta[:n_text, 0])
    for t in (0, T - 1):
        for n in range(N):
            i = t * N + n
            assert np.allclose(o_l[i, 0], 2 * s0 @ q[i, 0], atol=1e-10)


# --------------------------------------------------------------------------------------------
# Merge pins ([VDN] "Gating the Softmax and Linear Branch Outputs")
# --------------------------------------------------------------------------------------------

def pin_gate_closed_forms(orc, seed=11):
    """P14: zero gate weights give gates of 1/2; identity projections then give
    out = o_s/2 + RMSNorm(o_l)/2; a single non-zero gate weight w at [i][j] gates output channel j
    by sigmoid(w q_i) (weights are [in][out]); a single non-zero projection weight moves channel i
    to channel j."""
    rng = _rng(seed)
    M, d = 7, 6
    q = rng.standard_normal((M, d))
    o_s = rng.standard_normal((M, d))
    o_l = rng.standard_normal((M, d)) * 3
    gw = np.zeros((2, d, d))
    pw = np.stack([np.eye(d), np.eye(d)])
    rms = np.sqrt(np.mean(o_l ** 2, axis=-1, keepdims=True) + 1e-6)
    assert np.allclose(orc.merge(q, o_s, o_l, gw, pw), 0.5 * o_s + 0.5 * o_l / rms, atol=1e-12)
    # orientation of the gate weights: softmax gate only, one entry
    gw1 = np.zeros((2, d, d))
    gw1[0, 1, 4] = 2.5
    pw_s = np.stack([np.eye(d), np.zeros((d, d))])
    out = orc.merge(q, o_s, o_l, gw1, pw_s)
    g = np.full((M, d), 0.5)
    g[:, 4] = 1 / (1 + np.exp(-2.5 * q[:, 1]))
    assert np.allclose(out, g * o_s, atol=1e-12)
    # linear gate, one entry; projection moves channel 2 to channel 5
    gw2 = np.zeros((2, d, d))
    gw2[1, 3, 2] = -1.5
    pw2 = np.zeros((2, d, d))
    pw2[1, 2, 5] = 2.0
    out = orc.merge(q, o_s, o_l, gw2, pw2)
    expect = np.zeros((M, d))
    expect[:, 5] = 2.0 * (1 / (1 + np.exp(1.5 * q[:, 3]))) * (o_l / rms)[:, 2]
    assert np.allclose(out, expect, atol=1e-12)
    # RMSNorm: scale invariance of the linear branch
    a = orc.merge(q, o_s, o_l, gw2, pw2)
    b = orc.merge(q, o_s, 1e3 * o_l, gw2, pw2)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-9)


# --------------------------------------------------------------------------------------------
# Decay gate pins ([VDN] "Video Delta Attention: A Frame-Wise Solution": the inherited state is
# decayed channel-wise, S_bar = S Diag(alpha); "Stability of the Inherited State": the decayed
# transition Diag(alpha)(I + A)^-1 has operator norm at most one)
# --------------------------------------------------------------------------------------------

def _frame_sums(k, v, beta, n_text, N, f, h):
    """A_f and B_f by explicit sums over the frame's tokens (independent of the oracle)."""
    d = k.shape[-1]
    a = np.zeros((d, d))
    b = np.zeros((d, d))
    for u in range(f * N, (f + 1) * N):
        ku = np.asarray(k[u, h], np.float64)
        w = float(beta[n_text + u, h])
        a += w * np.outer(ku, ku)
        b += w * np.outer(np.asarray(v[u, h], np.float64), ku)
    return a, b


def pin_decay_one(orc, seed=13):
    """P15: alpha = 1 everywhere is exactly the undecayed layer."""
    T, N, C, n_text, H, d = 9, 3, 2, 2, 2, 4
    inp = tiny_inputs(T, N, n_text, H, d, seed)
    ref = orc.chunk_states(inp, T, N, C, True)
    inp["alpha"] = np.ones((T, H, d), np.float32)
    assert np.array_equal(orc.chunk_states(inp, T, N, C, True), ref)


def pin_decay_zero(orc, seed=14):
    """P16: alpha = 0 forgets everything before the frame being written: every scanned state is
    that frame's own solve from zero, B_f (I + A_f)^-1 (computed here with an explicit inverse)."""
    T, N, C, n_text, H, d = 8, 3, 1, 2, 1, 4
    inp = tiny_inputs(T, N, n_text, H, d, seed)
    inp["alpha"] = np.zeros((T, H, d), np.float32)
    st = orc.chunk_states(inp, T, N, C, False)
    for t in range(T):
        # anchors off, C = 1: forward region = frames <= t-2, reverse region = frames >= t+2
        want = np.zeros((d, d))
        for f in ([t - 2] if t >= 2 else []) + ([t + 2] if t + 2 < T else []):
            a, b = _frame_sums(inp["k"], inp["v"], inp["beta"], n_text, N, f, 0)
            want += b @ np.linalg.inv(np.eye(d) + a)
        if t < 2 or t + 2 >= T:                          # an empty region keeps the text state
            a, b = _frame_sums(inp["text_k"], inp["text_v"], np.concatenate(
                [0.5 * inp["beta"][:n_text], inp["beta"][n_text:]]), 0, n_text, 0, 0)
            s0 = b @ np.linalg.inv(np.eye(d) + a)
            want += s0 * ((t < 2) + (t + 2 >= T))
        assert np.allclose(st[t, 0], want, rtol=1e-9, atol=1e-10), t


def pin_decay_columns(orc, seed=15):
    """P17: writing frame f solves S_f (I + A_f) = S_prev Diag(alpha_f) + B_f, with the decay on
    the key channels (columns) of the inherited state and alpha of the frame being written, in
    both scan directions (checked on consecutive prefix states, anchors off, one frame per chunk)."""
    rng = _rng(seed)
    T, N, C, n_text, H, d = 9, 4, 1, 1, 1, 5
    inp = tiny_inputs(T, N, n_text, H, d, seed)
    inp["alpha"] = rng.random((T, H, d)).astype(np.float32)
    _, per_frame = orc.head_states(inp["k"], inp["v"], inp["beta"], inp["text_k"], inp["text_v"], 0,
                                   T, N, C, False, alpha=inp["alpha"])
    fwd = [per_frame[t][0] for t in range(2, T)]        # after frames 0..t-2
    rev = [per_frame[t][1] for t in range(T - 3, -1, -1)]   # after frames T-1 .. t+2
    for i in range(1, len(fwd)):
        f = i                                            # fwd[i] has written frames 0..i
        a, b = _frame_sums(inp["k"], inp["v"], inp["beta"], n_text, N, f, 0)
        lhs = fwd[i] @ (np.eye(d) + a) - b
        assert np.allclose(lhs, fwd[i - 1] * inp["alpha"][f, 0].astype(np.float64)[None, :],
                           rtol=1e-8, atol=1e-10), ("forward", f)
    for i in range(1, len(rev)):
        f = T - 1 - i                                    # rev[i] has written frames T-1 .. f
        a, b = _frame_sums(inp["k"], inp["v"], inp["beta"], n_text, N, f, 0)
        lhs = rev[i] @ (np.eye(d) + a) - b
        assert np.allclose(lhs, rev[i - 1] * inp["alpha"][f, 0].astype(np.float64)[None, :],
                           rtol=1e-8, atol=1e-10), ("reverse", f)


def pin_decay_nonexpansive(orc, seed=16):
    """P18: with 0 <= alpha <= 1 the decayed update is non-expansive in the inherited state:
    ||f(X) - f(Y)||_F <= ||X - Y||_F for f(S) = update(decay(S))."""
    rng = _rng(seed)
    d, U = 8, 40
    for trial in range(20):
        k = _unit(rng.standard_normal((U, d)))
        if trial % 2:
            k = _unit(k[:1] + 0.05 * rng.standard_normal((U, d)))   # crowded keys
        a, b = orc.frame_stats(k, rng.standard_normal((U, d)), rng.random(U))
        alpha = rng.random(d)
        x, y = rng.standard_normal((d, d)), rng.standard_normal((d, d))
        fx = orc.frame_update(orc.decay(x, alpha), a, b)
        fy = orc.frame_update(orc.decay(y, alpha), a, b)
        assert np.linalg.norm(fx - fy) <= np.linalg.norm(x - y) * (1 + 1e-12)


BRUTE_DECAY_CASES = [
    # T, N, C, n_text, H, d, anchors
    (7, 3, 2, 2, 2, 4, True),
    (9, 2, 1, 1, 1, 4, False),
    (10, 3, 3, 2, 1, 6, True),
]


def pin_bruteforce_decay(orc, seed=17):
    """P19: with a decay gate, the structured oracle equals the brute-force oracle (least-squares
    updates whose proximity target is the inherited state times the diagonal of alpha)."""
    for ci, (T, N, C, n_text, H, d, anchors) in enumerate(BRUTE_DECAY_CASES):
        inp = tiny_inputs(T, N, n_text, H, d, seed + ci)
        inp["alpha"] = _rng(seed + 100 + ci).random((T, H, d)).astype(np.float32)
        out_s, mids = orc.vdn_forward(inp, T, N, C, anchors, with_intermediates=True)
        out_b, _, ol_b = bruteforce.layer_dense(inp, T, N, C, anchors)
        assert np.allclose(mids["o_l"], ol_b, rtol=1e-9, atol=1e-9), ("o_l", ci)
        assert np.allclose(out_s, out_b, rtol=1e-5, atol=1e-5), ("out", ci)


# --------------------------------------------------------------------------------------------
# Whole-layer pins
# --------------------------------------------------------------------------------------------

def tiny_inputs(T, N, n_text, H, d, seed, dtype=np.float32):
    rng = _rng(seed)
    return dict(
        q=_unit(rng.standard_normal((T * N, H, d))).astype(dtype),
        k=_unit(rng.standard_normal((T * N, H, d))).astype(dtype),
        v=rng.standard_normal((T * N, H, d)).astype(dtype),
        text_k=_unit(rng.standard_normal((n_text, H, d))).astype(dtype),
        text_v=rng.standard_normal((n_text, H, d)).astype(dtype),
        beta=rng.random((n_text + T * N, H)).astype(dtype),
        gate_w=(rng.standard_normal((2, d, d)) / math.sqrt(d)).astype(dtype),
        proj_w=(rng.standard_normal((2, d, d)) / math.sqrt(d)).astype(dtype),
    )


BRUTE_CASES = [
    # T, N, C, n_text, H, d, anchors
    (16, 2, 2, 1, 1, 8, True),
    (7, 3, 2, 2, 2, 4, True),
    (7, 3, 2, 2, 1, 4, False),
    (1, 4, 5, 3, 1, 4, True),
    (2, 3, 1, 1, 1, 4, True),
    (3, 2, 5, 2, 1, 4, False),
    (11, 2, 3, 0, 1, 6, True),
    (13, 2, 1, 2, 2, 5, True),
    (10, 3, 5, 4, 1, 8, True),
]


def pin_bruteforce(orc, cases=BRUTE_CASES, seed=12):
    """P12: the structured oracle equals the brute-force oracle (dense mask, least-squares frame
    updates, per-frame rebuilt states) on tiny shapes, including T not divisible by C, T <= 3C,
    T = 1 and 2, no text, and anchors off."""
    for ci, (T, N, C, n_text, H, d, anchors) in enumerate(cases):
        inp = tiny_inputs(T, N, n_text, H, d, seed + ci)
        out_s, mids = orc.vdn_forward(inp, T, N, C, anchors, with_intermediates=True)
        out_b, os_b, ol_b = bruteforce.layer_dense(inp, T, N, C, anchors)
        assert np.allclose(mids["o_s"], os_b, rtol=1e-5, atol=1e-6), ("o_s", ci)
        assert np.allclose(mids["o_l"], ol_b, rtol=1e-9, atol=1e-9), ("o_l", ci)
        assert np.allclose(out_s, out_b, rtol=1e-5, atol=1e-5), ("out", ci)


# --------------------------------------------------------------------------------------------
# Text and audio tokens in the joint sequence.  [GLN] = "Video DeltaNet speeds MiniMax H3 video
# generation 14.5x" (glonce.com): the hybrid attention covers only video-to-video interactions;
# any interaction with a text or audio token keeps the full softmax attention.
# --------------------------------------------------------------------------------------------

def joint_inputs(T, N, n_text, n_audio, H, d, seed):
    """tiny_inputs plus audio tokens and the text/audio query rows."""
    rng = _rng(seed + 1000)
    inp = tiny_inputs(T, N, n_text, H, d, seed)
    inp["audio_k"] = _unit(rng.standard_normal((n_audio, H, d))).astype(np.float32)
    inp["audio_v"] = rng.standard_normal((n_audio, H, d)).astype(np.float32)
    inp["ctx_q"] = _unit(rng.standard_normal((n_text + n_audio, H, d))).astype(np.float32)
    return inp


def golden_attention_map():
    rows = {}
    with open(os.path.join(GOLDEN, "attention_map_T16_C2_text1_audio1.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            label, entries = line.split("|")
            rows[label.strip()] = entries.split()
    return rows


def pin_golden_attention_map(orc):
    """The hand-derived branch map of the visualisation workload (1 text, 1 audio token, 16 frames,
    chunks of 2).  Softmax visibility is read off the oracle's outputs with identical keys and a
    one-hot value per key (a uniform softmax over the visible keys), for the video rows and for
    the text/audio rows; 'B' and 'L' entries are read off the linear branch: changing a frame's
    or the text's values moves o_l exactly when the map says the key reaches the linear memory."""
    gold = golden_attention_map()
    T, N, C, H, d = 16, 1, 2, 1, 18
    labels = ["text", "audio"] + [f"f{t}" for t in range(T)]
    assert list(gold) == labels
    # column j of the sequence [text, audio, f0..f15] carries value e_j
    e = np.eye(d, dtype=np.float32)
    q = np.zeros((T, H, d), np.float32)
    q[..., 0] = 1
    inp = dict(q=q, k=np.array(q), v=e[2:][:, None, :].copy(),
               text_k=np.array(q[:1]), text_v=e[0][None, None, :].copy(),
               audio_k=np.array(q[:1]), audio_v=e[1][None, None, :].copy(),
               ctx_q=np.array(q[:2]))
    o_s = orc.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], T, N, C, True,
                             audio_k=inp["audio_k"], audio_v=inp["audio_v"])
    o_c = orc.context_rows(inp, T, N)
    seen = np.concatenate([o_c[:, 0], o_s[:, 0]]) > 1e-6          # [query][key]
    soft = np.array([[x in ("S", "B") for x in gold[lab]] for lab in labels])
    assert (seen == soft).all(), np.argwhere(seen != soft)
    assert (bruteforce.joint_mask(1, 1, T, N, C, True) == soft).all()
    # linear memory: perturb one key's value and see which video rows' o_l move
    rng = _rng(30)
    base = tiny_inputs(T, N, 1, H, 6, 31)
    base["audio_k"] = _unit(rng.standard_normal((1, H, 6))).astype(np.float32)
    base["audio_v"] = rng.standard_normal((1, H, 6)).astype(np.float32)
    ref = orc.vdn_forward(base, T, N, C, True, with_intermediates=True)[1]["o_l"]
    for j, lab in enumerate(labels):
        pert = {key: np.array(val) for key, val in base.items()}
        if j == 0:
            pert["text_v"] += 1.0
        elif j == 1:
            pert["audio_v"] += 1.0
        else:
            pert["v"][j - 2] += 1.0
        o_l = orc.vdn_forward(pert, T, N, C, True, with_intermediates=True)[1]["o_l"]
        moved = np.abs(o_l - ref).max(axis=(1, 2)) > 1e-9
        expect = np.array([gold[f"f{t}"][j] in ("B", "L") for t in range(T)])
        assert (moved == expect).all(), (lab, np.nonzero(moved != expect))


def pin_context_rows_sdpa(orc, seed=32):
    """Text and audio query rows are plain softmax attention over the whole sequence: torch's CPU
    scaled_dot_product_attention in float64 on the concatenated keys and values."""
    import torch
    for ci, (T, N, n_text, n_audio, H, d) in enumerate([(5, 3, 2, 3, 2, 8), (3, 4, 0, 2, 1, 16),
                                                         (4, 2, 3, 0, 2, 4)]):
        inp = joint_inputs(T, N, n_text, n_audio, H, d, seed + ci)
        got = orc.context_rows(inp, T, N)
        assert got.shape == (n_text + n_audio, H, d)
        for h in range(H):
            kk = np.concatenate([inp["text_k"][:, h], inp["audio_k"][:, h], inp["k"][:, h]]).astype(np.float64)
            vv = np.concatenate([inp["text_v"][:, h], inp["audio_v"][:, h], inp["v"][:, h]]).astype(np.float64)
            qq = inp["ctx_q"][:, h].astype(np.float64)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qq)[None, None], torch.from_numpy(kk)[None, None],
                torch.from_numpy(vv)[None, None])[0, 0].numpy()
            assert np.allclose(got[:, h], ref, atol=2e-6), (ci, h)


def pin_audio_softmax_only(orc, seed=33):
    """Audio tokens are softmax keys only: changing them moves o_s of every video row and leaves
    o_l bit for bit unchanged (the linear memory is initialised from the text alone)."""
    T, N, C, n_text, n_audio, H, d = 9, 2, 2, 2, 3, 2, 6
    inp = joint_inputs(T, N, n_text, n_audio, H, d, seed)
    _, a = orc.vdn_forward(inp, T, N, C, True, with_intermediates=True)
    pert = dict(inp)
    pert["audio_k"] = _unit(inp["audio_k"] + 0.5).astype(np.float32)
    pert["audio_v"] = inp["audio_v"] + 1.0
    _, b = orc.vdn_forward(pert, T, N, C, True, with_intermediates=True)
    assert np.array_equal(a["o_l"], b["o_l"])
    assert (np.abs(a["o_s"] - b["o_s"]).max(axis=(1, 2)) > 1e-4).all()


JOINT_CASES = [
    # T, N, C, n_text, n_audio, H, d, anchors
    (16, 1, 2, 1, 1, 1, 8, True),
    (7, 3, 2, 2, 3, 2, 4, True),
    (6, 2, 1, 0, 2, 1, 4, False),
    (1, 4, 5, 3, 1, 1, 4, True),
    (10, 2, 3, 2, 0, 2, 6, True),
]


def pin_bruteforce_joint(orc, seed=34):
    """The structured oracle with audio keys and text/audio query rows equals the brute-force
    oracle, whose single dense mask over [text, audio, video] is built entry by entry from the
    token kinds."""
    for ci, (T, N, C, n_text, n_audio, H, d, anchors) in enumerate(JOINT_CASES):
        inp = joint_inputs(T, N, n_text, n_audio, H, d, seed + ci)
        if n_audio == 0:
            inp.pop("audio_k")
            inp.pop("audio_v")
        out_s, mids = orc.vdn_forward(inp, T, N, C, anchors, with_intermediates=True)
        out_b, os_b, ol_b = bruteforce.layer_dense(inp, T, N, C, anchors)
        assert np.allclose(mids["o_s"], os_b, rtol=1e-5, atol=1e-6), ("o_s", ci)
        assert np.allclose(mids["o_l"], ol_b, rtol=1e-9, atol=1e-9), ("o_l", ci)
        assert np.allclose(out_s, out_b, rtol=1e-5, atol=1e-5), ("out", ci)
        ctx = orc.context_rows(inp, T, N)
        assert np.allclose(ctx, bruteforce.context_dense(inp, T, N, C, anchors), rtol=1e-5, atol=1e-6), ("ctx", ci)


# --------------------------------------------------------------------------------------------
# Backward pass.  The reverse-mode oracle (oracle/vdn_backward.py) against (a) torch autograd on an
# independent dense float64 forward written here from the same rules, and (b) central finite
# differences of the numpy forward oracle (softmax in float64) along random directions.
# --------------------------------------------------------------------------------------------

BWD_INPUTS = ("q", "k", "v", "beta", "text_k", "text_v", "gate_w", "proj_w")


def torch_layer_forward(x, T, N, C, anchors, eps=1e-6):
    """Dense float64 forward in torch: one mask over [text, video] keys built from the frame rule,
    every query frame's states rebuilt from the text state by repeated solves."""
    import torch
    q, k, v, beta = x["q"], x["k"], x["v"], x["beta"]
    tk, tv = x["text_k"], x["text_v"]
    alpha = x.get("alpha")
    TN, H, d = q.shape
    n_text = tk.shape[0]
    # global softmax keys: the text and, when present, the audio tokens (never in the linear memory)
    gk = torch.cat([tk, x["audio_k"]]) if x.get("audio_k") is not None else tk
    gv = torch.cat([tv, x["audio_v"]]) if x.get("audio_v") is not None else tv
    bset = (0, T - 1) if anchors else ()
    tau = 1.0 / math.sqrt(d)
    mask = torch.tensor(bruteforce.dense_mask(T, N, gk.shape[0], C, anchors))
    eye = torch.eye(d, dtype=torch.float64)
    outs = []
    for h in range(H):
        keys = torch.cat([gk[:, h], k[:, h]])
        vals = torch.cat([gv[:, h], v[:, h]])
        s = (q[:, h] @ keys.T) * tau
        s = s.masked_fill(~mask, float("-inf"))
        o_s = torch.softmax(s, dim=1) @ vals

        def step(z, kf, vf, bf, a=None):
            zbar = z if a is None else z * a[None, :]
            amat = (kf * bf[:, None]).T @ kf
            bmat = (vf * bf[:, None]).T @ kf
            return torch.linalg.solve((eye + amat).T, (zbar + bmat).T).T
        s0 = step(torch.zeros(d, d, dtype=torch.float64), tk[:, h], tv[:, h], 0.5 * beta[:n_text, h])
        rows = []
        for t in range(T):
            c = t // C
            zf, zr = s0, s0
            if t not in bset:
                for f in range(T):
                    if f not in bset and f // C < c - 1:
                        sl = slice(f * N, (f + 1) * N)
                        zf = step(zf, k[sl, h], v[sl, h], beta[n_text + f * N:n_text + (f + 1) * N, h],
                                  None if alpha is None else alpha[f, h])
                for f in range(T - 1, -1, -1):
                    if f not in bset and f // C > c + 1:
                        sl = slice(f * N, (f + 1) * N)
                        zr = step(zr, k[sl, h], v[sl, h], beta[n_text + f * N:n_text + (f + 1) * N, h],
                                  None if alpha is None else alpha[f, h])
            rows.append(q[t * N:(t + 1) * N, h] @ (zf + zr).T)
        o_l = torch.cat(rows)
        gs = torch.sigmoid(q[:, h] @ x["gate_w"][0])
        gl = torch.sigmoid(q[:, h] @ x["gate_w"][1])
        r = o_l / torch.sqrt(torch.mean(o_l * o_l, dim=1, keepdim=True) + eps)
        outs.append((gs * o_s) @ x["proj_w"][0] + (gl * r) @ x["proj_w"][1])
    return torch.stack(outs, dim=1)


def torch_context_rows(x):
    """Dense float64 text and audio query rows in torch: one softmax over [text, audio, video]."""
    import torch
    parts_k = [x["text_k"]] + ([x["audio_k"]] if x.get("audio_k") is not None else []) + [x["k"]]
    parts_v = [x["text_v"]] + ([x["audio_v"]] if x.get("audio_v") is not None else []) + [x["v"]]
    keys, vals = torch.cat(parts_k), torch.cat(parts_v)
    d = keys.shape[-1]
    outs = []
    for h in range(keys.shape[1]):
        p = torch.softmax((x["ctx_q"][:, h] @ keys[:, h].T) / math.sqrt(d), dim=1)
        outs.append(p @ vals[:, h])
    return torch.stack(outs, dim=1)


BWD_CASES = [
    # T, N, C, n_text, H, d, anchors, decay
    (7, 3, 2, 2, 2, 4, True, False),
    (6, 2, 1, 3, 1, 5, False, False),
    (9, 2, 2, 1, 1, 4, True, True),
    (5, 3, 5, 0, 1, 4, True, False),
]


def _bwd_inputs(T, N, n_text, H, d, decay, seed):
    inp = {key: val.astype(np.float64) for key, val in tiny_inputs(T, N, n_text, H, d, seed).items()}
    if decay:
        inp["alpha"] = 0.5 + 0.5 * _rng(seed + 7).random((T, H, d))
    return inp


def pin_backward_autograd(bwd, seed=40):
    """The reverse-mode oracle equals torch autograd through an independent dense forward."""
    import torch
    for ci, (T, N, C, n_text, H, d, anchors, decay) in enumerate(BWD_CASES):
        inp = _bwd_inputs(T, N, n_text, H, d, decay, seed + ci)
        dout = _rng(seed + 100 + ci).standard_normal((T * N, H, d))
        x = {key: torch.tensor(val, requires_grad=True) for key, val in inp.items()}
        out = torch_layer_forward(x, T, N, C, anchors)
        loss = torch.sum(out * torch.tensor(dout))
        names = [key for key in x if key != "alpha" or decay]
        auto = dict(zip(names, torch.autograd.grad(loss, [x[n] for n in names])))
        got = bwd.vdn_backward(inp, dout, T, N, C, anchors)
        for name in names:
            ref = auto[name].numpy()
            scale = max(1.0, float(np.abs(ref).max())) if ref.size else 1.0
            assert np.allclose(got[name], ref, rtol=1e-8, atol=1e-9 * scale), (ci, name, np.abs(got[name] - ref).max())


def pin_backward_finite_differences(bwd, seed=50):
    """Directional derivatives of <dout, out> by central differences of the numpy forward oracle
    (float64 softmax) equal <gradient, direction> for every input, one random direction each."""
    from oracle import vdn_oracle as orc
    for ci, (T, N, C, n_text, H, d, anchors, decay) in enumerate(BWD_CASES[:3]):
        inp = _bwd_inputs(T, N, n_text, H, d, decay, seed + ci)
        dout = _rng(seed + 200 + ci).standard_normal((T * N, H, d))
        got = bwd.vdn_backward(inp, dout, T, N, C, anchors)
        loss = lambda x: float(np.sum(dout * orc.vdn_forward(x, T, N, C, anchors, softmax_dtype=np.float64)))
        rng = _rng(seed + 300 + ci)
        for name in got:
            delta = rng.standard_normal(inp[name].shape)
            eps = 1e-5
            plus = dict(inp)
            minus = dict(inp)
            plus[name] = inp[name] + eps * delta
            minus[name] = inp[name] - eps * delta
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            an = float(np.sum(got[name] * delta))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (ci, name, fd, an)


JOINT_BWD_CASES = [
    # T, N, C, n_text, n_audio, H, d, anchors, decay
    (7, 3, 2, 2, 3, 2, 4, True, False),
    (6, 2, 1, 0, 2, 1, 5, False, False),
    (9, 2, 2, 1, 1, 1, 4, True, True),
    (5, 3, 5, 2, 0, 1, 4, True, False),
]


def _joint_bwd_inputs(T, N, n_text, n_audio, H, d, decay, seed):
    inp = {key: val.astype(np.float64) for key, val in joint_inputs(T, N, n_text, n_audio, H, d, seed).items()}
    if n_audio == 0:
        del inp["audio_k"], inp["audio_v"]
    if decay:
        inp["alpha"] = 0.5 + 0.5 * _rng(seed + 7).random((T, H, d))
    return inp


def pin_joint_backward_autograd(bwd, seed=70):
    """With audio keys and the text/audio query rows, the reverse-mode oracle equals torch autograd
    of <dout, out> + <dctx_out, ctx_out> through the dense joint forward."""
    import torch
    for ci, (T, N, C, n_text, n_audio, H, d, anchors, decay) in enumerate(JOINT_BWD_CASES):
        inp = _joint_bwd_inputs(T, N, n_text, n_audio, H, d, decay, seed + ci)
        dout = _rng(seed + 100 + ci).standard_normal((T * N, H, d))
        dctx = _rng(seed + 150 + ci).standard_normal((n_text + n_audio, H, d))
        x = {key: torch.tensor(val, requires_grad=True) for key, val in inp.items()}
        loss = torch.sum(torch_layer_forward(x, T, N, C, anchors) * torch.tensor(dout)) + \
            torch.sum(torch_context_rows(x) * torch.tensor(dctx))
        names = list(x)
        auto = dict(zip(names, torch.autograd.grad(loss, [x[n] for n in names])))
        got = bwd.vdn_backward(inp, dout, T, N, C, anchors, dctx_out=dctx)
        assert set(got) == set(names), (ci, sorted(got), sorted(names))
        for name in names:
            ref = auto[name].numpy()
            scale = max(1.0, float(np.abs(ref).max())) if ref.size else 1.0
            assert np.allclose(got[name], ref, rtol=1e-8, atol=1e-9 * scale), (ci, name, np.abs(got[name] - ref).max())


def pin_joint_backward_finite_differences(bwd, seed=80):
    """Directional derivatives of <dout, out> + <dctx_out, ctx_out> by central differences of the
    numpy forward oracle (float64 softmax, float64 context rows) equal <gradient, direction> for
    every input of a joint sequence, one random direction each."""
    from oracle import vdn_oracle as orc
    for ci, (T, N, C, n_text, n_audio, H, d, anchors, decay) in enumerate(JOINT_BWD_CASES[:2]):
        inp = _joint_bwd_inputs(T, N, n_text, n_audio, H, d, decay, seed + ci)
        dout = _rng(seed + 200 + ci).standard_normal((T * N, H, d))
        dctx = _rng(seed + 250 + ci).standard_normal((n_text + n_audio, H, d))
        got = bwd.vdn_backward(inp, dout, T, N, C, anchors, dctx_out=dctx)

        def loss(x):
            out = orc.vdn_forward(x, T, N, C, anchors, softmax_dtype=np.float64)
            return float(np.sum(dout * out) + np.sum(dctx * orc.context_rows(x, T, N, dtype=np.float64)))
        rng = _rng(seed + 300 + ci)
        for name in got:
            delta = rng.standard_normal(inp[name].shape)
            eps = 1e-5
            plus = dict(inp)
            minus = dict(inp)
            plus[name] = inp[name] + eps * delta
            minus[name] = inp[name] - eps * delta
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            an = float(np.sum(got[name] * delta))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (ci, name, fd, an)
