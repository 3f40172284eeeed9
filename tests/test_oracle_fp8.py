"""Pins of the FP8 softmax oracle (``oracle/fp8_softmax.py``), all on the CPU.

* the E4M3 rounding against torch's float8_e4m3fn conversion (a library routine) on random values
  over the whole range, on every representable value and on every midpoint between neighbours
  (ties to even);
* two hand-derived cases of the definition (one on the bound offset, one on the row-maximum offset
  with a weight in the subnormal range), whose rounded weights are worked out in the comments;
* uniform attention: identical keys give every visible key the same weight, so a frame-indicator
  value reveals each query's key set (text, window, anchors), exactly;
* closeness to the exact softmax within the error the rounding allows, and the envelopes of that
  error derived from the rounding steps alone (worst case, probabilistic, predicted RMS);
* the per-row allowance for scores that land near an E4M3 midpoint, by a hand-worked row and by
  brute-force perturbation of the scores;
* planted mistakes, each caught by one of the pins above.
"""

import importlib.util
import math
import os

import numpy as np
import pytest
import torch

import pins

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fp8_softmax.py")


def fresh():
    spec = importlib.util.spec_from_file_location("fp8_softmax_mutant", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).double().numpy()


def pin_e4m3_library(f8, seed=0):
    """Rounding agrees with torch's conversion wherever the result is finite (|x| < 464)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-5, 2.6, 200000)).astype(np.float32)
    x = x[np.abs(x) < 464]
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    vals = np.unique(codes[np.isfinite(codes)])
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)   # exact in float32
    for arr in (x, vals.astype(np.float32), mids, -mids):
        assert np.array_equal(f8.e4m3(arr), _torch_e4m3(arr))


def _two_key_case():
    d = 16
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    keys = np.zeros((2, d))
    keys[0, 0] = 0.5
    keys[1, 0] = -1.0
    vals = np.zeros((2, d))
    vals[0, 0] = 1.0
    vals[1, 1] = 1.0
    return q, keys, vals


def pin_hand_bound_offset(f8):
    """d = 16, c = log2(e)/4 = 0.36067; q = e1, k1 = e1/2, k2 = -e1, v1 = e1, v2 = e2.
    Scales: s_k = 2^(8-1) = 128 (max |k| = 1 = 0.5 * 2^1), so K8 = (64, -128) exactly, s_v = 128;
    c q = 0.36067 e1 = 0.7213 * 2^-1, so s_q = 2^9 and Q8 = e4m3(184.67) = 192 (step 16 in
    [128, 256)).  x = 192 (64, -128) / (512 * 128) = (0.1875, -0.375).  kmax = 1, bound b = c <= 4 is
    the offset.  Weights: 2^(8 + 0.1875 - c) = 227.0 -> 224; 2^(8 - 0.375 - c) = 153.8 -> 160.
    o = (224, 160) / 384 in the first two channels."""
    q, keys, vals = _two_key_case()
    o = f8.softmax_rows_fp8(q, keys, vals, *f8.head_scales(keys, vals))[0]
    expect = np.zeros(16)
    expect[0], expect[1] = 224 / 384, 160 / 384
    assert np.allclose(o, expect, rtol=0, atol=1e-12), o[:2]


def pin_hand_rowmax_offset(f8):
    """As above with q = 20 e1: c q = 7.2135 e1 = 0.9017 * 2^3, so s_q = 2^5 and Q8 = e4m3(230.8) =
    224; x = 224 (64, -128) / (32 * 128) = (3.5, -7); the bound c * 20 = 7.21 > 4, so the offset is
    max x = 3.5.  Weights: 2^8 = 256 (exact) and 2^(8 - 10.5) = 0.1768, in [2^-3, 2^-2) where E4M3
    steps by 2^-6 -> 11/64.  o = (256, 11/64) / (256 + 11/64)."""
    q, keys, vals = _two_key_case()
    q = q * 20.0
    o = f8.softmax_rows_fp8(q, keys, vals, *f8.head_scales(keys, vals))[0]
    tot = 256 + 11 / 64
    assert math.isclose(o[0], 256 / tot, rel_tol=0, abs_tol=1e-12), o[0]
    assert math.isclose(o[1], (11 / 64) / tot, rel_tol=0, abs_tol=1e-15), o[1]


def pin_uniform_visibility_fp8(f8):
    """Identical keys: every visible key gets the same rounded weight, so with one-hot frame values
    (exact in E4M3) o is each frame's share of the visible keys, exactly; the visible sets are the
    hand-derived golden frame sets of the 16-frame, chunk-2 workload."""
    T, N, C, H, d, n_text = 16, 3, 2, 1, 20, 2
    q = np.zeros((T * N, H, d))
    q[..., 0] = 1
    k = np.zeros_like(q)
    k[..., 0] = 1
    v = np.zeros_like(q)
    for f in range(T):
        v[f * N:(f + 1) * N, 0, f] = 1.0
    tk = np.zeros((n_text, H, d))
    tk[..., 0] = 1
    tv = np.zeros((n_text, H, d))
    tv[..., 16] = 1.0
    o = f8.softmax_branch_fp8(q, k, v, tk, tv, T, N, C, True)
    gold = pins.golden_frame_sets()
    for t in range(T):
        w, anc, _, _ = gold[t]
        vis = sorted(w + anc)
        nkeys = n_text + N * len(vis)
        expect = np.zeros(d)
        expect[vis] = N / nkeys
        expect[16] = n_text / nkeys
        for n in range(N):
            assert np.allclose(o[t * N + n, 0], expect, rtol=0, atol=1e-12), t


def pin_close_to_exact(f8, seed=3):
    """Against the exact softmax (float64) on unit-norm q, k and N(0,1) v: each E4M3 rounding
    moves a weight or a value by at most 2^-4 of itself (RMS 2^-4/sqrt(3) = 3.6 %), and o averages
    those moves, so the RMS error stays near 5 % of RMS(o); allowed: 6 % RMS, 30 % at the worst
    element."""
    rng = np.random.default_rng(seed)
    for d, n, qscale in ((128, 3000, 1.0), (64, 2000, 8.0)):
        q = pins._unit(rng.standard_normal((48, d))) * qscale
        k = pins._unit(rng.standard_normal((n, d)))
        v = rng.standard_normal((n, d))
        s = (q @ k.T) / math.sqrt(d)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        exact = (p @ v) / p.sum(axis=1, keepdims=True)
        o = f8.softmax_rows_fp8(q, k, v, *f8.head_scales(k, v))
        rms = np.sqrt((exact ** 2).mean())
        err = o - exact
        assert np.sqrt((err ** 2).mean()) <= 0.06 * rms
        assert np.abs(err).max() <= 0.30 * rms


def _bound_inputs(seed=7):
    """Rows over many keys with N(0,1) values: diffuse (unit queries), sharp (queries x64, so the
    bound exceeds 4 and the row maximum is the offset), very sharp over few keys, d = 64, and
    values small enough that some round in E4M3's subnormal range."""
    rng = np.random.default_rng(seed)
    cases = []
    for d, n, qscale, vscale in ((128, 3000, 1.0, 1.0), (128, 3000, 64.0, 1.0), (128, 200, 200.0, 1.0),
                                 (64, 800, 8.0, 1.0), (128, 1000, 1.0, 1e-3)):
        q = pins._unit(rng.standard_normal((48, d))) * qscale
        k = pins._unit(rng.standard_normal((n, d)))
        v = rng.standard_normal((n, d)) * vscale
        cases.append((q, k, v))
    return cases


def pin_exact_envelopes(f8):
    """The definition against the exact softmax (``exact_deviation_bounds``): its o is the exact
    softmax of ``vdn_oracle`` (float64); the definition's result lies inside the worst-case
    envelope and inside the probabilistic one at every element; and the RMS deviation predicted
    from the rounding steps matches the measured one within 0.8-1.25x on every input kind (so a
    change in the precision of any rounding step shows up)."""
    from oracle import vdn_oracle
    for q, k, v in _bound_inputs():
        sc = f8.head_scales(k, v)
        o, det, prob, rms = f8.exact_deviation_bounds(q, k, v, *sc)
        assert np.allclose(o, vdn_oracle.softmax_rows(q, k, v, np.float64), rtol=0, atol=1e-12)
        err = np.abs(f8.softmax_rows_fp8(q, k, v, *sc) - o)
        assert np.all(err <= det), float(np.max(err / det))
        assert np.all(err <= prob), float(np.max(err / prob))
        ratio = math.sqrt(float((err ** 2).mean()) / float((rms ** 2).mean()))
        assert 0.8 <= ratio <= 1.25, ratio


def pin_envelopes_have_teeth(f8):
    """On diffuse rows the probabilistic envelope stays below RMS(o) (the check is not vacuous);
    the worst-case one is the width of the value spread only when every rounding aligns."""
    q, k, v = _bound_inputs()[0]
    o, det, prob, rms = f8.exact_deviation_bounds(q, k, v, *f8.head_scales(k, v))
    r = float(np.sqrt((o ** 2).mean()))
    assert float(np.median(prob)) <= 0.6 * r
    assert float(np.median(rms)) <= 0.06 * r


def pin_allowance_hand(f8):
    """``ambiguous_rounding_effect`` on the two-key row-maximum case (q = 20 e1; weights 256 and
    2^-2.5 -> 11/64, see ``pin_hand_rowmax_offset``).  The small weight's exponent lies
    0.02356 log2 units from the E4M3 midpoint 11.5/64 above it; the large one 0.0875 from 272.
    Score-sum sizes sum|Q8 K8| / (s_q s_k): 3.5 (key 1), 7 (key 2), and the row maximum's 7 is
    added since the offset is the row maximum, so delta_1 = 10.5 r, delta_2 = 14 r (+ 2^-20
    (|exponent| + 8)).  r = 2^-12: nothing flagged, effect 0.  r = 2^-9 and 2^-7: key 2 only,
    effect 2 (1/64) max|v2 - o| / sum P8 = 2 (1/64) (256 / 256.171875) / 256.171875 = 1.21907e-4.
    r = 2^-6: both keys, + 2 * 32 * (11/64 / 256.171875) / 256.171875 = 1.67622e-4."""
    q, keys, vals = _two_key_case()
    q = q * 20.0
    sc = f8.head_scales(keys, vals)
    tot = 256 + 11 / 64
    e2 = 2 * (1 / 64) * (256 / tot) / tot
    e1 = 2 * 32 * ((11 / 64) / tot) / tot
    for r, want in ((2.0 ** -12, 0.0), (2.0 ** -9, e2), (2.0 ** -7, e2), (2.0 ** -6, e1 + e2)):
        got = f8.ambiguous_rounding_effect(q, keys, vals, *sc, rel_score_err=r)[0]
        assert math.isclose(got, want, rel_tol=1e-12, abs_tol=1e-18), (r, got, want)


def pin_allowance_brute_force(f8, seed=11, trials=40):
    """The allowance covers what it claims to: every score of a row is perturbed by an independent
    error of up to rel sum_i |Q8_i K8_ji| / (s_q s_k) (the row maximum with it, when it is the
    offset), the definition's remaining steps are redone from the perturbed scores, and the
    result moves by no more than ``ambiguous_rounding_effect`` with that rel.  Sharp rows over
    few keys, rel = 2^-9, so that weights do cross midpoints (counted, must be > 0)."""
    rng = np.random.default_rng(seed)
    d, n = 32, 60
    rel = 2.0 ** -9
    q = pins._unit(rng.standard_normal((24, d))) * rng.uniform(4.0, 40.0, (24, 1))
    k = pins._unit(rng.standard_normal((n, d)))
    v = rng.standard_normal((n, d))
    s_k, s_v, kmax = f8.head_scales(k, v)
    c = math.log2(math.e) / math.sqrt(d)
    k8, v8 = f8.e4m3(s_k * k), f8.e4m3(s_v * v)
    allow = f8.ambiguous_rounding_effect(q, k, v, s_k, s_v, kmax, rel_score_err=rel)
    flips = 0
    for i, qi in enumerate(q):
        s_q = f8.pow2_scale(np.abs(c * qi).max())
        q8 = f8.e4m3(s_q * c * qi)
        x = (k8 @ q8) / (s_q * s_k)
        size = (np.abs(k8) @ np.abs(q8)) / (s_q * s_k)
        b = c * math.sqrt(float(qi @ qi)) * kmax
        base_m = b if b <= f8.OFFSET_BOUND_LIMIT else x.max()
        p0 = f8.e4m3(np.exp2(f8.P_SHIFT + x - base_m))
        o0 = (p0 @ v8) / (s_v * p0.sum())
        for _ in range(trials):
            xp = x + rel * size * rng.uniform(-1.0, 1.0, n)
            m = b if b <= f8.OFFSET_BOUND_LIMIT else xp.max()
            p = f8.e4m3(np.exp2(f8.P_SHIFT + xp - m))
            o = (p @ v8) / (s_v * p.sum())
            flips += int(np.any(p != p0 * np.exp2(base_m - m)))
            assert np.abs(o - o0).max() <= allow[i] + 1e-12, (i, np.abs(o - o0).max(), allow[i])
    assert flips > 0


PINS = [pin_e4m3_library, pin_hand_bound_offset, pin_hand_rowmax_offset, pin_uniform_visibility_fp8,
        pin_close_to_exact, pin_exact_envelopes, pin_envelopes_have_teeth, pin_allowance_hand,
        pin_allowance_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(fresh())


# ---- planted mistakes ----

def m_truncating_round(f8):
    def e4m3(x):
        x = np.asarray(x, np.float64)
        a = np.abs(x)
        _, ex = np.frexp(a)
        step = np.ldexp(1.0, (np.maximum(ex - 1, -6) - 3).astype(np.int64))
        return np.copysign(np.minimum(np.floor(a / step) * step, 448.0), x)
    f8.e4m3 = e4m3


def m_ties_away(f8):
    def e4m3(x):
        x = np.asarray(x, np.float64)
        a = np.abs(x)
        _, ex = np.frexp(a)
        step = np.ldexp(1.0, (np.maximum(ex - 1, -6) - 3).astype(np.int64))
        return np.copysign(np.minimum(np.floor(a / step + 0.5) * step, 448.0), x)
    f8.e4m3 = e4m3


def m_no_subnormals(f8):
    orig = f8.e4m3

    def e4m3(x):
        r = orig(x)
        return np.where(np.abs(r) < 2.0 ** -6, 0.0, r)
    f8.e4m3 = e4m3


def m_unrounded_denominator(f8):
    def softmax_rows_fp8(qr, keys, vals, s_k, s_v, kmax):
        qr = np.asarray(qr, np.float64)
        c = math.log2(math.e) / math.sqrt(qr.shape[-1])
        k8, v8 = f8.e4m3(s_k * keys), f8.e4m3(s_v * vals)
        out = np.zeros(qr.shape)
        for i, q in enumerate(qr):
            s_q = f8.pow2_scale(np.abs(c * q).max())
            x = (k8 @ f8.e4m3(s_q * c * q)) / (s_q * s_k)
            b = c * math.sqrt(float(q @ q)) * kmax
            m = b if b <= 4 else x.max()
            p = np.exp2(8 + x - m)
            out[i] = (f8.e4m3(p) @ v8) / (s_v * p.sum())
        return out
    f8.softmax_rows_fp8 = softmax_rows_fp8


def m_always_rowmax(f8):
    f8.OFFSET_BOUND_LIMIT = -1.0


def m_no_shift(f8):
    f8.P_SHIFT = 0.0


def m_value_scale_kept(f8):
    orig = f8.softmax_rows_fp8

    def softmax_rows_fp8(qr, keys, vals, s_k, s_v, kmax):
        return orig(qr, keys, vals, s_k, s_v, kmax) * s_v
    f8.softmax_rows_fp8 = softmax_rows_fp8


def m_query_scale_dropped(f8):
    orig = f8.pow2_scale

    def softmax_rows_fp8(qr, keys, vals, s_k, s_v, kmax):
        qr = np.asarray(qr, np.float64)
        c = math.log2(math.e) / math.sqrt(qr.shape[-1])
        k8, v8 = f8.e4m3(s_k * keys), f8.e4m3(s_v * vals)
        out = np.zeros(qr.shape)
        for i, q in enumerate(qr):
            s_q = orig(np.abs(c * q).max())
            x = (k8 @ f8.e4m3(s_q * c * q)) / s_k             # wrong: s_q not divided out
            b = c * math.sqrt(float(q @ q)) * kmax
            m = b if b <= 4 else x.max()
            p8 = f8.e4m3(np.exp2(8 + x - m))
            out[i] = (p8 @ v8) / (s_v * p8.sum())
        return out
    f8.softmax_rows_fp8 = softmax_rows_fp8


def m_window_without_anchors(f8):
    orc = f8.orc
    orig = orc.key_frames

    class Shim:
        def __getattr__(self, name):
            return getattr(orc, name)

        @staticmethod
        def key_frames(t, T, C, anchors):
            return sorted(orc.frame_sets(t, T, C, anchors)[0])
    f8.orc = Shim()
    assert orig is orc.key_frames


def m_two_mantissa_bits(f8):
    """The definition rounds to two mantissa bits (E5M2-like spacing) instead of three."""
    def e4m3(x):
        x = np.asarray(x, np.float64)
        a = np.abs(x)
        _, ex = np.frexp(a)
        step = np.ldexp(1.0, (np.maximum(ex - 1, -6) - 2).astype(np.int64))
        return np.copysign(np.minimum(np.round(a / step) * step, 448.0), x)
    f8.e4m3 = e4m3


def m_envelope_without_value_rounding(f8):
    """The envelopes forget that the values are rounded too."""
    orig = f8.e4m3_half_step

    def e4m3_half_step(y):
        return orig(y) * 1e-9
    f8.e4m3_half_step = e4m3_half_step


def m_allowance_window_quartered(f8):
    orig = f8.ambiguous_rounding_effect

    def ambiguous_rounding_effect(qr, keys, vals, s_k, s_v, kmax, rel_score_err=2.0 ** -16):
        return orig(qr, keys, vals, s_k, s_v, kmax, rel_score_err / 4)
    f8.ambiguous_rounding_effect = ambiguous_rounding_effect


def m_allowance_one_quarter_step(f8):
    orig = f8.ambiguous_rounding_effect

    def ambiguous_rounding_effect(*args, **kw):
        return orig(*args, **kw) * 0.125
    f8.ambiguous_rounding_effect = ambiguous_rounding_effect


MUTANTS = [
    (m_two_mantissa_bits, pin_exact_envelopes),
    (m_envelope_without_value_rounding, pin_exact_envelopes),
    (m_allowance_window_quartered, pin_allowance_hand),
    (m_allowance_one_quarter_step, pin_allowance_brute_force),
    (m_truncating_round, pin_e4m3_library),
    (m_ties_away, pin_e4m3_library),
    (m_no_subnormals, pin_e4m3_library),
    (m_unrounded_denominator, pin_hand_bound_offset),
    (m_always_rowmax, pin_hand_bound_offset),
    (m_no_shift, pin_hand_rowmax_offset),
    (m_value_scale_kept, pin_hand_bound_offset),
    (m_query_scale_dropped, pin_hand_bound_offset),
    (m_window_without_anchors, pin_uniform_visibility_fp8),
]


@pytest.mark.parametrize("mutate,pin", MUTANTS, ids=[m.__name__ for m, _ in MUTANTS])
def test_mutant_is_caught(mutate, pin):
    f8 = fresh()
    pin(f8)
    mutate(f8)
    with pytest.raises(AssertionError):
        pin(f8)
