"""Pins of the MXFP8 epilogue oracle (oracle/mxfp8.py) against facts it does not compute itself:
the OCP E4M3 code table decoded bit by bit, closed forms of the block scale, products whose
operands are exactly representable, one-hot contractions that expose the blocking axis, scaling
laws of the definition, hand-worked allowance cases, and planted mistakes that these pins catch."""

import math

import numpy as np
import pytest

from oracle import mxfp8 as mx
from oracle import vdn_oracle as orc

D = 128


def e4m3_table():
    """Every finite OCP E4M3 value, decoded from its bits: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN."""
    vals = []
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append(-v if s else v)
    return np.unique(np.array(vals))


TABLE = e4m3_table()


def nearest_even(y):
    """Nearest table value to y, ties to the value with an even mantissa (bit 0 of the code)."""
    out = np.empty_like(y)
    for i, v in enumerate(y.ravel()):
        d = np.abs(TABLE - v)
        cand = TABLE[d == d.min()]
        if len(cand) == 1:
            out.ravel()[i] = cand[0]
        else:                                   # a tie: the even one (mantissa LSB 0)
            def even(c):
                a = abs(c)
                if a < 2.0 ** -6:
                    return round(a / 2.0 ** -9) % 2 == 0
                e = math.floor(math.log2(a))
                return round(a / 2.0 ** (e - 3)) % 2 == 0
            out.ravel()[i] = [c for c in cand if even(c)][0]
    return out


def test_table_shape():
    assert TABLE.max() == 448.0 and TABLE.min() == -448.0
    assert len(TABLE) == 253            # 254 finite codes, +0 and -0 equal
    assert np.min(TABLE[TABLE > 0]) == 2.0 ** -9


def test_block_exponent_closed_forms():
    b = np.zeros((5, 32))
    b[0, 3] = 2.0 ** 5                      # max exactly 2^k: X = k - 7, scaled max 128
    b[1, 7] = -(2.0 ** 5) * (1 - 2.0 ** -20)   # just below 2^k: X = k - 8, scaled max < 256
    b[2, :] = 0.0                           # all zero: X = 0
    b[3, 0] = 2.0 ** -140                   # tiny: clamped to -127
    b[4, :] = 1.0
    X = mx.block_exponents(b, -1)[:, 0]
    assert list(X) == [5 - 7, 5 - 8, 0, -127, -7]
    for i in (0, 1, 4):
        top = np.abs(b[i]).max() / 2.0 ** X[i]
        assert 128 <= top < 256


def test_quantize_matches_brute_force_nearest():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 64)) * np.exp(rng.uniform(-6, 6, (40, 1)))
    x[3, :32] = 0.0
    q, X = mx.mx_quantize(x, -1)
    scale = np.ldexp(1.0, np.repeat(X, 32, axis=-1))
    want = nearest_even(x / scale) * scale
    assert np.array_equal(q, want)


def test_quantize_ties_to_even():
    # scaled values 1 + 1/16 (between 1 and 1.125): tie -> 1 (even); 1 + 3/16 -> 1.25 (even)
    blk = np.full(32, 1.0 + 1.0 / 16)
    blk[1] = 1.0 + 3.0 / 16
    blk[2] = 200.0                           # sets X = 0 (max in [128, 256))
    q, X = mx.mx_quantize(blk[None, :], -1)
    assert X[0, 0] == 0
    assert q[0, 0] == 1.0 and q[0, 1] == 1.25 and q[0, 2] == 192.0


def test_representable_values_round_trip():
    rng = np.random.default_rng(2)
    codes = rng.choice(TABLE[np.abs(TABLE) <= 240], size=(8, 128))
    codes[:, ::32] = 192.0                   # on the grid; every block max in [128, 256): scale 1
    x = codes * 2.0 ** 5
    q, X = mx.mx_quantize(x, -1)
    assert np.all(X == 5) and np.array_equal(q, x)


def test_relative_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128))
    q, X = mx.mx_quantize(x, -1)
    y = np.abs(x) / np.ldexp(1.0, np.repeat(X, 32, axis=-1))
    normal = y >= 2.0 ** -6
    assert np.all(np.abs(q - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] + 1e-300)


def test_matmul_blocks_columns_of_w_along_rows():
    # x = one-hot e_i picks row i of MX(W): W's column j is quantised along i, so row i of the
    # result is W[i, :] rounded with the block of column j that holds i
    rng = np.random.default_rng(4)
    w = rng.standard_normal((128, 16))
    w[5, 3] = 50.0                           # a large entry sets the scale of its block only
    for i in (5, 6, 40):
        x = np.zeros(128)
        x[i] = 1.0
        got = mx.mx_matmul(x, w)
        for j in range(16):
            blk = w[(i // 32) * 32:(i // 32) * 32 + 32, j]
            m = np.abs(blk).max()
            X = math.frexp(m)[1] - 8
            want = nearest_even(np.array([w[i, j] / 2.0 ** X]))[0] * 2.0 ** X
            assert got[j] == want, (i, j)


def representable(rng, shape, axis):
    """Random values that MX quantisation leaves unchanged along ``axis``."""
    v = rng.choice(TABLE[(np.abs(TABLE) >= 1) & (np.abs(TABLE) <= 128)], size=shape)
    idx = [slice(None)] * len(shape)
    idx[axis] = slice(0, None, 32)
    v[tuple(idx)] = 192.0
    return v * 2.0 ** -9


def test_epilogue_equals_exact_when_every_rounding_is_exact():
    # gate weights 0 -> sigmoid(0) = 1/2 for both gates, so x_s = o_s / 2 and z_l = o_l / 2 are
    # representable when o_s, o_l are; then MX changes nothing and the definition is the exact
    # epilogue
    rng = np.random.default_rng(5)
    n = 24
    q = representable(rng, (n, D), 1)
    o_s = representable(rng, (n, D), 1)
    o_l = representable(rng, (n, D), 1)
    gw = np.zeros((2, D, D))
    pw = np.stack([representable(rng, (D, D), 0), representable(rng, (D, D), 0)])
    got = mx.epilogue_mx(q, o_s, o_l, gw, pw)
    want = orc.merge(q, o_s, o_l, gw, pw)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13 * np.abs(want).max())


def random_case(seed, n=40):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, D))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    gw = rng.standard_normal((2, D, D)) / np.sqrt(D)
    pw = rng.standard_normal((2, D, D)) / np.sqrt(D)
    o_s = rng.standard_normal((n, D)) * 0.3
    o_l = rng.standard_normal((n, D)) * 2.0
    return q, o_s, o_l, gw, pw


def test_deviation_inside_worst_case_envelope():
    for seed in range(4):
        q, o_s, o_l, gw, pw = random_case(seed)
        dev = np.abs(mx.epilogue_mx(q, o_s, o_l, gw, pw) - orc.merge(q, o_s, o_l, gw, pw))
        bound = mx.epilogue_mx_deviation_bound(q, o_s, o_l, gw, pw)
        assert np.all(dev <= bound)
        rms = np.sqrt(np.mean(orc.merge(q, o_s, o_l, gw, pw) ** 2))
        # three mantissa bits on both operands of every product: a few per cent, never zero
        assert 0.005 < np.sqrt(np.mean(dev ** 2)) / rms < 0.1


def test_linear_branch_quantised_before_rmsnorm():
    # scaling o_l by c leaves the exact layer unchanged (up to eps) but moves every z_l element
    # relative to the E4M3 grid, so the definition's output changes at the rounding level; a
    # version that quantised r * z_l instead would not change at all
    q, o_s, o_l, gw, pw = random_case(7)
    a = mx.epilogue_mx(q, o_s, o_l, gw, pw)
    b = mx.epilogue_mx(q, o_s, 3.0 * o_l, gw, pw)
    d = np.abs(a - b)
    rms = np.sqrt(np.mean(a ** 2))
    assert d.max() > 1e-4 * rms
    assert np.all(d <= mx.epilogue_mx_deviation_bound(q, o_s, o_l, gw, pw)
                  + mx.epilogue_mx_deviation_bound(q, o_s, 3.0 * o_l, gw, pw) + 1e-9 * rms)
    # a power-of-two scale keeps every code (block exponents shift): unchanged up to eps
    c = mx.epilogue_mx(q, o_s, 4.0 * o_l, gw, pw)
    assert np.max(np.abs(a - c)) < 1e-6 * rms


def test_readout_slots():
    T, N, C, H, d = 7, 3, 3, 2, 32
    nc = (T + C - 1) // C
    rng = np.random.default_rng(8)
    states = np.zeros((2, nc + 1, H, d, d))
    for s in range(nc + 1):
        states[0, s] = (s + 1) * np.eye(d)           # forward slot s: (s+1) I
        states[1, s] = 10 * (s + 1) * np.eye(d)      # reverse slot s: 10 (s+1) I
    q = rng.standard_normal((T * N, H, d))
    o = mx.readout(states, q, T, N, C, True)
    for t in range(T):
        slot = nc if t in (0, T - 1) else t // C
        assert np.allclose(o[t * N:(t + 1) * N], 11 * (slot + 1) * q[t * N:(t + 1) * N])
    o2 = mx.readout(states, q, T, N, C, False)
    assert np.allclose(o2[:N], 11 * q[:N])            # frame 0 without anchors: chunk 0
    # S q, not S^T q
    states[0, 0] = rng.standard_normal((H, d, d))
    states[1, 0] = 0
    o3 = mx.readout(states, q, T, N, C, False)
    for h in range(H):
        assert np.allclose(o3[N, h], states[0, 0, h] @ q[N, h])


def test_flip_weights_hand_worked():
    blk = np.full((1, 32), 3.0)
    blk[0, 0] = 192.0                        # scale 1 (192 is on the grid)
    blk[0, 1] = 1.0 + 1.0 / 16               # exactly a midpoint (step 1/8 at 1)
    blk[0, 2] = 1.0 + 1.0 / 16 + 2.0 ** -12  # 2^-12 away from it
    f0 = mx._flip_weights(blk, 0.0)
    assert f0[0, 1] == 0.125 and f0[0, 2] == 0 and f0[0, 0] == 0
    f1 = mx._flip_weights(blk, 2.0 ** -11)
    assert f1[0, 2] == 0.125 and f1[0, 3] == 0
    # a block maximum at a power of two: the exponent is ambiguous, every element gets a coarse step
    b2 = np.full((1, 32), 3.0)
    b2[0, 0] = 128.0
    f2 = mx._flip_weights(b2, 1e-9)
    assert np.all(f2[0] > 0)
    assert f2[0, 5] == 0.25                  # 3 on the grid of 2^1 (1.5, step 1/8): 1/4


def test_allowance_vanishes_without_error_and_grows_with_it():
    q, o_s, o_l, gw, pw = random_case(9)
    a0 = mx.epilogue_mx_allowance(q, o_s, o_l, np.zeros_like(o_l), gw, pw, rel_vec=0.0)
    assert np.all(a0 == 0)
    a1 = mx.epilogue_mx_allowance(q, o_s, o_l, np.abs(o_l) * 2.0 ** -15, gw, pw)
    a2 = mx.epilogue_mx_allowance(q, o_s, o_l, np.abs(o_l) * 2.0 ** -8, gw, pw)
    assert np.all(a2 >= a1) and a2.sum() > a1.sum() > 0


# ---- planted mistakes: each must make one of the pins above fail ----

def _mutant_quantize_truncate(x, axis=-1):
    X = mx.block_exponents(x, axis)
    scale = np.ldexp(1.0, np.repeat(X, 32, axis=axis))
    y = np.asarray(x, np.float64) / scale
    step = mx.e4m3_step(y)
    return np.trunc(y / step) * step * scale, X


_block_exponents = mx.block_exponents


def _mutant_block_exponents(x, axis=-1):
    return _block_exponents(x, axis) + 1


def test_planted_mistakes_are_caught(monkeypatch):
    monkeypatch.setattr(mx, "mx_quantize", _mutant_quantize_truncate)
    with pytest.raises(AssertionError):
        test_quantize_matches_brute_force_nearest()
    monkeypatch.undo()
    monkeypatch.setattr(mx, "block_exponents", _mutant_block_exponents)
    with pytest.raises(AssertionError):
        test_block_exponent_closed_forms()
    monkeypatch.undo()
    # blocking W along its columns instead of its rows
    monkeypatch.setattr(mx, "mx_matmul", lambda x, w: mx.mx_quantize(x, -1)[0] @ mx.mx_quantize(w, 1)[0])
    with pytest.raises(AssertionError):
        test_matmul_blocks_columns_of_w_along_rows()
    monkeypatch.undo()
    # quantising r * z_l instead of z_l

    def epi_r_first(q, o_s, o_l, gate_w, proj_w, eps=orc.RMS_EPS):
        gw, pw = np.asarray(gate_w, float), np.asarray(proj_w, float)
        x_s = orc.sigmoid(mx.mx_matmul(q, gw[0])) * o_s
        r = 1.0 / np.sqrt(np.mean(o_l * o_l, axis=-1, keepdims=True) + eps)
        z = orc.sigmoid(mx.mx_matmul(q, gw[1])) * o_l * r
        return mx.mx_matmul(x_s, pw[0]) + mx.mx_matmul(z, pw[1])
    monkeypatch.setattr(mx, "epilogue_mx", epi_r_first)
    with pytest.raises(AssertionError):
        test_linear_branch_quantised_before_rmsnorm()
    monkeypatch.undo()
    # an allowance that ignores block-exponent ambiguity

    def flip_no_block(v, win, axis=-1):
        v = np.asarray(v, float)
        win = np.broadcast_to(np.asarray(win, float), v.shape)
        X = mx.block_exponents(v, axis)
        scale = np.ldexp(1.0, np.repeat(X, 32, axis=axis))
        y = np.abs(v) / scale
        s = mx.e4m3_step(y)
        mid = np.floor(y / s) * s + s / 2
        return np.where(np.abs(y - mid) * scale <= win, s * scale, 0.0)
    monkeypatch.setattr(mx, "_flip_weights", flip_no_block)
    with pytest.raises(AssertionError):
        test_flip_weights_hand_worked()
