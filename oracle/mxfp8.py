"""CPU oracle of the FP8 (MXFP8) epilogue variant of the VDN layer.

TEST INFRASTRUCTURE ONLY (same rules as ``vdn_oracle``: only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; it shares nothing with the GPU path).

The pages run the production layer with FP8 linear layers and name MXFP8 for the multi-GPU runs
([VDN] "Adapting the Pretrained H3 backbone"; the project page's SGLang section), but fix no
rounding.  This module is the definition used here for the epilogue's four d x d products (the
two sigmoid gates and the two output projections of [VDN] "Gating the Softmax and Linear Branch
Outputs"); every rounding is a stated, deterministic step.  The linear readout o_l = S q, the
RMSNorm, the sigmoids and the gating products stay exact.

Block format (MX-style, as the OCP microscaling formats: 32 elements share one power-of-two
scale, each element an OCP FP8 E4M3 value): a contraction vector is cut into blocks of 32
consecutive elements; a block with largest magnitude m = f 2^e (f in [0.5, 1)) gets the scale
2^X with X = max(e - 8, -127) (X = 0 for an all-zero block), so the scaled block's largest
magnitude lies in [128, 256) and nothing saturates (the OCP rule uses one less headroom bit and
saturates its largest elements; this reading keeps them exact to three mantissa bits).  Elements
are e4m3(x / 2^X) (round to nearest, ties to even); the dequantised value is that times 2^X.

For x W (x a row vector over the contraction index i, W [in][out]) x is quantised along i in
blocks of 32, and every column j of W along i in blocks of 32; the product of the dequantised
operands is then exact.

Definition, per token row and head, with q, o_s, o_l [d], gate_w, proj_w [2][d][d] ([in][out]):

    g_m = MX(q) MX(Wg_m)                         (m = 0, 1)
    x_s = sigmoid(g_0) * o_s,   z_l = sigmoid(g_1) * o_l
    r   = 1 / sqrt(mean(o_l^2) + 1e-6)
    out = MX(x_s) MX(Wp_0) + r (MX(z_l) MX(Wp_1))

z_l is quantised before the RMSNorm scale r is applied (r is one number per token, so the exact
layer is unchanged by that order; after rounding it is part of the definition).
"""

from __future__ import annotations

import numpy as np

from oracle import vdn_oracle as orc
from oracle.fp8_softmax import e4m3

BLOCK = 32
SCALE_HEADROOM = 8            # scaled block maxima in [2^7, 2^8)
X_MIN = -127                  # smallest power of two an E8M0 scale holds


def block_exponents(x, axis=-1) -> np.ndarray:
    """X of every 32-element block of ``x`` along ``axis`` (the axis length a multiple of 32);
    shape: x's with that axis divided by 32."""
    x = np.moveaxis(np.asarray(x, np.float64), axis, -1)
    n = x.shape[-1]
    assert n % BLOCK == 0
    m = np.abs(x.reshape(x.shape[:-1] + (n // BLOCK, BLOCK))).max(axis=-1)
    _, e = np.frexp(m)                                   # m = f 2^e, f in [0.5, 1)
    X = np.maximum(e.astype(np.int64) - SCALE_HEADROOM, X_MIN)
    X = np.where(m == 0.0, 0, X)
    return np.moveaxis(X, -1, axis)


def mx_quantize(x, axis=-1):
    """(dequantised values, block exponents) of ``x`` quantised in 32-element blocks along
    ``axis``; the values have x's shape."""
    x = np.asarray(x, np.float64)
    X = block_exponents(x, axis)
    Xe = np.repeat(X, BLOCK, axis=axis)
    scale = np.ldexp(1.0, Xe)
    return e4m3(x / scale) * scale, X


def mx_matmul(x, w):
    """MX(x) MX(w) for x [..., in] and w [in, out]: x blocked along its last axis, every column of
    w along its rows.  Exact product of the dequantised operands (fp64)."""
    xq, _ = mx_quantize(x, axis=-1)
    wq, _ = mx_quantize(w, axis=0)
    return xq @ wq


def epilogue_mx(q, o_s, o_l, gate_w, proj_w, eps=orc.RMS_EPS):
    """The MXFP8 epilogue for token rows (any leading shape, last axis d); fp64."""
    q = np.asarray(q, np.float64)
    o_s = np.asarray(o_s, np.float64)
    o_l = np.asarray(o_l, np.float64)
    gw = np.asarray(gate_w, np.float64)
    pw = np.asarray(proj_w, np.float64)
    x_s = orc.sigmoid(mx_matmul(q, gw[0])) * o_s
    z_l = orc.sigmoid(mx_matmul(q, gw[1])) * o_l
    r = 1.0 / np.sqrt(np.mean(o_l * o_l, axis=-1, keepdims=True) + eps)
    return mx_matmul(x_s, pw[0]) + r * mx_matmul(z_l, pw[1])


def readout(states, q, T, N, C, anchors):
    """o_l = (S_fwd + S_rev) q of every video token from a state buffer in the library's layout
    [2][Nc + 1][H][d][d] (forward slots, then reverse slots; slot Nc is the initial state, read by
    the boundary frames): frame t reads slot Nc if it is a boundary frame, else chunk t // C."""
    states = np.asarray(states, np.float64)
    q = np.asarray(q, np.float64)
    nc = (T + C - 1) // C
    H, d = q.shape[1], q.shape[2]
    out = np.zeros((T * N, H, d))
    for t in range(T):
        bnd = anchors and (t == 0 or t == T - 1)
        slot = nc if bnd else t // C
        s = states[0, slot] + states[1, slot]                  # [H][d][d]
        rows = slice(t * N, (t + 1) * N)
        out[rows] = np.einsum("hji,nhi->nhj", s, q[rows])
    return out


# ----------------------------------------------------------------------------------------------
# What separates a GPU result from this definition and from the exact epilogue.
# ----------------------------------------------------------------------------------------------

def e4m3_step(y) -> np.ndarray:
    """Spacing of the E4M3 grid at |y| (y already scaled into the block's range)."""
    a = np.abs(np.asarray(y, np.float64))
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -6)
    return np.ldexp(1.0, (e - 3).astype(np.int64))


def _flip_weights(v, win, axis=-1):
    """Per element of ``v`` (quantised along ``axis`` in blocks of 32): how far its dequantised
    value can move if ``v`` is only known to within +-``win`` (elementwise, absolute).  One grid
    step when a rounding midpoint lies within the window.  For a block whose largest magnitude is
    within the window of a power of two (where the block exponent changes) the element may be
    rounded on the grid of either exponent: every element of the block then gets one step of the
    coarser grid (2^(X+1)).  Zero elsewhere."""
    v = np.asarray(v, np.float64)
    win = np.broadcast_to(np.asarray(win, np.float64), v.shape)
    X = block_exponents(v, axis)
    scale = np.ldexp(1.0, np.repeat(X, BLOCK, axis=axis))
    y = np.abs(v) / scale
    srel = e4m3_step(y)
    mid = np.floor(y / srel) * srel + srel / 2
    flip = np.where(np.abs(y - mid) * scale <= win, srel * scale, 0.0)
    vm = np.moveaxis(np.abs(v), axis, -1)
    wm = np.moveaxis(win, axis, -1)
    sh = vm.shape[:-1] + (vm.shape[-1] // BLOCK, BLOCK)
    amax = vm.reshape(sh).max(axis=-1)
    wmax = wm.reshape(sh).max(axis=-1)
    _, e = np.frexp(amax)
    e = e.astype(np.int64)
    near = (amax > 0) & ((np.ldexp(1.0, e) - amax <= wmax) | (amax - np.ldexp(1.0, e - 1) <= wmax))
    coarse = e4m3_step(y / 2) * 2 * scale                 # one step on the grid of 2^(X+1)
    blk = np.where(np.moveaxis(np.repeat(near, BLOCK, axis=-1), -1, axis), coarse, 0.0)
    return np.maximum(flip, blk)


def epilogue_mx_allowance(q, o_s, o_l, o_l_window, gate_w, proj_w, rel_vec=2.0 ** -17, eps=orc.RMS_EPS):
    """Element-wise bound, per output, on |GPU result - epilogue_mx| that follows from where a
    GPU computation of the same definition may round an E4M3 element differently: the inputs of
    MX(x_s) and MX(z_l) are computed values (fp32 gate sums, a fast sigmoid, the readout), so an
    element within their error of a rounding midpoint, or a block maximum within it of a power of
    two, may land on the neighbouring value.  q and the weights are exact inputs; their
    quantisation is the same on both sides.

    o_l_window: elementwise bound on the GPU's readout error (absolute).
    rel_vec: relative error of the GPU's gate logit, sigmoid and products, applied to the
      magnitudes they are computed from (the gate logit error is rel_vec * sum |q' w'|).
    Returns the allowance [..., d] (fp64): sum_i flip_i |w'_ij| over both projections (the second
    scaled by r), plus rel_vec times the magnitude sums of the projections themselves."""
    q = np.asarray(q, np.float64)
    o_s = np.asarray(o_s, np.float64)
    o_l = np.asarray(o_l, np.float64)
    gw = np.asarray(gate_w, np.float64)
    pw = np.asarray(proj_w, np.float64)
    qq, _ = mx_quantize(q, -1)
    terms = []
    for m in range(2):
        wq, _ = mx_quantize(gw[m], 0)
        g = qq @ wq
        gmag = np.abs(qq) @ np.abs(wq)
        sg = orc.sigmoid(g)
        dsg = rel_vec * gmag / 4.0 + rel_vec * sg          # sigmoid' <= 1/4, plus its own error
        terms.append((sg, dsg))
    (s0, ds0), (s1, ds1) = terms
    x_s = s0 * o_s
    z_l = s1 * o_l
    win_x = ds0 * np.abs(o_s) + rel_vec * np.abs(x_s)
    win_z = ds1 * np.abs(o_l) + s1 * np.asarray(o_l_window, np.float64) + rel_vec * np.abs(z_l)
    fx = _flip_weights(x_s, win_x, -1)
    fz = _flip_weights(z_l, win_z, -1)
    w0, _ = mx_quantize(pw[0], 0)
    w1, _ = mx_quantize(pw[1], 0)
    r = 1.0 / np.sqrt(np.mean(o_l * o_l, axis=-1, keepdims=True) + eps)
    xq, _ = mx_quantize(x_s, -1)
    zq, _ = mx_quantize(z_l, -1)
    mag = np.abs(xq) @ np.abs(w0) + r * (np.abs(zq) @ np.abs(w1))
    # the GPU's r comes from its own readout: |dr| / r <= (sum |o_l| w + sum w^2 / 2) / (sum o_l^2 + d eps)
    wl = np.asarray(o_l_window, np.float64)
    rel_r = (np.sum(np.abs(o_l) * wl + wl * wl / 2, axis=-1, keepdims=True) /
             (np.sum(o_l * o_l, axis=-1, keepdims=True) + o_l.shape[-1] * eps)) + rel_vec
    return fx @ np.abs(w0) + r * (fz @ np.abs(w1)) + rel_vec * mag + rel_r * r * (np.abs(zq) @ np.abs(w1))


def epilogue_mx_deviation_bound(q, o_s, o_l, gate_w, proj_w, eps=orc.RMS_EPS):
    """Worst-case bound, per output, on |epilogue_mx - exact epilogue| from the E4M3 roundings
    alone.  A block element y (scaled into [0, 256)) is off by at most half a grid step:
    relative 2^-4 for y >= 2^-6, absolute 2^-10 below.  Products: |a'b' - ab| <= |da||b| +
    |a||db| + |da||db|; the gate error passes through the sigmoid with slope <= 1/4."""
    q = np.asarray(q, np.float64)
    o_s = np.asarray(o_s, np.float64)
    o_l = np.asarray(o_l, np.float64)
    gw = np.asarray(gate_w, np.float64)
    pw = np.asarray(proj_w, np.float64)

    def half_step(v, axis):
        X = block_exponents(v, axis)
        scale = np.ldexp(1.0, np.repeat(X, BLOCK, axis=axis))
        return e4m3_step(v / scale) / 2 * scale

    def prod_bound(x, w):            # bound on |MX(x) MX(w) - x w|, and |x| |w|
        dx = half_step(x, -1)
        dw = half_step(w, 0)
        ax, aw = np.abs(x), np.abs(w)
        return dx @ aw + ax @ dw + dx @ dw, ax @ aw

    g = [q @ gw[m] for m in range(2)]
    dg = [prod_bound(q, gw[m])[0] for m in range(2)]
    s = [orc.sigmoid(v) for v in g]
    x_s, z_l = s[0] * o_s, s[1] * o_l
    dx_s = dg[0] / 4.0 * np.abs(o_s)               # |x_s' - x_s| before its own rounding
    dz_l = dg[1] / 4.0 * np.abs(o_l)
    r = 1.0 / np.sqrt(np.mean(o_l * o_l, axis=-1, keepdims=True) + eps)
    # MX(x') W' - x W = (MX(x') - x') W' + (x' - x) W' + x (W' - W), W' = MX(W)
    w0, _ = mx_quantize(pw[0], 0)
    w1, _ = mx_quantize(pw[1], 0)
    xs_p = np.abs(x_s) + dx_s                      # |x'| bound
    zl_p = np.abs(z_l) + dz_l
    b0 = half_step_bound(xs_p, dx_s) @ np.abs(w0) + dx_s @ np.abs(w0) + np.abs(x_s) @ np.abs(w0 - pw[0])
    b1 = half_step_bound(zl_p, dz_l) @ np.abs(w1) + dz_l @ np.abs(w1) + np.abs(z_l) @ np.abs(w1 - pw[1])
    return b0 + r * b1


def half_step_bound(mag, slack):
    """Half a grid step at magnitude up to ``mag`` inside its block, for a block whose largest
    element may reach max(mag + slack) (a larger maximum only coarsens the grid): the scale is
    the block's 2^(e - 8), the half step 2^-4 of the element (2^-10 of the scale below 2^-6)."""
    mag = np.asarray(mag, np.float64)
    sh = mag.shape[:-1] + (mag.shape[-1] // BLOCK, BLOCK)
    top = (mag + np.asarray(slack, np.float64)).reshape(sh).max(axis=-1)
    _, e = np.frexp(top)
    scale = np.ldexp(1.0, np.maximum(e.astype(np.int64) - SCALE_HEADROOM, X_MIN))
    scale = np.repeat(scale, BLOCK, axis=-1).reshape(mag.shape)
    return np.maximum(mag * 2.0 ** -4, scale * 2.0 ** -10)
