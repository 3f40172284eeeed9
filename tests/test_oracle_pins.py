"""The CPU oracle against what the pages and mathematics fix (no GPU)."""

import numpy as np
import pytest
import torch

import pins
from oracle import vdn_oracle as orc


@pytest.mark.parametrize("pin", [
    pins.pin_objective_minimum, pins.pin_sherman_morrison, pins.pin_repeated_keys,
    pins.pin_orthonormal_keys, pins.pin_spectrum, pins.pin_contraction, pins.pin_neumann,
    pins.pin_cho_solve, pins.pin_golden_frame_sets, pins.pin_partition,
    pins.pin_uniform_keys_visibility, pins.pin_beta_zero, pins.pin_text_once,
    pins.pin_boundary_text_only, pins.pin_gate_closed_forms, pins.pin_bruteforce,
    pins.pin_decay_one, pins.pin_decay_zero, pins.pin_decay_columns, pins.pin_decay_nonexpansive,
    pins.pin_bruteforce_decay, pins.pin_golden_attention_map, pins.pin_context_rows_sdpa,
    pins.pin_audio_softmax_only, pins.pin_bruteforce_joint,
], ids=lambda f: f.__name__)
def test_pin(pin):
    pin(orc)


def test_single_chunk_is_dense_attention():
    """P13: with one chunk covering every frame and anchors off, the softmax branch is plain dense
    attention over text and video keys (checked against torch's CPU SDPA), and the linear branch
    holds only the text (2 S0 q)."""
    rng = np.random.default_rng(20)
    T, N, C, n_text, H, d = 4, 5, 4, 3, 2, 8
    inp = pins.tiny_inputs(T, N, n_text, H, d, 21)
    o_s = orc.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], T, N, C, False)
    for h in range(H):
        qh = torch.from_numpy(inp["q"][:, h])[None, None]
        kh = torch.from_numpy(np.concatenate([inp["text_k"][:, h], inp["k"][:, h]]))[None, None]
        vh = torch.from_numpy(np.concatenate([inp["text_v"][:, h], inp["v"][:, h]]))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh)[0, 0].numpy()
        assert np.allclose(o_s[:, h], ref, atol=1e-5)
    o_l = orc.linear_branch(inp["q"], inp["k"], inp["v"], inp["beta"], inp["text_k"], inp["text_v"],
                            T, N, C, False)
    for h in range(H):
        s0 = orc.text_state(inp["text_k"][:, h], inp["text_v"][:, h], inp["beta"][:n_text, h])
        assert np.allclose(o_l[:, h], inp["q"][:, h].astype(np.float64) @ (2 * s0).T, atol=1e-10)



def test_text_half_state_reading_is_exactly_once():
    """The alternative reading of the text halving (solve at full beta, halve the state) makes the
    two readouts sum to exactly the full-beta text solve; kept selectable for later correction."""
    rng = np.random.default_rng(22)
    tk = pins._unit(rng.standard_normal((5, 4)))
    tv = rng.standard_normal((5, 4))
    tb = rng.random(5)
    half = orc.text_state(tk, tv, tb, "half_state")
    full = orc.frame_update(np.zeros((4, 4)), *orc.frame_stats(tk, tv, tb))
    assert np.allclose(half + half, full, atol=1e-14)


def test_anchor_density_near_page_figure():
    """Weak check of the anchors' extra attention density against the page's 3.57% ([VDN] "Local
    Softmax and Long-Range Linear Memory"): at the 102-latent-frame length of the release's
    latent shape with 5-frame chunks, the frame pairs that anchors add beyond the window make up
    about 3.57% of all frame pairs under this reading.  Not a pin: other masks give the same."""
    T, C = 102, 5
    extra = sum(len(orc.frame_sets(t, T, C, True)[1]) for t in range(T))
    dens = 100.0 * extra / (T * T)
    assert abs(dens - 3.57) < 0.01, dens
