"""Seeded synthetic inputs for the VDN layer workloads.

This module only draws random numbers and shapes them: it holds none of the layer's arithmetic.
Both the GPU tests/benchmark and the CPU oracle consume what it produces, so it lives in a module
of its own.

Draw order (numpy ``default_rng(seed)``, float32 draws): q [T*N,H,d], k [T*N,H,d], v [T*N,H,d],
text_k [n_text,H,d], text_v [n_text,H,d], beta_raw [n_text+T*N,H], gate_w [2,d,d], proj_w [2,d,d].
Then q, k and text_k are L2-normalised along d (in float64, cast back to float32);
beta = beta_raw ~ U(0,1) for the uniform recipe or sigmoid(N(0,1)) for the sigmoid recipe;
weights ~ N(0, 1/d); v and text_v ~ N(0, 1).  bf16 workloads round q, k, v, text_k, text_v and
the weights to bfloat16 (round to nearest even, through torch); beta stays float32.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    n_text: int
    T: int
    N: int
    C: int
    H: int
    d: int
    dtype: str          # "fp32" or "bf16"
    beta_dist: str      # "uniform" or "sigmoid"
    anchors: bool = True

    @property
    def tokens(self) -> int:
        return self.T * self.N


# The five layer workloads: a tiny fp32 case, then bf16 cases up to one GPU's head share of a
# 768p clip and a long clip.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, 16, 2, 1, 16, "fp32", "uniform"),
    "small": Workload("small", 64, 20, 256, 5, 4, 64, "bf16", "sigmoid"),
    "medium": Workload("medium", 256, 60, 1024, 5, 8, 128, "bf16", "sigmoid"),
    "768p": Workload("768p", 512, 75, 1536, 5, 5, 128, "bf16", "sigmoid"),
    "long": Workload("long", 512, 180, 1536, 5, 5, 128, "bf16", "sigmoid"),
}


def custom(n_text, T, N, C, H, d, dtype="bf16", beta_dist="sigmoid", anchors=True, name="custom"):
    return Workload(name, n_text, T, N, C, H, d, dtype, beta_dist, anchors)


def _l2n(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    n = np.sqrt((x64 * x64).sum(axis=-1, keepdims=True))
    n = np.where(n == 0, 1.0, n)
    return (x64 / n).astype(np.float32)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float32).numpy()


def make_inputs(w: Workload, seed: int = 0, stress: bool = False, decay: bool = False, n_audio: int = 0,
                ctx_rows: bool = False) -> dict:
    """float32 numpy inputs (bf16-rounded for bf16 workloads).

    ``stress=True`` replaces each frame's keys by normalise(shared + 0.1 * noise) so that one
    direction of the per-frame key Gram matrix is crowded (large top eigenvalue).
    ``decay=True`` adds ``alpha`` ``[T, H, d]`` float32 ~ U(0.5, 1), a per-frame channel-wise decay
    gate, drawn after every other input (so the other inputs do not change).
    ``n_audio > 0`` adds audio tokens ``audio_k`` (L2-normalised N(0,1)) and ``audio_v`` (N(0,1)),
    ``[n_audio, H, d]``; ``ctx_rows=True`` adds the text and audio query rows ``ctx_q``
    ``[n_text + n_audio, H, d]`` (L2-normalised N(0,1)).  Both come from a second generator,
    ``default_rng([seed, 1])``, drawn in that order, so the other inputs do not change.
    """
    rng = np.random.default_rng(seed)
    TN, H, d = w.T * w.N, w.H, w.d
    f32 = np.float32
    q = rng.standard_normal((TN, H, d), dtype=f32)
    k = rng.standard_normal((TN, H, d), dtype=f32)
    v = rng.standard_normal((TN, H, d), dtype=f32)
    text_k = rng.standard_normal((w.n_text, H, d), dtype=f32)
    text_v = rng.standard_normal((w.n_text, H, d), dtype=f32)
    if w.beta_dist == "uniform":
        beta = rng.random((w.n_text + TN, H), dtype=f32)
    else:
        braw = rng.standard_normal((w.n_text + TN, H), dtype=f32)
        beta = (1.0 / (1.0 + np.exp(-braw.astype(np.float64)))).astype(f32)
    gate_w = (rng.standard_normal((2, d, d), dtype=f32) / np.sqrt(d)).astype(f32)
    proj_w = (rng.standard_normal((2, d, d), dtype=f32) / np.sqrt(d)).astype(f32)
    if stress:
        shared = rng.standard_normal((w.T, 1, H, d), dtype=f32)
        noise = rng.standard_normal((w.T, w.N, H, d), dtype=f32)
        k = (shared + f32(0.1) * noise).reshape(TN, H, d)
    q = _l2n(q)
    k = _l2n(k)
    text_k = _l2n(text_k)
    out = dict(q=q, k=k, v=v, text_k=text_k, text_v=text_v, beta=beta, gate_w=gate_w, proj_w=proj_w)
    if decay:
        out["alpha"] = (0.5 + 0.5 * rng.random((w.T, H, d), dtype=f32)).astype(f32)
    if n_audio > 0 or ctx_rows:
        rng2 = np.random.default_rng([seed, 1])
        if n_audio > 0:
            out["audio_k"] = _l2n(rng2.standard_normal((n_audio, H, d), dtype=f32))
            out["audio_v"] = rng2.standard_normal((n_audio, H, d), dtype=f32)
        if ctx_rows:
            out["ctx_q"] = _l2n(rng2.standard_normal((w.n_text + n_audio, H, d), dtype=f32))
    if w.dtype == "bf16":
        for key in ("q", "k", "v", "text_k", "text_v", "gate_w", "proj_w", "audio_k", "audio_v", "ctx_q"):
            if key in out:
                out[key] = _round_bf16(out[key])
    return out


def sample_rows(w: Workload, per_frame: int = 2, seed: int = 1) -> np.ndarray:
    """A seeded sample of video-token indices: every frame's first and last token plus
    ``per_frame`` random tokens of each frame (covers boundary frames, chunk edges and tails)."""
    rng = np.random.default_rng(seed)
    rows = []
    for t in range(w.T):
        base = t * w.N
        picks = {0, w.N - 1}
        picks.update(int(x) for x in rng.integers(0, w.N, size=per_frame))
        rows.extend(base + p for p in sorted(picks))
    return np.array(sorted(set(rows)), dtype=np.int64)
