"""Rotary position embedding, fp64 — oracle (test infrastructure).

The pages describe RoPE only as a position-dependent rotation R_m inserted
between the key and query factors (page "Multi-Head Latent Attention (MLA)",
section "The RoPE problem"; page "Multi-head Latent Attention (MLA): how
DeepSeek cuts KV cache memory", section "What MLA costs").  The reading used
here is the original rotary form: consecutive pairs (2j, 2j+1) are rotated by
the angle pos * base^(-2j/d).  The pages do not fix which coordinates pair
up; any pairing is a relabelling of the RoPE weight columns (pinned: the
half-split pairing on permuted columns gives the same outputs), and the GPU
path uses this one.
"""
import numpy as np


def angles(pos, d_rope: int, base: float) -> np.ndarray:
    """[..., d_rope/2] rotation angles for integer positions ``pos``."""
    j = np.arange(d_rope // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * j / d_rope)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta


def apply(v: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate the last axis of ``v`` (pairs (2j, 2j+1)) by position ``pos``.

    ``pos`` broadcasts against ``v.shape[:-1]``.
    """
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    ang = angles(pos, d, base)
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty(np.broadcast_shapes(v.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out
