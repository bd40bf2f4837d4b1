"""Absorbed (merged-weight) MLA, fp64 numpy — oracle (test infrastructure).

The two merges of page "Multi-Head Latent Attention (MLA)", section "Two
merges are where the compute win comes from" (also page "How DeepSeek
Rewrote the Transformer", "The short version": the up-projections are
absorbed into the query and output computations):

* query side: W_UQK[h] = W_UQ[h] W_UK[h]^T, so the nope score is
  (c_Q W_UQK[h]) · c_i, computed straight from the cached latent;
* output side: W_UVO[h] = W_UV[h] W_O[h], so y = sum_h (sum_i p c_i) W_UVO[h].

The decoupled RoPE part of the score is unchanged: q_pe_h · k_pe_i.  This is
the same function as ``expanded`` up to rounding; the tests pin the two
together at fp64 precision, which lets this form stand in for the expanded
one at the long-context sizes where expanding every latent costs too much.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import rope as _rope


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def merged_weights(W: Dict[str, np.ndarray], heads: Optional[Sequence[int]] = None,
                   want_uvo: bool = True):
    """W_UQK [Hs, d_LQ, d_L] and W_UVO [Hs, d_L, d_model] in fp64."""
    W_UQ, W_UK = _f64(W["W_UQ"]), _f64(W["W_UK"])
    H = W_UQ.shape[1]
    hs = list(range(H)) if heads is None else list(heads)
    uqk = np.stack([W_UQ[:, h, :] @ W_UK[:, h, :].T for h in hs])
    uvo = None
    if want_uvo:
        W_UV, W_O = _f64(W["W_UV"]), _f64(W["W_O"])
        uvo = np.stack([W_UV[:, h, :] @ W_O[h] for h in hs])
    return uqk, uvo


def query_latent(W: Dict[str, np.ndarray], uqk: np.ndarray, x: np.ndarray, pos,
                 base: float, heads: Optional[Sequence[int]] = None):
    """q_lat [n, Hs, d_L] and q_pe [n, Hs, d_rope] for tokens x at ``pos``."""
    x = _f64(x)
    c_q = x @ _f64(W["W_DQ"])
    q_lat = np.einsum("nl,hlc->nhc", c_q, uqk, optimize=True)
    W_QR = _f64(W["W_QR"])
    hs = list(range(W_QR.shape[1])) if heads is None else list(heads)
    q_pe = _rope.apply(np.einsum("nl,lhr->nhr", c_q, W_QR[:, hs, :], optimize=True),
                       np.asarray(pos)[:, None], base)
    return q_lat, q_pe


def attention(q_lat: np.ndarray, q_pe: np.ndarray, c: np.ndarray, k_pe: np.ndarray,
              q_pos: Sequence[int], scale: float, uvo: Optional[np.ndarray] = None) -> dict:
    """Scores straight from latents; returns o_lat [n, Hs, d_L], lse, y."""
    q_lat, q_pe, c, k_pe = _f64(q_lat), _f64(q_pe), _f64(c), _f64(k_pe)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    m = c.shape[0]
    visible = np.arange(m)[None, None, :] <= q_pos[:, None, None]   # [n, 1, m]
    s = (np.einsum("nhc,mc->nhm", q_lat, c, optimize=True)
         + np.einsum("nhr,mr->nhm", q_pe, k_pe, optimize=True)) * scale
    s = np.where(visible, s, -np.inf)
    mx = s.max(axis=2, keepdims=True)
    e = np.exp(s - mx)
    den = e.sum(axis=2, keepdims=True)
    p = e / den
    o_lat = np.einsum("nhm,mc->nhc", p, c, optimize=True)
    out = {"o_lat": o_lat, "lse": mx[..., 0] + np.log(den[..., 0])}
    if uvo is not None:
        out["y"] = np.einsum("nhc,hcd->nd", o_lat, uvo, optimize=True)
    return out


def out_proj(o_lat: np.ndarray, uvo: np.ndarray) -> np.ndarray:
    """y [n, d_model] = sum_h o_lat[:, h] W_UVO[h]."""
    return np.einsum("nhc,hcd->nd", _f64(o_lat), uvo, optimize=True)
