"""Expanded MLA, fp64 numpy — oracle (test infrastructure).

The method as the pages state it, with no merged weights:

* compress: each token x_i is projected to one latent c_i = x_i W_DKV shared
  by all heads (page "Latent Space Strikes Again", section "The Core Idea",
  step 1; page "Multi-Head Latent Attention (MLA)", section "The
  construction": L = X W_L; page "How DeepSeek Rewrote the Transformer",
  section 07: L_KV = X W_DKV);
* decoupled RoPE: a small non-latent key k_pe_i = RoPE_i(x_i W_KR), one
  vector shared by all heads, is cached beside c_i, and the query gets a
  matching non-latent part (page "Multi-Head Latent Attention (MLA)", section
  "The RoPE problem"); the cache then holds d_L + d_rope numbers per token
  (page "How DeepSeek Rewrote the Transformer", section 08);
* query: c_Q = x W_DQ, q_nope_h = c_Q W_UQ[h], q_pe_h = RoPE(c_Q W_QR[h])
  (page "Latent Space Strikes Again", "The Core Idea": q = B_Q U_Q x;
  page "Multi-Head Latent Attention (MLA)", "The construction":
  W_Q = W_LQ W_LQQ);
* expand: k_{h,i} = [c_i W_UK[h] ‖ k_pe_i], v_{h,i} = c_i W_UV[h]
  (page "Latent Space Strikes Again", step 2: k_i = B_K c_i, v_i = B_V c_i);
* attend: scores q_h·k_{h,i} scaled by 1/sqrt(d_nope + d_rope), later tokens
  masked, softmax per row, weighted sum of values, heads stacked and
  multiplied by W_O (page "How DeepSeek Rewrote the Transformer", section 03
  "Queries and keys"; page "Latent Space Strikes Again", the attention
  formula).

Row-vector convention throughout.  Weight shapes:
W_DQ [d_model, d_LQ], W_UQ [d_LQ, H, d_nope], W_QR [d_LQ, H, d_rope],
W_DKV [d_model, d_L], W_KR [d_model, d_rope], W_UK [d_L, H, d_nope],
W_UV [d_L, H, d_v], W_O [H, d_v, d_model].
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import rope as _rope


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def latent_rows(W: Dict[str, np.ndarray], x: np.ndarray, pos, base: float):
    """Cache rows for tokens ``x`` [n, d_model] at positions ``pos`` [n].

    Returns (c [n, d_L], k_pe [n, d_rope]) in fp64.
    """
    x = _f64(x)
    c = x @ _f64(W["W_DKV"])
    k_pe = _rope.apply(x @ _f64(W["W_KR"]), np.asarray(pos), base)
    return c, k_pe


def query(W: Dict[str, np.ndarray], x: np.ndarray, pos, base: float):
    """Query parts for tokens ``x`` [n, d_model] at positions ``pos`` [n].

    Returns (c_Q [n, d_LQ], q_nope [n, H, d_nope], q_pe [n, H, d_rope]).
    """
    x = _f64(x)
    c_q = x @ _f64(W["W_DQ"])
    W_UQ, W_QR = _f64(W["W_UQ"]), _f64(W["W_QR"])
    q_nope = (c_q @ W_UQ.reshape(W_UQ.shape[0], -1)).reshape(len(c_q), *W_UQ.shape[1:])
    q_rot = (c_q @ W_QR.reshape(W_QR.shape[0], -1)).reshape(len(c_q), *W_QR.shape[1:])
    q_pe = _rope.apply(q_rot, np.asarray(pos)[:, None], base)
    return c_q, q_nope, q_pe


def attention(W: Dict[str, np.ndarray], q_nope: np.ndarray, q_pe: np.ndarray,
              c: np.ndarray, k_pe: np.ndarray, q_pos: Sequence[int], scale: float,
              heads: Optional[Sequence[int]] = None, want_p: bool = False,
              want_y: bool = True, head_block: Optional[int] = None) -> dict:
    """Causal softmax attention with per-head keys/values expanded from c.

    q_nope [n, H, d_nope], q_pe [n, H, d_rope]; c [m, d_L], k_pe [m, d_rope]
    hold the m visible keys at positions 0..m-1; query i sees keys j <= q_pos[i].
    ``heads`` restricts the computation to a subset of heads (then ``y`` is
    the partial sum over those heads only and is omitted unless all heads
    are used).

    Returns dict with o_h [n, Hs, d_v], o_lat [n, Hs, d_L] (= sum_j p c_j,
    the latent-space head output), lse [n, Hs] (natural log of the softmax
    denominator of the scaled scores), optional p [n, Hs, m], and y
    [n, d_model].
    """
    W_UK, W_UV, W_O = _f64(W["W_UK"]), _f64(W["W_UV"]), _f64(W["W_O"])
    H = W_UK.shape[1]
    c, k_pe = _f64(c), _f64(k_pe)
    q_nope, q_pe = _f64(q_nope), _f64(q_pe)
    n, m = q_nope.shape[0], c.shape[0]
    q_pos = np.asarray(q_pos, dtype=np.int64)
    assert q_pos.shape == (n,) and (q_pos < m).all() and (q_pos >= 0).all()
    hs = list(range(H)) if heads is None else list(heads)
    d_v, d_L, d_model = W_UV.shape[2], c.shape[1], W_O.shape[2]
    if head_block is None:
        per_head = m * (W_UK.shape[2] + d_v) * 8 + n * m * 8 * 3
        head_block = int(max(1, min(16, (512 << 20) // max(per_head, 1))))
    visible = np.arange(m)[None, :] <= q_pos[:, None]          # [n, m]

    o_h = np.zeros((n, len(hs), d_v))
    o_lat = np.zeros((n, len(hs), d_L))
    lse = np.zeros((n, len(hs)))
    p_all = np.zeros((n, len(hs), m)) if want_p else None
    y = np.zeros((n, d_model))
    for s in range(0, len(hs), head_block):
        blk = hs[s:s + head_block]
        hb = len(blk)
        # up-project every visible latent to this block's per-head keys/values
        k_nope = (c @ W_UK[:, blk, :].reshape(d_L, -1)).reshape(m, hb, -1).transpose(1, 0, 2)  # [hb, m, d_nope]
        v = (c @ W_UV[:, blk, :].reshape(d_L, -1)).reshape(m, hb, -1).transpose(1, 0, 2)       # [hb, m, d_v]
        qn = q_nope[:, blk, :].transpose(1, 0, 2)                    # [hb, n, d_nope]
        qp = q_pe[:, blk, :].transpose(1, 0, 2)                      # [hb, n, d_rope]
        scores = (qn @ k_nope.transpose(0, 2, 1)) + (qp @ k_pe.T[None])  # [hb, n, m]
        scores = scores * scale
        scores = np.where(visible[None], scores, -np.inf)
        mx = scores.max(axis=2, keepdims=True)
        e = np.exp(scores - mx)
        den = e.sum(axis=2, keepdims=True)
        p = e / den                                                  # [hb, n, m]
        ob = p @ v                                                   # [hb, n, d_v]
        o_h[:, s:s + len(blk)] = ob.transpose(1, 0, 2)
        o_lat[:, s:s + len(blk)] = (p @ c).transpose(1, 0, 2)
        lse[:, s:s + len(blk)] = (mx[..., 0] + np.log(den[..., 0])).T
        if want_p:
            p_all[:, s:s + len(blk)] = p.transpose(1, 0, 2)
        if want_y:
            y += ob.transpose(1, 0, 2).reshape(n, -1) @ W_O[blk].reshape(hb * d_v, d_model)
    out = {"o_h": o_h, "o_lat": o_lat, "lse": lse}
    if want_p:
        out["p"] = p_all
    if want_y and len(hs) == H:
        out["y"] = y
    elif want_y:
        out["y_partial"] = y
    return out


def decode_step(W: Dict[str, np.ndarray], base: float, scale: float,
                x_new: np.ndarray, first_pos: int,
                c_hist: np.ndarray, k_pe_hist: np.ndarray, **kw) -> dict:
    """One step for one sequence: append n_q new tokens, then attend.

    ``x_new`` [n_q, d_model] sits at positions first_pos .. first_pos+n_q-1;
    ``c_hist``/``k_pe_hist`` hold the rows of positions 0 .. first_pos-1.
    The new tokens' own rows are appended first, so each new token sees
    itself and every earlier token (page "How DeepSeek Rewrote the
    Transformer", section 04: the new row needs all keys but only its own
    query row).
    """
    n_q = x_new.shape[0]
    pos = first_pos + np.arange(n_q)
    c_new, k_new = latent_rows(W, x_new, pos, base)
    c = np.concatenate([_f64(c_hist).reshape(-1, c_new.shape[1]), c_new])
    k_pe = np.concatenate([_f64(k_pe_hist).reshape(-1, k_new.shape[1]), k_new])
    _, q_nope, q_pe = query(W, x_new, pos, base)
    out = attention(W, q_nope, q_pe, c, k_pe, pos, scale, **kw)
    out["c_new"], out["k_pe_new"] = c_new, k_new
    return out
