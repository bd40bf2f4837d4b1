"""Checks that tie the CPU oracle to what the pages and mathematics fix.

Each ``pin_*`` takes the oracle modules as arguments (so a test can hand in
a copy with a planted mistake) and returns the worst error it measured; the
tests assert that the real oracle passes every pin and that each planted
mistake fails at least one of them.
"""
from __future__ import annotations

import numpy as np
import torch

from synthetic import MLAConfig, make_case, config

from . import brute_mla

TINY = config(0)
# A mid-size shape with RoPE on, several heads and more keys than one tile.
MID = MLAConfig(name="mid", d_model=96, n_heads=6, d_latent=40, d_q_latent=56,
                d_nope=24, d_rope=16, d_v=24, dtype="f32", batch=2,
                cached=37, n_q=3, paged=False, init="fanin")


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _tokens(case, b):
    return np.concatenate([case.x_hist[b], case.x_new[b]]).astype(np.float64)


def _run_decode(E, case, b, W=None, **kw):
    cfg = case.cfg
    W = case.weights if W is None else W
    S = int(case.cached[b])
    c_h, k_h = E.latent_rows(W, case.x_hist[b], np.arange(S), cfg.rope_base)
    return E.decode_step(W, cfg.rope_base, cfg.softmax_scale, case.x_new[b], S, c_h, k_h,
                         want_p=True, **kw)


# Head blocks the expanded oracle is run with by the pins: its default (one
# block at these head counts), one head per block, and a block size that
# leaves a ragged last block (4 of the 6 MID heads, 3 of the 4 TINY heads).
HEAD_BLOCKS = (None, 1, 3, 4)


# ------------------------------------------------------------------ P1 ----
def pin_mha(E, seed=11):
    """No positional part: MLA equals textbook MHA with W_K = W_DKV W_UK.

    Page "Multi-Head Latent Attention (MLA)", sections "The construction"
    (W_K = W_L W_LK, W_V = W_L W_LV, W_Q = W_LQ W_LQQ) and "The RoPE problem"
    (without positional embeddings the factorisation is exact).  The MHA side
    is torch's scaled_dot_product_attention in fp64 on the CPU with a causal
    mask, over the full token sequence, last rows.
    """
    worst = 0.0
    for cfg in (TINY, MID):
        case = make_case(cfg, seed, history="x")
        W = dict(case.weights)
        W["W_QR"] = np.zeros_like(W["W_QR"])
        W["W_KR"] = np.zeros_like(W["W_KR"])
        Wd = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in W.items()}
        H = cfg.n_heads
        W_Q = torch.einsum("ml,lhd->mhd", Wd["W_DQ"], Wd["W_UQ"])
        W_K = torch.einsum("ml,lhd->mhd", Wd["W_DKV"], Wd["W_UK"])
        W_V = torch.einsum("ml,lhd->mhd", Wd["W_DKV"], Wd["W_UV"])
        for b in range(cfg.batch):
            X = torch.from_numpy(_tokens(case, b))
            Q = torch.einsum("tm,mhd->htd", X, W_Q)
            K = torch.einsum("tm,mhd->htd", X, W_K)
            V = torch.einsum("tm,mhd->htd", X, W_V)
            O = torch.nn.functional.scaled_dot_product_attention(
                Q[None], K[None], V[None], is_causal=True, scale=cfg.softmax_scale)[0]
            o_mha = O[:, -cfg.n_q:].transpose(0, 1).numpy()
            y_mha = torch.einsum("htd,hdm->tm", O, Wd["W_O"])[-cfg.n_q:].numpy()
            for hb in HEAD_BLOCKS:
                out = _run_decode(E, case, b, W, head_block=hb)
                worst = max(worst, _rel(out["y"], y_mha), _rel(out["o_h"], o_mha))
            # a subset of heads, in a scrambled order, in blocks of two
            hs = [H - 1, 0, H // 2]
            sub = _run_decode(E, case, b, W, heads=hs, head_block=2)
            worst = max(worst, _rel(sub["o_h"], o_mha[:, hs]))
    return worst


# ------------------------------------------------------------------ P2 ----
def pin_absorbed(E, A, seed=12):
    """Merged weights (W_UQ W_UK^T, W_UV W_O) give the expanded result.

    Page "Multi-Head Latent Attention (MLA)", section "Two merges are where
    the compute win comes from"; RoPE on, so the decoupled part is included.
    """
    worst = 0.0
    for cfg in (TINY, MID):
        case = make_case(cfg, seed, history="x")
        W = case.weights
        uqk, uvo = A.merged_weights(W)
        for b in range(cfg.batch):
            S = int(case.cached[b])
            out = _run_decode(E, case, b)
            c = np.concatenate([E.latent_rows(W, case.x_hist[b], np.arange(S), cfg.rope_base)[0], out["c_new"]])
            kp = np.concatenate([E.latent_rows(W, case.x_hist[b], np.arange(S), cfg.rope_base)[1], out["k_pe_new"]])
            pos = S + np.arange(cfg.n_q)
            q_lat, q_pe = A.query_latent(W, uqk, case.x_new[b], pos, cfg.rope_base)
            ab = A.attention(q_lat, q_pe, c, kp, pos, cfg.softmax_scale, uvo)
            worst = max(worst, _rel(ab["y"], out["y"]), _rel(ab["o_lat"], out["o_lat"]),
                        _rel(ab["lse"], out["lse"]), _rel(A.out_proj(ab["o_lat"], uvo), out["y"]))
    return worst


# ------------------------------------------------------------------ P3 ----
def pin_softmax(E, seed=13):
    """Rows of the attention pattern sum to one, are >= 0, and are exactly 0
    on masked (later) tokens (page "How DeepSeek Rewrote the Transformer",
    section 03, "Mask" and "Normalize")."""
    worst = 0.0
    case = make_case(MID, seed, history="x")
    W = case.weights
    # Prefill the whole sequence so every row has a different causal limit.
    X = _tokens(case, 0)
    T = X.shape[0]
    c, kp = E.latent_rows(W, X, np.arange(T), MID.rope_base)
    _, qn, qp = E.query(W, X, np.arange(T), MID.rope_base)
    out = E.attention(W, qn, qp, c, kp, np.arange(T), MID.softmax_scale, want_p=True)
    p = out["p"]
    worst = max(worst, float(np.abs(p.sum(axis=2) - 1.0).max()))
    worst = max(worst, float(max(0.0, -p.min())))
    later = np.arange(T)[None, :] > np.arange(T)[:, None]
    worst = max(worst, float(np.abs(p[np.broadcast_to(later[:, None, :], p.shape)]).max()))
    return worst


# ------------------------------------------------------------------ P4 ----
def pin_brute(E, seed=14):
    """Vectorised oracle vs pure-Python correctly rounded sums on the tiny config."""
    cfg = TINY.with_(n_q=2, cached=15)
    case = make_case(cfg, seed, history="x")
    Wl = {k: np.asarray(v, np.float64).tolist() for k, v in case.weights.items()}
    toks = _tokens(case, 0)
    bf = brute_mla.decode(Wl, toks.tolist(), cfg.n_q, cfg.rope_base, cfg.softmax_scale)
    worst = 0.0
    for hb in HEAD_BLOCKS:
        out = _run_decode(E, case, 0, head_block=hb)
        worst = max(worst, _rel(out["y"], bf["y"]), _rel(out["o_h"], bf["o_h"]), _rel(out["o_lat"], bf["o_lat"]),
                    _rel(out["p"], bf["p"]), _rel(out["lse"], bf["lse"]))
    # a subset of heads, in a scrambled order, in blocks of one and of two:
    # each head's outputs equal the brute force's for that head, and the
    # partial output projection is the subset's share of y
    H = cfg.n_heads
    hs = [H - 1, 1]
    o_ref = np.asarray(bf["o_h"])[:, hs]
    W_O = np.asarray(case.weights["W_O"], np.float64)
    y_part = sum(o_ref[:, i] @ W_O[h] for i, h in enumerate(hs))
    for hb in (1, 2):
        sub = _run_decode(E, case, 0, heads=hs, head_block=hb)
        worst = max(worst, _rel(sub["o_h"], o_ref), _rel(sub["o_lat"], np.asarray(bf["o_lat"])[:, hs]),
                    _rel(sub["p"], np.asarray(bf["p"])[:, hs]), _rel(sub["lse"], np.asarray(bf["lse"])[:, hs]),
                    _rel(sub["y_partial"], y_part))
    return worst


# ------------------------------------------------------------------ P5 ----
def pin_kvcache(E, seed=15):
    """Decoding the last token over cached rows equals the last row of full
    causal attention recomputed over every token (page "How DeepSeek Rewrote
    the Transformer", section 04)."""
    worst = 0.0
    case = make_case(MID.with_(n_q=1), seed, history="x")
    W = case.weights
    X = _tokens(case, 0)
    T = X.shape[0]
    c, kp = E.latent_rows(W, X, np.arange(T), MID.rope_base)
    _, qn, qp = E.query(W, X, np.arange(T), MID.rope_base)
    full = E.attention(W, qn, qp, c, kp, np.arange(T), MID.softmax_scale)
    for t in (1, T // 2, T - 1):
        dec = E.decode_step(W, MID.rope_base, MID.softmax_scale, X[t:t + 1], t, c[:t], kp[:t])
        worst = max(worst, _rel(dec["y"][0], full["y"][t]))
    return worst


# ------------------------------------------------------------------ P6 ----
def pin_rope(R, E, seed=16):
    """RoPE is a rotation (norm preserved, identity at position 0), equals
    multiplication of consecutive pairs by exp(i*pos*theta_j), and makes
    scores depend only on the position difference, so shifting every
    position leaves the output unchanged (page "Multi-Head Latent Attention
    (MLA)", section "The RoPE problem")."""
    rng = np.random.default_rng(seed)
    d, base = 16, 10000.0
    v = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 4097, 100000])
    r = R.apply(v, pos, base)
    worst = float(np.abs(np.linalg.norm(r, axis=1) - np.linalg.norm(v, axis=1)).max())
    worst = max(worst, float(np.abs(r[0] - v[0]).max()))
    z = v[:, 0::2] + 1j * v[:, 1::2]
    theta = base ** (-np.arange(d // 2) * 2.0 / d)
    zr = z * np.exp(1j * pos[:, None] * theta[None, :])
    worst = max(worst, float(np.abs(r[:, 0::2] - zr.real).max()), float(np.abs(r[:, 1::2] - zr.imag).max()))
    # relative-position property of the score
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    s1 = R.apply(q, 50, base) @ R.apply(k, 20, base)
    s2 = R.apply(q, 1030, base) @ R.apply(k, 1000, base)
    worst = max(worst, abs(s1 - s2) / abs(s1))
    # shifting every position of a whole decode step
    case = make_case(MID, seed, history="x")
    W = case.weights
    S = int(case.cached[0])
    outs = []
    for shift in (0, 977):
        c, kp = E.latent_rows(W, case.x_hist[0], shift + np.arange(S), MID.rope_base)
        cn, kn = E.latent_rows(W, case.x_new[0], shift + S + np.arange(MID.n_q), MID.rope_base)
        _, qn, qp = E.query(W, case.x_new[0], shift + S + np.arange(MID.n_q), MID.rope_base)
        outs.append(E.attention(W, qn, qp, np.concatenate([c, cn]), np.concatenate([kp, kn]),
                                S + np.arange(MID.n_q), MID.softmax_scale)["y"])
    worst = max(worst, _rel(outs[1], outs[0]))
    return worst


# ------------------------------------------------------------------ P8 ----
def pin_special(E, seed=18):
    """One visible key: p = 1 and the head output is that key's value.
    Identical rows: p = 1/L and the output is the shared value."""
    case = make_case(MID, seed, history="x")
    W = case.weights
    S = int(case.cached[0])
    c, kp = E.latent_rows(W, case.x_hist[0], np.arange(S), MID.rope_base)
    _, qn, qp = E.query(W, case.x_hist[0][:1], np.array([0]), MID.rope_base)
    out = E.attention(W, qn, qp, c, kp, np.array([0]), MID.softmax_scale, want_p=True)
    v0 = np.einsum("l,lhd->hd", c[0], np.asarray(W["W_UV"], np.float64))
    worst = max(float(np.abs(out["p"][0, :, 0] - 1.0).max()), _rel(out["o_h"][0], v0),
                _rel(out["o_lat"][0], np.broadcast_to(c[0], out["o_lat"][0].shape)))
    L = 9
    cc, kk = np.repeat(c[:1], L, 0), np.repeat(kp[:1], L, 0)
    _, qn, qp = E.query(W, case.x_new[0][:1], np.array([L - 1]), MID.rope_base)
    out = E.attention(W, qn, qp, cc, kk, np.array([L - 1]), MID.softmax_scale, want_p=True)
    # identical rows at different positions still differ through RoPE, so
    # use the no-RoPE weights for the uniform case
    W0 = dict(W)
    W0["W_QR"] = np.zeros_like(W["W_QR"])
    out = E.attention(W0, qn, qp * 0.0, cc, kk * 0.0, np.array([L - 1]), MID.softmax_scale, want_p=True)
    worst = max(worst, float(np.abs(out["p"][0] - 1.0 / L).max()))
    return worst


ALL_PINS = ("mha", "absorbed", "softmax", "brute", "kvcache", "rope", "special")


def run_all(E, A, R):
    return {
        "mha": pin_mha(E),
        "absorbed": pin_absorbed(E, A),
        "softmax": pin_softmax(E),
        "brute": pin_brute(E),
        "kvcache": pin_kvcache(E),
        "rope": pin_rope(R, E),
        "special": pin_special(E),
    }
