"""Pure-Python scalar MLA, written from the definition with math.fsum.

Used only to pin the vectorized fp64 oracle on the tiny config: every sum is
correctly rounded (math.fsum) and every index is spelled out, so a
transposed operand, a wrong head index or a dropped term in the oracle's
einsums shows up as a disagreement.  It shares no code with ``oracle/``.

Definition followed: cache c_i = x_i W_DKV and k_pe_i = RoPE_i(x_i W_KR);
query c_Q = x W_DQ, q_nope_h = c_Q W_UQ[h], q_pe_h = RoPE(c_Q W_QR[h]);
keys k_{h,i} = [c_i W_UK[h] ‖ k_pe_i], values v_{h,i} = c_i W_UV[h];
scaled causal softmax; heads combined through W_O (pages "Latent Space
Strikes Again", "The Core Idea"; "Multi-Head Latent Attention (MLA)", "The
construction" and "The RoPE problem"; "How DeepSeek Rewrote the
Transformer", section 03).
"""
import math


def _rot(vec, pos, base):
    d = len(vec)
    out = [0.0] * d
    for j in range(d // 2):
        ang = pos * base ** (-(2.0 * j) / d)
        a, b = vec[2 * j], vec[2 * j + 1]
        ca, sa = math.cos(ang), math.sin(ang)
        out[2 * j] = math.fsum([a * ca, -b * sa])
        out[2 * j + 1] = math.fsum([a * sa, b * ca])
    return out


def _vecmat(v, M, col):
    """sum_k v[k] * M(k, col) with M given as a callable."""
    return math.fsum(v[k] * M(k, col) for k in range(len(v)))


def decode(W, tokens, n_new, base, scale):
    """W: dict of nested lists; tokens: list of d_model lists at positions 0..T-1.

    The last ``n_new`` tokens are queries (causal).  Returns dict with y
    [n_new][d_model], o_h [n_new][H][d_v], o_lat [n_new][H][d_L],
    p [n_new][H][T] and lse [n_new][H] (natural log of the softmax
    denominator of the scaled scores).
    """
    T = len(tokens)
    d_model = len(tokens[0])
    d_L = len(W["W_DKV"][0])
    d_rope = len(W["W_KR"][0])
    d_LQ = len(W["W_DQ"][0])
    H = len(W["W_UQ"][0])
    d_nope = len(W["W_UQ"][0][0])
    d_v = len(W["W_UV"][0][0])

    c = [[_vecmat(tokens[i], lambda k, l: W["W_DKV"][k][l], l) for l in range(d_L)] for i in range(T)]
    kr = [[_vecmat(tokens[i], lambda k, r: W["W_KR"][k][r], r) for r in range(d_rope)] for i in range(T)]
    k_pe = [_rot(kr[i], i, base) for i in range(T)]

    res = {"y": [], "o_h": [], "o_lat": [], "p": [], "lse": []}
    for t in range(T - n_new, T):
        x = tokens[t]
        cq = [_vecmat(x, lambda k, l: W["W_DQ"][k][l], l) for l in range(d_LQ)]
        y = [[] for _ in range(d_model)]
        o_all, ol_all, p_all, lse_all = [], [], [], []
        for h in range(H):
            qn = [math.fsum(cq[l] * W["W_UQ"][l][h][d] for l in range(d_LQ)) for d in range(d_nope)]
            qr = [math.fsum(cq[l] * W["W_QR"][l][h][r] for l in range(d_LQ)) for r in range(d_rope)]
            qp = _rot(qr, t, base)
            scores = []
            for i in range(t + 1):
                kn = [math.fsum(c[i][l] * W["W_UK"][l][h][d] for l in range(d_L)) for d in range(d_nope)]
                dot = math.fsum([qn[d] * kn[d] for d in range(d_nope)] + [qp[r] * k_pe[i][r] for r in range(d_rope)])
                scores.append(dot * scale)
            mx = max(scores)
            e = [math.exp(s - mx) for s in scores]
            den = math.fsum(e)
            p = [v / den for v in e] + [0.0] * (T - t - 1)
            vals = [[math.fsum(c[i][l] * W["W_UV"][l][h][d] for l in range(d_L)) for d in range(d_v)]
                    for i in range(t + 1)]
            o = [math.fsum(p[i] * vals[i][d] for i in range(t + 1)) for d in range(d_v)]
            ol = [math.fsum(p[i] * c[i][l] for i in range(t + 1)) for l in range(d_L)]
            for mcol in range(d_model):
                y[mcol].extend(o[d] * W["W_O"][h][d][mcol] for d in range(d_v))
            o_all.append(o)
            ol_all.append(ol)
            p_all.append(p)
            lse_all.append(mx + math.log(den))
        res["y"].append([math.fsum(terms) for terms in y])
        res["o_h"].append(o_all)
        res["o_lat"].append(ol_all)
        res["p"].append(p_all)
        res["lse"].append(lse_all)
    return res
