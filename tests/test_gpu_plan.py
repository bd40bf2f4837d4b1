"""The attention work plan's cuts, through the C ABI (MI355X only).

The plan kernel cuts the concatenated 32-key blocks of all streams (a stream
is one query row of one head group) into contiguous per-work-group ranges in
one of three ways (even ranges, stream-aligned chunks, or ranges of equal
estimated cost); streams cut by a range boundary are put back together by
the log-sum-exp merge (page "How DeepSeek Rewrote the Transformer",
section 03, "Normalize").  Each case below is a length mix chosen so that a
given cut is taken on a 256-CU device (checked first with a host model of
the plan's choice), and one mix has more streams than the plan keeps in
LDS.  mla_attention alone is compared with the oracle on sampled streams,
with the query of every checked row from the oracle's query path rounded to
bf16 (the interface's query type), at the bf16 bars.
"""
import numpy as np
import pytest
import torch

import head_latent_attention_13_amd as mla
from oracle import absorbed as OA
from synthetic import config, make_rows, make_weights, make_x, round_bf16

from .gpu_common import DEV, Guarded, assert_close, contiguous_cache, dims_of, i32

pytestmark = pytest.mark.gpu

TILE = 32        # keys per block
SEG_COST = 6     # the plan's cost of a segment, in blocks
LDS_STREAMS = 2048


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()


def note(msg):
    print(f"[gpu-step] {msg}", flush=True)


def plan_choice(kv, n_q, G):
    """Host model of which cut the plan takes (its cost comparison; integer
    arithmetic as on the device).  Returns (cut, streams staged in LDS)."""
    tiles = [(L - n_q + j + 1 + TILE - 1) // TILE for L in kv for j in range(n_q)]
    U = len(tiles)
    x = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int64)
    T = int(x[-1])
    xs = [int(x[u]) for u in range(U) if tiles[u] > 0]
    nz = len(xs)
    per0 = max(1, -(-T // G))
    hist = np.zeros(G, np.int64)
    for u in range(U):
        if tiles[u] > 0 and x[u] % per0:
            hist[x[u] // per0] += 1
    cost_even = per0 + SEG_COST * (1 + int(hist.max()))
    per = max(per0, -(-T // (G - nz))) if G > nz else 0
    cost_al = per + SEG_COST if per > 0 else None
    staged = U <= LDS_STREAMS
    best = min(cost_even, cost_al) if cost_al is not None else cost_even
    FT = T + SEG_COST * nz
    lower = FT // G + SEG_COST if G > 2 * nz else -(-FT // G)
    cost_bal = None
    if staged and G <= 1024 and nz > 0 and lower + SEG_COST // 2 <= best:
        gb, jb = [], []
        for w in range(G):
            t = w * FT // G
            j = max(i for i in range(nz) if xs[i] + SEG_COST * i <= t)
            x0, x1 = xs[j], (xs[j + 1] if j + 1 < nz else T)
            f_in = x0 + SEG_COST * (j + 1)
            gb.append(x0 if t < f_in else min(x1, x0 + (t - f_in)))
            jb.append(j)
        gb.append(T)
        jb.append(nz)
        cost_bal = 0
        for w in range(G):
            if gb[w + 1] > gb[w]:
                end_at_start = jb[w + 1] == nz or gb[w + 1] == xs[jb[w + 1]]
                j1 = jb[w + 1] - 1 if end_at_start else jb[w + 1]
                cost_bal = max(cost_bal, gb[w + 1] - gb[w] + SEG_COST * (j1 - jb[w] + 1))
    if cost_bal is not None and cost_bal <= best - SEG_COST // 2:
        return "balanced", staged
    if cost_al is not None and cost_al <= cost_even:
        return "aligned", staged
    return "even", staged


def lengths_random(n, lo, hi, seed):
    return np.random.default_rng(seed).integers(lo, hi, n).astype(np.int64)


CASES = {
    # 16 x 4096 keys: 128 blocks per stream, every stream starts on an even
    # range boundary
    "even": (np.full(16, 4096, np.int64), 1, "even", True, (0, 7, 15)),
    # 16 x 4097 keys: one more block per stream shifts every start inside a range
    "aligned": (np.full(16, 4097, np.int64), 1, "aligned", True, (0, 15)),
    # 128 sequences of 32..799 keys: more streams than half the work-groups
    "balanced": (lengths_random(128, 32, 800, 7), 1, "balanced", True, (0, 1, 63, 64, 127)),
    # 3 sequences x a 700-token causal chunk: 2100 streams, beyond the LDS records
    "many_streams": (np.array([2000, 737, 5700], np.int64), 700, "even", False, (0, 1, 2)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_plan_cut_matches_oracle(name):
    kv, n_q, want_cut, want_staged, checked = CASES[name]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    G = min(n_cu, 1024)
    got = plan_choice(kv, n_q, G)
    if G == 256:
        assert got == (want_cut, want_staged), (name, got)
    B = len(kv)
    cfg = config(1).with_(batch=B, n_q=n_q, cached=0, name=f"plan-{name}")
    H, R, L = cfg.n_heads, cfg.row, cfg.d_latent
    rng = np.random.default_rng(500 + len(name))
    W = make_weights(cfg, np.random.default_rng(501))
    uqk, _ = OA.merged_weights(W, want_uvo=False)
    rows = make_rows(cfg, kv, rng)
    x_new = make_x(cfg, (B, n_q, cfg.d_model), rng)
    js = np.unique(np.array([0, 1, 31, 32, n_q // 2, n_q - 2, n_q - 1]).clip(0, n_q - 1))
    cached = kv - n_q
    q = np.zeros((B, n_q, H, R), np.float32)
    qr = {}
    for b in checked:
        q_lat, q_pe = OA.query_latent(W, uqk, x_new[b][js], cached[b] + js, cfg.rope_base)
        q_lat, q_pe = round_bf16(q_lat.astype(np.float32)), round_bf16(q_pe.astype(np.float32))
        q[b, js, :, :L], q[b, js, :, L:] = q_lat, q_pe
        qr[b] = (q_lat.astype(np.float64), q_pe.astype(np.float64))
    cache, _ = contiguous_cache(cfg, rows, int(kv.max()))
    dims = dims_of(cfg)
    ws = torch.zeros(mla.mla_workspace_size(dims, B, n_q), dtype=torch.uint8, device=DEV)
    qd = torch.from_numpy(q.reshape(B * n_q, H, R)).to(DEV).to(torch.bfloat16)
    o_lat = Guarded(B * n_q, H, L)
    lse = Guarded(B * n_q, H)
    note(f"plan {name}: {B} sequences, n_q={n_q}, cut {got[0]}")
    mla.mla_attention(dims, qd, i32(kv), B, n_q, cache, o_lat.t, lse.t, ws)
    torch.cuda.synchronize()
    o_lat.check("o_lat")
    lse.check("lse")
    assert mla.mla_read_device_error(ws) == 0
    og = o_lat.t.view(B, n_q, H, L).cpu().numpy()
    lg = lse.t.view(B, n_q, H).cpu().numpy()
    for b in checked:
        ref = OA.attention(qr[b][0], qr[b][1], rows[b][:, :L], rows[b][:, L:], cached[b] + js, cfg.softmax_scale)
        assert_close(og[b][js], ref["o_lat"], cfg, f"o_lat[b={b}, len={kv[b]}]")
        assert_close(lg[b][js], ref["lse"], cfg, f"lse[b={b}]")
