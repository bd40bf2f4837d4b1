"""E4M3 latent cache (codes plus one power-of-two scale per row) vs the CPU
oracle, through the C ABI (MI355X only).

  * mla_cache_store_rows quantises given fp32 rows: codes and scales are
    compared bit for bit with oracle.fp8.quantize_rows on the same rows
    (both sides take the rounding decisions on those fp32 values).
  * mla_compress_append computes its rows in fp32 and quantises them: each
    dequantised value lies within one code step of the oracle's fp64 row
    (half a step of rounding, plus the fp32 GEMM's distance from the fp64
    value, which can move a value across a rounding midpoint).
  * decode on E4M3 caches whose codes and scales are drawn directly
    (synthetic.make_e4m3_rows): the oracle attends over the dequantised
    rows (oracle.fp8.dequantize_rows), which the kernel reproduces exactly
    in bf16 (code * 2^k is a bf16 value), so the bar is the bf16 one
    (rel-L2 <= 1e-2, max-abs <= 3e-2) at the V2 contiguous, paged and
    long-context workloads and a causal multi-token chunk.
"""
import numpy as np
import pytest
import torch

import head_latent_attention_13_amd as mla
from oracle import absorbed as OA
from oracle import expanded as OE
from oracle import fp8
from synthetic import Case, config, make_case, make_e4m3_rows, make_x

from .gpu_common import DEV, Guarded, assert_close, dev, dims_of, i32, upload_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()


def note(msg):
    print(f"[gpu-step] {msg}", flush=True)


# ------------------------------------------------------------- caches ----
def e4_contiguous(cfg, seqs, s_max):
    """seqs: [(codes [S, R], k [S])] -> contiguous E4M3 cache."""
    B = len(seqs)
    pool = torch.zeros(B, s_max, cfg.row, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, s_max, dtype=torch.float32, device=DEV)
    for b, (c, k) in enumerate(seqs):
        n = len(c)
        if n:
            pool[b, :n] = torch.from_numpy(c).to(DEV)
            scales[b, :n] = torch.from_numpy(np.exp2(k.astype(np.float64)).astype(np.float32)).to(DEV)
    return mla.Cache(pool=pool, s_max=s_max, scales=scales), pool, scales


def e4_paged(cfg, seqs, table, n_pages, kv_len, poison=False):
    P = cfg.page_size
    pool = torch.full((n_pages, P, cfg.row), 0x7F if poison else 0, dtype=torch.uint8, device=DEV)
    scales = torch.full((n_pages, P), float("nan") if poison else 0.0, dtype=torch.float32, device=DEV)
    tbl = torch.from_numpy(table).to(DEV)
    for b, (c, k) in enumerate(seqs):
        npg = (int(kv_len[b]) + P - 1) // P
        tc = torch.zeros(npg * P, cfg.row, dtype=torch.uint8, device=DEV)
        ts = torch.zeros(npg * P, dtype=torch.float32, device=DEV)
        if poison:
            tc.fill_(0x7F)
            ts.fill_(float("nan"))
        n = len(c)
        tc[:n] = torch.from_numpy(c).to(DEV)
        ts[:n] = torch.from_numpy(np.exp2(k.astype(np.float64)).astype(np.float32)).to(DEV)
        pool[tbl[b, :npg].long()] = tc.view(npg, P, cfg.row)
        scales[tbl[b, :npg].long()] = ts.view(npg, P)
    cache = mla.Cache(pool=pool, page_table=tbl, page_size=P, n_pages=n_pages,
                      max_pages_per_seq=table.shape[1], scales=scales)
    return cache, pool, scales


def deq(cfg, seq):
    c, k = seq
    return fp8.dequantize_rows(c, np.exp2(k.astype(np.float64)))


def e4_case(idx, seed):
    """Workload idx with every row the decode sees drawn as E4M3 codes (the
    new tokens' own rows included): it attends over kv_len = cached + n_q
    rows, none of them appended by the library."""
    case = make_case(config(idx), seed, history="e4m3")
    return case, case.kv_len, case.e4m3


def oracle_e4(case, seqs, b, js=None, **kw):
    """Expanded oracle over the dequantised rows of sequence b (its new
    tokens' rows included); queries js of its new tokens."""
    cfg = case.cfg
    S = int(case.cached[b])
    js = np.arange(cfg.n_q) if js is None else np.asarray(js)
    rows = deq(cfg, seqs[b])
    _, qn, qp = OE.query(case.weights, case.x_new[b][js], S + js, cfg.rope_base)
    return OE.attention(case.weights, qn, qp, rows[:, :cfg.d_latent], rows[:, cfg.d_latent:], S + js,
                        cfg.softmax_scale, **kw)


def decode(layer, cfg, case, kv, cache):
    B, n_q = cfg.batch, cfg.n_q
    x = dev(case.x_new.reshape(B * n_q, cfg.d_model), cfg)
    o_lat = Guarded(B * n_q, cfg.n_heads, cfg.d_latent)
    lse = Guarded(B * n_q, cfg.n_heads)
    y = Guarded(B * n_q, cfg.d_model)
    layer.decode(x, i32(kv), B, n_q, cache, o_lat.t, lse.t)
    layer.out_proj(o_lat.t, B * n_q, y.t)
    torch.cuda.synchronize()
    o_lat.check("o_lat")
    lse.check("lse")
    y.check("y")
    return o_lat.t, lse.t, y.t


# ------------------------------------------------------- store / append ----
@pytest.mark.parametrize("paged", [False, True])
def test_store_rows_bit_exact(paged):
    cfg = config(1).with_(batch=6, cached=0, n_q=3, name="store")
    B, n_q, R = 6, 3, cfg.row
    rng = np.random.default_rng(31)
    rows = (rng.standard_normal((B * n_q, R)) * np.exp2(rng.uniform(-12, 12, (B * n_q, 1)))).astype(np.float32)
    rows[0] = 0.0                                      # scale 1, codes 0
    rows[1] = 0.0
    rows[1, 5] = np.float32(448.0 * 2.0 ** -3)        # amax exactly on a binade edge
    # normal fp32 values all below 448 * 2^-126: the scale exponent stops at -126
    rows[2] = (rng.uniform(2e-38, 5e-36, R) * rng.choice([-1.0, 1.0], R)).astype(np.float32)
    pos = np.array([0, 7, 40, 63, 1, 20], np.int64)
    s_max = 70
    dims = dims_of(cfg)
    ws = torch.zeros(mla.mla_workspace_size(dims, B, n_q), dtype=torch.uint8, device=DEV)
    if paged:
        P = 32
        n_pages = 3 * B + 5
        table = np.random.default_rng(32).permutation(n_pages)[:3 * B].reshape(B, 3).astype(np.int32)
        pool = torch.zeros(n_pages, P, R, dtype=torch.uint8, device=DEV)
        scales = torch.zeros(n_pages, P, dtype=torch.float32, device=DEV)
        cache = mla.Cache(pool=pool, page_table=i32(table), page_size=P, n_pages=n_pages, max_pages_per_seq=3,
                          scales=scales)
    else:
        pool = torch.zeros(B, s_max, R, dtype=torch.uint8, device=DEV)
        scales = torch.zeros(B, s_max, dtype=torch.float32, device=DEV)
        cache = mla.Cache(pool=pool, s_max=s_max, scales=scales)
    note(f"store rows e4m3 paged={paged}")
    mla.mla_cache_store_rows(dims, torch.from_numpy(rows).to(DEV), i32(pos), B, n_q, cache, ws)
    torch.cuda.synchronize()
    assert mla.mla_read_device_error(ws) == 0
    ref_codes, ref_scales = fp8.quantize_rows(rows)
    pool_h, sc_h = pool.cpu().numpy(), scales.cpu().numpy()
    for m in range(B * n_q):
        b, t = divmod(m, n_q)
        p = int(pos[b]) + t
        if paged:
            pg = int(table[b, p // 32])
            got_c, got_s = pool_h[pg, p % 32], sc_h[pg, p % 32]
        else:
            got_c, got_s = pool_h[b, p], sc_h[b, p]
        assert np.array_equal(got_c, ref_codes[m]), f"codes of row {m}"
        assert got_s == ref_scales[m], f"scale of row {m}: {got_s} vs {ref_scales[m]}"


def test_store_rows_bf16_and_position_errors():
    cfg = config(1).with_(batch=2, cached=0, n_q=2, name="store16")
    R = cfg.row
    rng = np.random.default_rng(33)
    rows = rng.standard_normal((4, R)).astype(np.float32)
    dims = dims_of(cfg)
    ws = torch.zeros(mla.mla_workspace_size(dims, 2, 2), dtype=torch.uint8, device=DEV)
    pool = torch.zeros(2, 10, R, dtype=torch.bfloat16, device=DEV)
    cache = mla.Cache(pool=pool, s_max=10)
    note("store rows bf16, second sequence past the cache")
    mla.mla_cache_store_rows(dims, torch.from_numpy(rows).to(DEV), i32([3, 9]), 2, 2, cache, ws)
    torch.cuda.synchronize()
    assert mla.mla_read_device_error(ws) & 1
    ref = torch.from_numpy(rows).to(torch.bfloat16)
    got = pool.cpu()
    assert torch.equal(got[0, 3:5], ref[0:2])
    assert torch.equal(got[1, 9], ref[2])       # position 9 fits, position 10 does not
    assert (got[1, :9] == 0).all()


@pytest.mark.parametrize("paged", [False, True])
def test_append_within_one_code_step(paged):
    base = make_case(config(1), 1)
    cfg = config(1).with_(batch=8, cached=0, n_q=1, name="append_e4")
    rng = np.random.default_rng(34)
    x = make_x(cfg, (8, cfg.d_model), rng)
    pos = rng.integers(0, 200, 8)
    layer = mla.MLALayer(dims_of(cfg), upload_weights(base), max_batch=8)
    if paged:
        P = cfg.page_size
        n_pages = 4 * 8 + 3
        table = rng.permutation(n_pages)[:32].reshape(8, 4).astype(np.int32)
        pool = torch.zeros(n_pages, P, cfg.row, dtype=torch.uint8, device=DEV)
        scales = torch.zeros(n_pages, P, dtype=torch.float32, device=DEV)
        cache = mla.Cache(pool=pool, page_table=i32(table), page_size=P, n_pages=n_pages, max_pages_per_seq=4,
                          scales=scales)
    else:
        pool = torch.zeros(8, 256, cfg.row, dtype=torch.uint8, device=DEV)
        scales = torch.zeros(8, 256, dtype=torch.float32, device=DEV)
        cache = mla.Cache(pool=pool, s_max=256, scales=scales)
    note(f"append e4m3 paged={paged}")
    layer.append(dev(x, cfg), i32(pos), 8, 1, cache)
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    c_ref, k_ref = OE.latent_rows(base.weights, x, pos, cfg.rope_base)
    ref = np.concatenate([c_ref, k_ref], axis=1)
    pool_h, sc_h = pool.cpu().numpy(), scales.cpu().numpy()
    for b in range(8):
        p = int(pos[b])
        if paged:
            pg = int(table[b, p // cfg.page_size])
            codes, s = pool_h[pg, p % cfg.page_size], float(sc_h[pg, p % cfg.page_size])
        else:
            codes, s = pool_h[b, p], float(sc_h[b, p])
        assert s > 0 and np.log2(s) == np.round(np.log2(s)), s
        got = fp8.decode(codes) * s
        a = np.abs(ref[b]) / s
        step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3)) * s
        assert np.all(np.abs(got - ref[b]) <= step), f"row {b}: {np.max(np.abs(got - ref[b]) / step)} steps"
        # the scale is the one the oracle picks for the fp64 row (up to a
        # binade edge within fp32 distance)
        k_ref = int(fp8.row_scale_exponents(ref[b][None].astype(np.float32))[0])
        assert abs(int(np.log2(s)) - k_ref) <= 1


# ------------------------------------------------------------- decode ----
def test_decode_e4m3_v2_contiguous():
    case, kv, seqs = e4_case(1, 41)
    cfg = case.cfg
    layer = mla.MLALayer(dims_of(cfg), upload_weights(case), max_batch=cfg.batch)
    cache, _, _ = e4_contiguous(cfg, seqs, int(kv.max()))
    note("e4m3 v2 contiguous: decode")
    o_lat, lse, y = decode(layer, cfg, case, kv, cache)
    for b in (0, 7, 15):
        ref = oracle_e4(case, seqs, b)
        assert_close(o_lat.cpu().numpy()[b], ref["o_lat"][0], cfg, f"e4m3 o_lat[b={b}]")
        assert_close(lse.cpu().numpy()[b], ref["lse"][0], cfg, f"e4m3 lse[b={b}]")
        assert_close(y.cpu().numpy()[b], ref["y"][0], cfg, f"e4m3 y[b={b}]")
    assert layer.device_error() == 0


def test_decode_e4m3_v2_paged_and_layout_independence():
    case, kv, seqs = e4_case(2, 42)
    cfg = case.cfg
    layer = mla.MLALayer(dims_of(cfg), upload_weights(case), max_batch=cfg.batch)
    cache, _, _ = e4_paged(cfg, seqs, case.page_table, case.n_pages, kv)
    note("e4m3 v2 paged: decode")
    o_lat, lse, y = decode(layer, cfg, case, kv, cache)
    order = np.argsort(kv)
    for b in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        ref = oracle_e4(case, seqs, b)
        assert_close(o_lat.cpu().numpy()[b], ref["o_lat"][0], cfg, f"e4m3 o_lat[b={b}, len={kv[b]}]")
        assert_close(lse.cpu().numpy()[b], ref["lse"][0], cfg, f"e4m3 lse[b={b}]")
        assert_close(y.cpu().numpy()[b], ref["y"][0], cfg, f"e4m3 y[b={b}]")
    note("e4m3 v2: contiguous copy and NaN-poisoned free slots")
    ccache, _, _ = e4_contiguous(cfg, seqs, int(kv.max()))
    o_c, l_c, y_c = decode(layer, cfg, case, kv, ccache)
    assert torch.equal(o_lat, o_c) and torch.equal(lse, l_c) and torch.equal(y, y_c)
    pcache, _, _ = e4_paged(cfg, seqs, case.page_table, case.n_pages, kv, poison=True)
    o_p, l_p, y_p = decode(layer, cfg, case, kv, pcache)
    assert torch.equal(o_lat, o_p) and torch.equal(lse, l_p) and torch.equal(y, y_p)
    assert layer.device_error() == 0


def test_decode_e4m3_v2_long_context():
    case, kv, seqs = e4_case(3, 43)
    cfg = case.cfg
    layer = mla.MLALayer(dims_of(cfg), upload_weights(case), max_batch=cfg.batch)
    cache, _, _ = e4_paged(cfg, seqs, case.page_table, case.n_pages, kv)
    note("e4m3 v2 long: decode")
    o_lat, lse, y = decode(layer, cfg, case, kv, cache)
    b = 1
    heads = [0, 31, 96, 127]
    ref = oracle_e4(case, seqs, b, heads=heads, want_y=False)
    assert_close(o_lat.cpu().numpy()[b][heads], ref["o_lat"][0], cfg, "e4m3 long o_lat (sampled heads)")
    assert_close(lse.cpu().numpy()[b][heads], ref["lse"][0], cfg, "e4m3 long lse (sampled heads)")
    W = case.weights
    uqk, uvo = OA.merged_weights(W)
    S = int(case.cached[b])
    rows = deq(cfg, seqs[b])
    q_lat, q_pe = OA.query_latent(W, uqk, case.x_new[b], np.array([S]), cfg.rope_base)
    ab = OA.attention(q_lat, q_pe, rows[:, :cfg.d_latent], rows[:, cfg.d_latent:], np.array([S]),
                      cfg.softmax_scale, uvo)
    assert_close(y.cpu().numpy()[b], ab["y"][0], cfg, "e4m3 long y")
    assert_close(o_lat.cpu().numpy()[b], ab["o_lat"][0], cfg, "e4m3 long o_lat (all heads, absorbed oracle)")


@pytest.mark.parametrize("lengths,n_q", [([1], 1), ([31, 33, 64], 1), ([300, 97], 48)])
def test_decode_e4m3_ragged_and_causal_chunk(lengths, n_q):
    base = make_case(config(1), 1)
    cfg = config(1).with_(batch=len(lengths), cached=0, n_q=n_q, name=f"e4edge{lengths}x{n_q}")
    rng = np.random.default_rng(5000 + sum(lengths) + n_q)
    cached = np.array(lengths, np.int64)
    x_new = make_x(cfg, (cfg.batch, n_q, cfg.d_model), rng)
    kv = cached + n_q
    seqs = make_e4m3_rows(cfg, kv, rng)
    case = Case(cfg=cfg, seed=0, weights=base.weights, cached=cached, x_new=x_new, e4m3=seqs)
    layer = mla.MLALayer(dims_of(cfg), upload_weights(base), max_batch=cfg.batch, max_nq=n_q)
    cache, _, _ = e4_contiguous(cfg, seqs, int(kv.max()))
    note(f"e4m3 edge {lengths} n_q={n_q}")
    o_lat, lse, y = decode(layer, cfg, case, kv, cache)
    o_lat = o_lat.view(cfg.batch, n_q, cfg.n_heads, cfg.d_latent).cpu().numpy()
    lse = lse.view(cfg.batch, n_q, cfg.n_heads).cpu().numpy()
    y = y.view(cfg.batch, n_q, cfg.d_model).cpu().numpy()
    for b in range(cfg.batch):
        ref = oracle_e4(case, seqs, b)
        assert_close(o_lat[b], ref["o_lat"], cfg, f"e4m3 o_lat[b={b}]")
        assert_close(lse[b], ref["lse"], cfg, f"e4m3 lse[b={b}]")
        assert_close(y[b], ref["y"], cfg, f"e4m3 y[b={b}]")
    assert layer.device_error() == 0
