"""Factored weight form (q_lat[h] = (c_Q W_UQ[h]) W_UK[h]^T and
y = sum_h (o_lat[h] W_UV[h]) W_O[h] at run time) vs the CPU oracle, through
the C ABI (MI355X only).

The factored form computes the same function as the merged one (page
"Multi-Head Latent Attention (MLA)", "The construction" and "Two merges");
its extra roundings (c_Q W_UQ[h] and o_lat[h] W_UV[h] to dtype) stay inside
the same tolerances: rel-L2 <= 1e-2 and max-abs <= 3e-2 for bf16, 1e-5 for
fp32.  Large configurations are compared on sampled sequences, heads or
query tokens, each of which the oracle computes exactly.
"""
import functools

import numpy as np
import pytest
import torch

import head_latent_attention_13_amd as mla
from oracle import absorbed as OA
from oracle import expanded as OE
from synthetic import Case, config, make_case, make_rows, make_x

from .gpu_common import (DEV, assert_close, contiguous_cache, dev, dims_of, i32, paged_cache, run_step, unpack,
                         upload_weights)

pytestmark = pytest.mark.gpu
FORM = "factored"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()


@functools.lru_cache(maxsize=4)
def case_of(idx, history="rows", batch=None):
    cfg = config(idx)
    if batch is not None:
        cfg = cfg.with_batch(batch)
    return make_case(cfg, idx, history=history)


def oracle_seq(case, b, **kw):
    cfg = case.cfg
    rows_c, rows_k = case.rows[b][:, :cfg.d_latent], case.rows[b][:, cfg.d_latent:]
    return OE.decode_step(case.weights, cfg.rope_base, cfg.softmax_scale, case.x_new[b], int(case.cached[b]),
                          rows_c, rows_k, **kw)


def note(msg):
    print(f"[gpu-step] {msg}", flush=True)


def test_factored_tiny_f32_end_to_end_and_packing():
    case = case_of(0, history="x")
    cfg = case.cfg
    S = int(case.cached[0])
    note("factored tiny: pack")
    layer = mla.MLALayer(dims_of(cfg, FORM), upload_weights(case), max_batch=1, max_nq=max(S, 1))
    # the packed factors are the raw weights, element for element
    offs, sizes, total = mla.mla_absorbed_layout(layer.dims)
    buf = layer.absorbed.cpu().numpy()
    H, L, R = cfg.n_heads, cfg.d_latent, cfg.row
    W = case.weights

    def packed(K, N):
        return (-(-K // 4) * 4) * (-(-N // 16) * 16) * 4

    def take(at, K, N):
        return unpack(buf[at:at + packed(K, N)].view(np.float32), K, N, False), at + -(-packed(K, N) // 256) * 256

    uq, at = take(offs[2], cfg.d_q_latent, H * cfg.d_nope)
    qr, at = take(at, cfg.d_q_latent, H * cfg.d_rope)
    ukt, at = take(at, cfg.d_nope, H * L)
    uk, at = take(at, L, H * cfg.d_nope)
    assert at == offs[3]
    uv, at = take(offs[3], L, H * cfg.d_v)
    wo, at = take(at, H * cfg.d_v, cfg.d_model)
    assert at == total
    assert np.array_equal(uq, W["W_UQ"].reshape(cfg.d_q_latent, -1))
    assert np.array_equal(qr, W["W_QR"].reshape(cfg.d_q_latent, -1))
    assert np.array_equal(ukt.reshape(cfg.d_nope, H, L), W["W_UK"].transpose(2, 1, 0))
    assert np.array_equal(uk, W["W_UK"].reshape(L, -1))
    assert np.array_equal(uv, W["W_UV"].reshape(L, -1))
    assert np.array_equal(wo, W["W_O"].reshape(H * cfg.d_v, cfg.d_model))
    cache, pool = contiguous_cache(cfg, [np.zeros((0, R), np.float32)], S + cfg.n_q)
    layer.append(dev(case.x_hist[0], cfg), i32([0]), 1, S, cache)
    note("factored tiny: decode step")
    o_lat, lse, y = run_step(layer, cfg, case, cache)
    c_all, k_all = OE.latent_rows(W, case.x_hist[0], np.arange(S), cfg.rope_base)
    ref = OE.decode_step(W, cfg.rope_base, cfg.softmax_scale, case.x_new[0], S, c_all, k_all)
    assert_close(o_lat.cpu().numpy()[0], ref["o_lat"][0], cfg, "o_lat")
    assert_close(lse.cpu().numpy()[0], ref["lse"][0], cfg, "lse")
    assert_close(y.cpu().numpy()[0], ref["y"][0], cfg, "y")
    assert layer.device_error() == 0


def test_factored_v2_decode_contiguous_vs_merged():
    case = case_of(1)
    cfg = case.cfg
    note("factored v2 contiguous: pack + cache")
    layer = mla.MLALayer(dims_of(cfg, FORM), upload_weights(case), max_batch=cfg.batch)
    cache, _ = contiguous_cache(cfg, case.rows, int(case.cached.max()) + 1)
    note("factored v2 contiguous: decode step")
    o_lat, lse, y = run_step(layer, cfg, case, cache)
    for b in (0, 7, 15):
        ref = oracle_seq(case, b)
        assert_close(o_lat.cpu().numpy()[b], ref["o_lat"][0], cfg, f"o_lat[b={b}]")
        assert_close(lse.cpu().numpy()[b], ref["lse"][0], cfg, f"lse[b={b}]")
        assert_close(y.cpu().numpy()[b], ref["y"][0], cfg, f"y[b={b}]")
    # the merged form of the same layer agrees within the same bar
    note("factored v2 contiguous: merged form")
    merged = mla.MLALayer(dims_of(cfg, "merged"), upload_weights(case), max_batch=cfg.batch)
    mcache, _ = contiguous_cache(cfg, case.rows, int(case.cached.max()) + 1)
    o_m, l_m, y_m = run_step(merged, cfg, case, mcache)
    assert_close(o_lat.cpu().numpy(), o_m.cpu().numpy().astype(np.float64), cfg, "o_lat factored vs merged")
    assert_close(y.cpu().numpy(), y_m.cpu().numpy().astype(np.float64), cfg, "y factored vs merged")
    assert layer.device_error() == 0 and merged.device_error() == 0


def test_factored_v2_decode_paged():
    case = case_of(2)
    cfg = case.cfg
    kv = case.cached + 1
    note("factored v2 paged: pack + cache")
    layer = mla.MLALayer(dims_of(cfg, FORM), upload_weights(case), max_batch=cfg.batch)
    cache, _ = paged_cache(cfg, case.rows, case.page_table, case.n_pages, kv)
    note("factored v2 paged: decode step")
    o_lat, lse, y = run_step(layer, cfg, case, cache)
    order = np.argsort(case.cached)
    for b in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        ref = oracle_seq(case, b)
        assert_close(o_lat.cpu().numpy()[b], ref["o_lat"][0], cfg, f"o_lat[b={b}, len={kv[b]}]")
        assert_close(y.cpu().numpy()[b], ref["y"][0], cfg, f"y[b={b}]")
    assert layer.device_error() == 0


def test_factored_v3_chunked_prefill():
    case = case_of(4)
    cfg = case.cfg
    n_q = cfg.n_q
    note("factored v3 prefill: pack + cache")
    layer = mla.MLALayer(dims_of(cfg, FORM), upload_weights(case), max_batch=cfg.batch, max_nq=n_q)
    cache, _ = contiguous_cache(cfg, case.rows, int(case.cached.max()) + n_q)
    note("factored v3 prefill: chunk step")
    o_lat, lse, y = run_step(layer, cfg, case, cache)
    o_lat = o_lat.view(cfg.batch, n_q, cfg.n_heads, cfg.d_latent)
    y = y.view(cfg.batch, n_q, cfg.d_model)
    b = 0
    S = int(case.cached[b])
    js = np.array([0, 2, 700, 1023])
    W = case.weights
    xs = case.x_new[b]
    c_new, k_new = OE.latent_rows(W, xs, S + np.arange(n_q), cfg.rope_base)
    c = np.concatenate([case.rows[b][:, :cfg.d_latent], c_new])
    k = np.concatenate([case.rows[b][:, cfg.d_latent:], k_new])
    _, qn, qp = OE.query(W, xs[js], S + js, cfg.rope_base)
    ref = OE.attention(W, qn, qp, c, k, S + js, cfg.softmax_scale)
    assert_close(o_lat.cpu().numpy()[b][js], ref["o_lat"], cfg, "o_lat (sampled queries)")
    assert_close(y.cpu().numpy()[b][js], ref["y"], cfg, "y (sampled queries)")
    assert layer.device_error() == 0


@pytest.mark.parametrize("lengths,n_q", [
    ([0, 40], 5),             # 10 token rows: streaming GEMMs
    ([70], 33),               # 33 rows: 64-row tiles
    ([10, 50, 90, 130], 25),  # 100 rows: 128-row tiles, one row block
    ([3, 17, 40, 64, 90, 111, 150, 199], 25),  # 200 rows: two row blocks
])
def test_factored_edge_shapes(lengths, n_q):
    base = case_of(1)
    cfg = config(1).with_(batch=len(lengths), cached=0, n_q=n_q, name=f"fedge{lengths}x{n_q}")
    rng = np.random.default_rng(2000 + 7 * len(lengths) + n_q)
    cached = np.array(lengths, dtype=np.int64)
    case = Case(cfg=cfg, seed=22, weights=base.weights, cached=cached,
                x_new=make_x(cfg, (cfg.batch, n_q, cfg.d_model), rng), rows=make_rows(cfg, cached, rng))
    note(f"factored edge {lengths} n_q={n_q}")
    layer = mla.MLALayer(dims_of(cfg, FORM), upload_weights(case), max_batch=cfg.batch, max_nq=n_q)
    cache, _ = contiguous_cache(cfg, case.rows, int(case.cached.max()) + n_q)
    o_lat, lse, y = run_step(layer, cfg, case, cache)
    o_lat = o_lat.view(cfg.batch, n_q, cfg.n_heads, cfg.d_latent).cpu().numpy()
    y = y.view(cfg.batch, n_q, cfg.d_model).cpu().numpy()
    for b in range(cfg.batch):
        ref = oracle_seq(case, b)
        assert_close(o_lat[b], ref["o_lat"], cfg, f"o_lat[b={b}]")
        assert_close(y[b], ref["y"], cfg, f"y[b={b}]")
    assert layer.device_error() == 0


@functools.lru_cache(maxsize=1)
def _v2_merged_query_weight():
    return OA.merged_weights(case_of(1).weights)[0]


@pytest.mark.parametrize("batch,n_q", [(1, 1), (5, 1), (16, 1), (2, 8), (17, 1)])
def test_factored_query_projection(batch, n_q):
    """q = [c_Q W_UQ[h] W_UK[h]^T | RoPE(c_Q W_QR[h])] for every row and head
    against the oracle's absorbed query (merged W_UQ[h] W_UK[h]^T in fp64):
    up to 16 rows run as c_Q and one fused per-head launch, 17 rows through
    the separate products; sequences sit at different positions, and 2 x 8
    puts several queries of one sequence in a block."""
    base = case_of(1)
    cfg = base.cfg.with_(batch=batch, n_q=n_q, name=f"fq{batch}x{n_q}")
    rng = np.random.default_rng(900 + 10 * batch + n_q)
    x_new = make_x(cfg, (batch, n_q, cfg.d_model), rng)
    cached = rng.integers(0, 3000, batch)
    note(f"factored query projection {batch}x{n_q}")
    layer = mla.MLALayer(dims_of(cfg, FORM), upload_weights(base), max_batch=batch, max_nq=n_q)
    x = dev(x_new.reshape(batch * n_q, cfg.d_model), cfg)
    q = torch.empty(batch * n_q, cfg.n_heads, cfg.row, dtype=torch.bfloat16, device=DEV)
    layer.q_proj(x, i32(cached + n_q), batch, n_q, q)
    torch.cuda.synchronize()
    qg = q.float().cpu().numpy().reshape(batch, n_q, cfg.n_heads, cfg.row)
    uqk = _v2_merged_query_weight()
    for b in range(batch):
        pos = np.arange(cached[b], cached[b] + n_q)
        q_lat, q_pe = OA.query_latent(base.weights, uqk, x_new[b], pos, cfg.rope_base)
        assert_close(qg[b, :, :, :cfg.d_latent], q_lat, cfg, f"q latent part b={b}")
        assert_close(qg[b, :, :, cfg.d_latent:], q_pe, cfg, f"q rope part b={b}")


@pytest.mark.parametrize("form", ["factored", "merged"])
def test_decode_twelve_heads(form):
    """Twelve heads at the V2 widths: in the factored form the fused query
    kernel covers heads 0..11 of its 16 (the rest exit), in the merged form
    the tiled absorption builds 12 heads' products; the attention runs one
    partial head group.  o_lat, lse and y of every sequence against the
    oracle."""
    cfg = config(1).with_(n_heads=12, batch=3, cached=(700, 1300), name="heads12")
    case = make_case(cfg, seed=41)
    note(f"{form}, 12 heads: pack + cache")
    layer = mla.MLALayer(dims_of(cfg, form), upload_weights(case), max_batch=cfg.batch)
    cache, _ = contiguous_cache(cfg, case.rows, int(case.cached.max()) + 1)
    o_lat, lse, y = run_step(layer, cfg, case, cache)
    for b in range(cfg.batch):
        ref = oracle_seq(case, b)
        assert_close(o_lat.cpu().numpy()[b], ref["o_lat"][0], cfg, f"o_lat[b={b}]")
        assert_close(lse.cpu().numpy()[b], ref["lse"][0], cfg, f"lse[b={b}]")
        assert_close(y.cpu().numpy()[b], ref["y"][0], cfg, f"y[b={b}]")
    assert layer.device_error() == 0
