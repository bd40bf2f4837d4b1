"""Expanded-form chunked prefill (mla_prefill_expanded) vs the CPU oracle,
through the C ABI (MI355X only).

The expanded form up-projects every cached latent to per-head keys and
values and runs causal attention per head (page "How DeepSeek Rewrote the
Transformer", sections 03-04); the oracle's ``expanded`` module is that
definition in fp64.  Bar: rel-L2 <= 1e-2 and max-abs <= 3e-2 (bf16 cache,
fp32 accumulation).  The V3 chunk is compared on sampled query tokens, each
of which the oracle computes exactly, and against the absorbed-form GPU path
on every token.
"""
import numpy as np
import pytest
import torch

import head_latent_attention_13_amd as mla
from oracle import expanded as OE
from synthetic import Case, config, make_case, make_rows, make_x

from .gpu_common import (CHUNK_QUERIES, DEV, assert_close, chunk_case, chunk_oracle, contiguous_cache, dev, dims_of,
                         i32, run_step, upload_weights)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()


def note(msg):
    print(f"[gpu-step] {msg}", flush=True)


def prefill(layer, cfg, case, cache):
    """append the chunk, then the expanded prefill of it: y and lse."""
    B, n_q = cfg.batch, cfg.n_q
    x = dev(case.x_new.reshape(B * n_q, cfg.d_model), cfg)
    layer.append(x, i32(case.cached), B, n_q, cache)
    y = torch.empty(B * n_q, cfg.d_model, dtype=torch.float32, device=DEV)
    lse = torch.empty(B * n_q, cfg.n_heads, dtype=torch.float32, device=DEV)
    layer.prefill_expanded(x, i32(case.cached + n_q), B, n_q, cache, y, lse)
    torch.cuda.synchronize()
    return y, lse


def test_prefill_v3_chunk_sampled_and_vs_absorbed():
    case = chunk_case(4, False)
    cfg = case.cfg
    n_q = cfg.n_q
    note("prefill v3: pack + cache")
    layer = mla.MLALayer(dims_of(cfg, "factored"), upload_weights(case), max_batch=cfg.batch, max_nq=n_q)
    cache, _ = contiguous_cache(cfg, case.rows, int(case.cached.max()) + n_q)
    note("prefill v3: expanded chunk")
    y, lse = prefill(layer, cfg, case, cache)
    y = y.view(cfg.batch, n_q, cfg.d_model).cpu().numpy()
    lse = lse.view(cfg.batch, n_q, cfg.n_heads).cpu().numpy()
    js = CHUNK_QUERIES
    for b in range(cfg.batch):
        ref = chunk_oracle(4, False, b)
        assert_close(y[b][js], ref["y"], cfg, f"y[b={b}] ({len(js)} queries)")
        assert_close(lse[b][js], ref["lse"], cfg, f"lse[b={b}]")
    # the absorbed form of the same layer on every token
    note("prefill v3: absorbed form")
    _, lse_a, y_a = run_step(layer, cfg, case, cache, do_append=False)
    assert_close(y.reshape(-1, cfg.d_model), y_a.cpu().numpy().astype(np.float64), cfg, "y expanded vs absorbed")
    assert_close(lse.reshape(-1, cfg.n_heads), lse_a.cpu().numpy().astype(np.float64), cfg, "lse expanded vs absorbed")
    assert layer.prefill_error() == 0 and layer.device_error() == 0


@pytest.mark.parametrize("lengths,n_q", [
    ([0], 1),                 # one query, one key
    ([0, 40], 5),
    ([70], 33),
    ([3, 300], 130),          # two query blocks, the second partial
    ([100, 0, 37], 64),
])
def test_prefill_edge_shapes(lengths, n_q):
    base = make_case(config(1), 1)
    cfg = config(1).with_(batch=len(lengths), cached=0, n_q=n_q, name=f"pedge{lengths}x{n_q}")
    rng = np.random.default_rng(3000 + 7 * len(lengths) + n_q)
    cached = np.array(lengths, dtype=np.int64)
    case = Case(cfg=cfg, seed=23, weights=base.weights, cached=cached,
                x_new=make_x(cfg, (cfg.batch, n_q, cfg.d_model), rng), rows=make_rows(cfg, cached, rng))
    note(f"prefill edge {lengths} n_q={n_q}")
    layer = mla.MLALayer(dims_of(cfg, "factored"), upload_weights(case), max_batch=cfg.batch, max_nq=n_q)
    cache, _ = contiguous_cache(cfg, case.rows, int(case.cached.max()) + n_q)
    y, lse = prefill(layer, cfg, case, cache)
    y = y.view(cfg.batch, n_q, cfg.d_model).cpu().numpy()
    lse = lse.view(cfg.batch, n_q, cfg.n_heads).cpu().numpy()
    for b in range(cfg.batch):
        rows_c, rows_k = case.rows[b][:, :cfg.d_latent], case.rows[b][:, cfg.d_latent:]
        ref = OE.decode_step(case.weights, cfg.rope_base, cfg.softmax_scale, case.x_new[b], int(case.cached[b]),
                             rows_c, rows_k)
        assert_close(y[b], ref["y"], cfg, f"y[b={b}]")
        assert_close(lse[b], ref["lse"], cfg, f"lse[b={b}]")
    assert layer.prefill_error() == 0


def test_prefill_bad_length_is_flagged_and_contained():
    base = make_case(config(1), 1)
    cfg = config(1).with_(batch=2, cached=0, n_q=8, name="pbad")
    rng = np.random.default_rng(77)
    cached = np.array([20, 30], dtype=np.int64)
    case = Case(cfg=cfg, seed=24, weights=base.weights, cached=cached,
                x_new=make_x(cfg, (2, 8, cfg.d_model), rng), rows=make_rows(cfg, cached, rng))
    layer = mla.MLALayer(dims_of(cfg, "factored"), upload_weights(case), max_batch=2, max_nq=8)
    s_max = 40
    cache, _ = contiguous_cache(cfg, case.rows, s_max)
    x = dev(case.x_new.reshape(16, cfg.d_model), cfg)
    layer.append(x, i32(cached), 2, 8, cache)
    y = torch.empty(16, cfg.d_model, dtype=torch.float32, device=DEV)
    note("prefill: kv_len beyond the cache")
    layer.prefill_expanded(x, i32([28, s_max + 5]), 2, 8, cache, y, None)
    torch.cuda.synchronize()
    assert layer.prefill_error() & 4
    yy = y.view(2, 8, cfg.d_model).cpu().numpy()
    assert np.isnan(yy[1]).all()
    ref = OE.decode_step(case.weights, cfg.rope_base, cfg.softmax_scale, case.x_new[0], 20,
                         case.rows[0][:, :cfg.d_latent], case.rows[0][:, cfg.d_latent:])
    assert_close(yy[0], ref["y"], cfg, "y next to a bad sequence")


def test_prefill_kv_gemms_stop_at_kv_len():
    """A cache much longer than the sequences: the per-head key / value
    up-projections cover only the slots below kv_len (row blocks past every
    length exit at once), the result still matches the oracle, and the
    slots past the lengths (NaN here) are never read."""
    base = make_case(config(1), 1)
    n_q, s_max = 64, 2048
    cfg = config(1).with_(batch=2, cached=0, n_q=n_q, name="pkvlen")
    rng = np.random.default_rng(4242)
    cached = np.array([100, 236], dtype=np.int64)
    case = Case(cfg=cfg, seed=25, weights=base.weights, cached=cached,
                x_new=make_x(cfg, (2, n_q, cfg.d_model), rng), rows=make_rows(cfg, cached, rng))
    layer = mla.MLALayer(dims_of(cfg, "factored"), upload_weights(case), max_batch=2, max_nq=n_q)
    pool = torch.full((2, s_max, cfg.row), float("nan"), dtype=torch.bfloat16, device=DEV)
    for b, r in enumerate(case.rows):
        pool[b, :len(r)] = dev(r, cfg)
    cache = mla.Cache(pool=pool, s_max=s_max)
    need = mla.mla_prefill_workspace_size(layer.dims, 2, n_q, s_max)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)
    ws[:256] = 0  # the device error word
    layer.pf_workspace = ws
    note("prefill: kv_len far below s_max")
    y, lse = prefill(layer, cfg, case, cache)
    assert layer.prefill_error() == 0
    y = y.view(2, n_q, cfg.d_model).cpu().numpy()
    lse = lse.view(2, n_q, cfg.n_heads).cpu().numpy()
    for b in range(2):
        ref = OE.decode_step(case.weights, cfg.rope_base, cfg.softmax_scale, case.x_new[b], int(cached[b]),
                             case.rows[b][:, :cfg.d_latent], case.rows[b][:, cfg.d_latent:])
        assert_close(y[b], ref["y"], cfg, f"y[b={b}]")
        assert_close(lse[b], ref["lse"], cfg, f"lse[b={b}]")
    # keys and values of all 2 x 2048 slots would fill ~268 MB of the
    # workspace; only the row blocks holding slots below kv_len are written
    untouched = float((ws == 0x5A).float().mean())
    assert untouched > 0.5, f"only {untouched:.2f} of the workspace left unwritten"
