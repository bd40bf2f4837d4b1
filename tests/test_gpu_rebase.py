"""Online-softmax rebase and multi-tile fp32 paths vs the CPU oracle, through
the C ABI (MI355X only).

The attention kernels keep a running maximum per head and rebase their
statistics (rescaling the partial output) when a later key block's maximum
exceeds it by more than a slack.  With i.i.d. cache rows that never happens
after the first block.  Here the history rows follow
``synthetic.quiet_then_loud``: the first 32 rows of every sequence are
scaled by 0.05 and the rest by 5..6, so every head's maximum jumps between
the first key block and the second, inside the work-group segment that
starts at a sequence's first block.  Each test first checks that
precondition on the CPU from the oracle's own scores (the softmax
definition of page "How DeepSeek Rewrote the Transformer", section 03,
"Normalize"), then compares the GPU outputs with the oracle.

Bars: rel-L2 <= 1e-2 and max-abs <= 3e-2 (bf16 cache, fp32 accumulation);
1e-5 for the fp32 configuration.
"""
import functools

import numpy as np
import pytest
import torch

import head_latent_attention_13_amd as mla
from synthetic import Case, config, make_case, make_rows, make_x, quiet_then_loud

from .gpu_common import (CHUNK_QUERIES, Guarded, assert_close, chunk_case, chunk_oracle, contiguous_cache, dev,
                         dims_of, i32, oracle_for, paged_cache, run_step, upload_weights)

pytestmark = pytest.mark.gpu

SLACK_LOG2 = 8.0   # the kernels' rebase slack (log2 units)
TILE = 32          # key rows per block


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()


def note(msg):
    print(f"[gpu-step] {msg}", flush=True)


def n_cu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def rebase_fraction(ref):
    """Fraction of heads, per query row, whose second key block's largest
    score exceeds the first block's by more than the slack (log2 units),
    from the oracle's probabilities and log-sum-exp (score = ln p + lse)."""
    p, lse = ref["p"], ref["lse"]
    with np.errstate(divide="ignore"):
        s = (np.log(p[..., :2 * TILE]) + lse[..., None]) / np.log(2.0)
    jump = s[..., TILE:2 * TILE].max(-1) - s[..., :TILE].max(-1)
    return (jump > SLACK_LOG2).mean(axis=-1)


def assert_rebases(ref, what):
    frac = rebase_fraction(ref)
    print(f"[rebase] {what}: heads rebasing after the first key block per query: min {frac.min():.3f}", flush=True)
    assert (frac > 0.5).all(), f"{what}: the inputs do not force a rebase in every stream ({frac})"


def assert_first_segment_spans_two_blocks(kv_len, n_q, n_hg=1):
    """The attention plan gives each work-group ceil(T / G) key blocks or more
    (T blocks in all); with at least two per work-group the segment that
    starts at a stream's first block also holds its second."""
    T = sum(n_hg * sum((int(L) - n_q + j + 1 + TILE - 1) // TILE for j in range(n_q)) for L in kv_len)
    assert (T + n_cu() - 1) // n_cu() >= 2, T


# ------------------------------------------------------------- bf16 ----
def test_rebase_v2_contiguous():
    case = make_case(config(1), 101, amplitude=quiet_then_loud)
    cfg = case.cfg
    assert_first_segment_spans_two_blocks(case.cached + 1, 1)
    layer = mla.MLALayer(dims_of(cfg), upload_weights(case), max_batch=cfg.batch)
    cache, pool = contiguous_cache(cfg, case.rows, int(case.cached.max()) + 1)
    before = pool.clone()
    note("rebase v2 contiguous: decode step")
    o_lat, lse, y = run_step(layer, cfg, case, cache)
    # the append wrote exactly one row per sequence
    changed = (pool.view(torch.int16) != before.view(torch.int16)).any(-1).cpu().numpy()
    for b in range(cfg.batch):
        assert set(np.flatnonzero(changed[b])) <= {int(case.cached[b])}, b
    for b in (0, 9, 15):
        ref = oracle_for(case, b, want_p=True)
        assert_rebases(ref, f"v2 contiguous b={b}")
        assert_close(o_lat.cpu().numpy()[b], ref["o_lat"][0], cfg, f"o_lat[b={b}]")
        assert_close(lse.cpu().numpy()[b], ref["lse"][0], cfg, f"lse[b={b}]")
        assert_close(y.cpu().numpy()[b], ref["y"][0], cfg, f"y[b={b}]")
    assert layer.device_error() == 0


def test_rebase_v2_paged():
    case = make_case(config(2), 102, amplitude=quiet_then_loud)
    cfg = case.cfg
    kv = case.cached + 1
    assert_first_segment_spans_two_blocks(kv, 1)
    layer = mla.MLALayer(dims_of(cfg), upload_weights(case), max_batch=cfg.batch)
    cache, pool = paged_cache(cfg, case.rows, case.page_table, case.n_pages, kv)
    before = pool.clone()
    note("rebase v2 paged: decode step")
    o_lat, lse, y = run_step(layer, cfg, case, cache)
    # the append wrote exactly the slot of each sequence's new token
    changed = (pool.view(torch.int16) != before.view(torch.int16)).any(-1).cpu().numpy()
    P = cfg.page_size
    want = {(int(case.page_table[b, int(case.cached[b]) // P]), int(case.cached[b]) % P) for b in range(cfg.batch)}
    assert set(zip(*np.nonzero(changed))) <= want
    order = np.argsort(case.cached)
    for b in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        ref = oracle_for(case, b, want_p=True)
        assert_rebases(ref, f"v2 paged b={b}")
        assert_close(o_lat.cpu().numpy()[b], ref["o_lat"][0], cfg, f"o_lat[b={b}, len={kv[b]}]")
        assert_close(lse.cpu().numpy()[b], ref["lse"][0], cfg, f"lse[b={b}]")
        assert_close(y.cpu().numpy()[b], ref["y"][0], cfg, f"y[b={b}]")
    assert layer.device_error() == 0


def test_rebase_v3_chunk_absorbed():
    case = chunk_case(104, True)
    cfg = case.cfg
    n_q = cfg.n_q
    layer = mla.MLALayer(dims_of(cfg), upload_weights(case), max_batch=cfg.batch, max_nq=n_q)
    cache, _ = contiguous_cache(cfg, case.rows, int(case.cached.max()) + n_q)
    note("rebase v3 chunk (absorbed): step")
    o_lat, lse, y = run_step(layer, cfg, case, cache)
    o_lat = o_lat.view(cfg.batch, n_q, cfg.n_heads, cfg.d_latent).cpu().numpy()
    lse = lse.view(cfg.batch, n_q, cfg.n_heads).cpu().numpy()
    y = y.view(cfg.batch, n_q, cfg.d_model).cpu().numpy()
    for b in range(cfg.batch):
        js = CHUNK_QUERIES
        assert_rebases(oracle_for(case, b, js[:8], want_p=True, want_y=False), f"v3 chunk b={b}")
        ref = chunk_oracle(104, True, b)
        assert_close(o_lat[b][js], ref["o_lat"], cfg, f"o_lat[b={b}] ({len(js)} queries)")
        assert_close(lse[b][js], ref["lse"], cfg, f"lse[b={b}]")
        assert_close(y[b][js], ref["y"], cfg, f"y[b={b}]")
    assert layer.device_error() == 0


def test_rebase_v3_chunk_expanded_prefill():
    case = chunk_case(104, True)
    cfg = case.cfg
    n_q, B = cfg.n_q, cfg.batch
    layer = mla.MLALayer(dims_of(cfg, "factored"), upload_weights(case), max_batch=B, max_nq=n_q)
    cache, _ = contiguous_cache(cfg, case.rows, int(case.cached.max()) + n_q)
    x = dev(case.x_new.reshape(B * n_q, cfg.d_model), cfg)
    layer.append(x, i32(case.cached), B, n_q, cache)
    y = Guarded(B * n_q, cfg.d_model)
    lse = Guarded(B * n_q, cfg.n_heads)
    note("rebase v3 chunk (expanded prefill)")
    layer.prefill_expanded(x, i32(case.cached + n_q), B, n_q, cache, y.t, lse.t)
    torch.cuda.synchronize()
    y.check("y")
    lse.check("lse")
    yy = y.t.view(B, n_q, cfg.d_model).cpu().numpy()
    ll = lse.t.view(B, n_q, cfg.n_heads).cpu().numpy()
    for b in range(B):
        js = CHUNK_QUERIES
        assert_rebases(oracle_for(case, b, js[:8], want_p=True, want_y=False), f"v3 prefill b={b}")
        ref = chunk_oracle(104, True, b)
        assert_close(yy[b][js], ref["y"], cfg, f"y[b={b}] ({len(js)} queries)")
        assert_close(ll[b][js], ref["lse"], cfg, f"lse[b={b}]")
    assert layer.prefill_error() == 0


# ------------------------------------------------------------- fp32 ----
@pytest.mark.parametrize("lengths,n_q,loud", [
    ([300, 2047, 6001], 1, False),   # many key blocks per stream, streams cut over work-groups and merged
    ([300, 2047, 6001], 1, True),    # the same with a rebase after the first block
    ([300, 1000, 2000], 5, False),   # five query rows per sequence (causal inside the chunk)
    ([300, 1000, 2000], 5, True),
])
def test_f32_multi_block(lengths, n_q, loud):
    """The fp32 configuration's kernels beyond one key block: the multi-block
    loop, split partials and their merge, and the rebase."""
    cfg = config(0).with_(batch=len(lengths), cached=0, n_q=n_q, name=f"f32{lengths}x{n_q}")
    rng = np.random.default_rng(500 + n_q + 2 * loud)
    cached = np.array(lengths, dtype=np.int64)
    # the fp32 configuration's weights (variance 1/fan-in) give scores with a
    # spread of about 0.017 log2 units; these amplitudes make the second key
    # block's maximum exceed the first's by more than the slack
    amp = functools.partial(quiet_then_loud, lo=400.0, hi=480.0) if loud else None
    case = Case(cfg=cfg, seed=25, weights=make_case(config(0), 0).weights, cached=cached,
                x_new=make_x(cfg, (cfg.batch, n_q, cfg.d_model), rng), rows=make_rows(cfg, cached, rng, amp))
    if n_q > 1 or loud:
        assert_first_segment_spans_two_blocks(cached + n_q, n_q)
    note(f"f32 multi-block {lengths} n_q={n_q} loud={loud}")
    layer = mla.MLALayer(dims_of(cfg), upload_weights(case), max_batch=cfg.batch, max_nq=n_q)
    cache, _ = contiguous_cache(cfg, case.rows, int(case.cached.max()) + n_q)
    o_lat, lse, y = run_step(layer, cfg, case, cache)
    o_lat = o_lat.view(cfg.batch, n_q, cfg.n_heads, cfg.d_latent).cpu().numpy()
    lse = lse.view(cfg.batch, n_q, cfg.n_heads).cpu().numpy()
    y = y.view(cfg.batch, n_q, cfg.d_model).cpu().numpy()
    for b in range(cfg.batch):
        ref = oracle_for(case, b, want_p=loud)
        if loud:
            assert_rebases(ref, f"f32 b={b}")
        assert_close(o_lat[b], ref["o_lat"], cfg, f"o_lat[b={b}]")
        assert_close(lse[b], ref["lse"], cfg, f"lse[b={b}]")
        assert_close(y[b], ref["y"], cfg, f"y[b={b}]")
    assert layer.device_error() == 0
