"""mla_attention_noalloc (the entry point for callers that cannot allocate)
against mla_attention on the same inputs, through the C ABI (MI355X only).

Both run the same plan, split and merge kernels; with the same number of
split work-groups (up to 127 (sequence, head group) units at the V2 shape)
the outputs are bit-identical, and with fewer (the scratch caps the
partials) they agree within the bf16 bar of the parity tests.  The calls
come in a row on one scratch, each smaller than the one before, so stale
plan records or partials of an earlier call would show.
"""
import numpy as np
import pytest
import torch

import head_latent_attention_13_amd as mla
from synthetic import config

from .gpu_common import BF16_MAX_ABS, BF16_REL_L2, DEV, dims_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    mla.load()


def note(msg):
    print(f"[no-alloc] {msg}", flush=True)


CFG = config(1)
H, R, DL = CFG.n_heads, CFG.row, CFG.d_latent


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def contiguous(kv_len, seed):
    B, S = len(kv_len), max(kv_len)
    pool = (torch.randn(B, S, R, generator=_gen(seed), device=DEV) * 0.5).to(torch.bfloat16)
    return mla.Cache(pool=pool, s_max=S), pool


def paged(kv_len, seed, page=64):
    B = len(kv_len)
    npg = [(k + page - 1) // page for k in kv_len]
    n_pages = sum(npg) + 7
    pool = (torch.randn(n_pages, page, R, generator=_gen(seed), device=DEV) * 0.5).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_pages).astype(np.int32)
    table = np.full((B, max(npg)), -1, np.int32)
    o = 0
    for b in range(B):
        table[b, :npg[b]] = perm[o:o + npg[b]]
        o += npg[b]
    tbl = torch.from_numpy(table).to(DEV)
    return mla.Cache(pool=pool, page_table=tbl, page_size=page, n_pages=n_pages, max_pages_per_seq=table.shape[1]), pool


def both(kv_len, n_q, cache, seed, dev_err=None):
    """Outputs of mla_attention (own workspace) and mla_attention_noalloc."""
    B = len(kv_len)
    dims = dims_of(CFG)
    q = (torch.randn(B * n_q, H, R, generator=_gen(seed + 1), device=DEV) * 0.5).to(torch.bfloat16)
    kv = torch.tensor(kv_len, dtype=torch.int32, device=DEV)
    ws = torch.zeros(mla.mla_workspace_size(dims, B, n_q), dtype=torch.uint8, device=DEV)
    o_ref = torch.full((B * n_q, H, DL), float("nan"), device=DEV)
    l_ref = torch.full((B * n_q, H), float("nan"), device=DEV)
    mla.mla_attention(dims, q, kv, B, n_q, cache, o_ref, l_ref, ws)
    o = torch.full((B * n_q, H, DL), float("nan"), device=DEV)
    lse = torch.full((B * n_q, H), float("nan"), device=DEV)
    mla.mla_attention_noalloc(dims, q, kv, B, n_q, cache, o, lse, dev_err)
    torch.cuda.synchronize()
    assert mla.mla_read_device_error(ws) == 0
    return o, lse, o_ref, l_ref


def close(a, r, what):
    a, r = a.double().cpu(), r.double().cpu()
    assert torch.isfinite(a).all(), f"{what}: non-finite output"
    rel = float((a - r).norm() / r.norm())
    mabs = float((a - r).abs().max())
    note(f"{what}: rel-L2 {rel:.2e} max-abs {mabs:.2e}")
    assert rel <= BF16_REL_L2 and mabs <= BF16_MAX_ABS, (what, rel, mabs)


def test_two_calls_in_a_row_match_the_workspace_entry_point():
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    note("call 1: batch 16 x 4096 rows, contiguous")
    kv1 = [4096] * 16
    cache, _ = contiguous(kv1, 11)
    o, lse, o_ref, l_ref = both(kv1, 1, cache, 11, err)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "same split: bit-identical"
    close(o, o_ref, "call 1 o_lat")
    note("call 2: batch 5, ragged lengths, two query tokens, paged")
    kv2 = [2, 33, 700, 2048, 95]
    cache, _ = paged(kv2, 12)
    o, lse, o_ref, l_ref = both(kv2, 2, cache, 12, err)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "same split: bit-identical"
    close(o, o_ref, "call 2 o_lat")
    assert int(err.item()) == 0


def test_capped_split_many_sequences():
    # 150 units: the scratch holds the partials of fewer than one work-group
    # per CU, so the split differs from the workspace call's
    rng = np.random.default_rng(13)
    kv = [int(k) for k in rng.integers(1, 600, size=150)]
    note("150 sequences, paged, capped split")
    cache, _ = paged(kv, 13)
    o, lse, o_ref, l_ref = both(kv, 1, cache, 13)
    close(o, o_ref, "o_lat")
    close(lse, l_ref, "lse")
    note("then a smaller call on the same scratch")
    cache, _ = contiguous([300, 64], 14)
    o, lse, o_ref, l_ref = both([300, 64], 1, cache, 14)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_e4m3_cache_matches_the_workspace_entry_point():
    """An E4M3 latent cache (codes and per-row scales written by
    mla_cache_store_rows): the no-allocation entry point converts the same
    tiles as mla_attention and matches it bit for bit at the same split."""
    dims = dims_of(CFG)
    kv = [300, 1537, 64, 4097]
    B, S = len(kv), max(kv)
    rows = torch.randn(B * S, R, generator=_gen(71), device=DEV) * 0.5
    pool = torch.zeros(B, S, R, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, S, dtype=torch.float32, device=DEV)
    cache = mla.Cache(pool=pool, s_max=S, scales=scales)
    ws = torch.zeros(256, dtype=torch.uint8, device=DEV)
    note("E4M3 cache: 4 sequences, 64..4097 rows")
    mla.mla_cache_store_rows(dims, rows, torch.zeros(B, dtype=torch.int32, device=DEV), B, S, cache, ws)
    torch.cuda.synchronize()
    assert mla.mla_read_device_error(ws) == 0
    o, lse, o_ref, l_ref = both(kv, 1, cache, 72)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "same split: bit-identical"
    assert torch.isfinite(o).all()


def test_device_error_word_and_limits():
    dims = dims_of(CFG)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv = [100, 40]
    cache, _ = paged(kv, 15)
    cache.page_table[1, 0] = cache.n_pages + 3  # outside the pool: flagged, read as zeros
    q = torch.zeros(2, H, R, dtype=torch.bfloat16, device=DEV)
    o = torch.empty(2, H, DL, device=DEV)
    note("page id outside the pool")
    mla.mla_attention_noalloc(dims, q, torch.tensor(kv, dtype=torch.int32, device=DEV), 2, 1, cache, o, None, err)
    torch.cuda.synchronize()
    assert int(err.item()) & 2
    # beyond the scratch: refused before any launch
    with pytest.raises(mla.MLAError) as ei:
        big = torch.full((400,), 8, dtype=torch.int32, device=DEV)
        qq = torch.zeros(400, H, R, dtype=torch.bfloat16, device=DEV)
        oo = torch.empty(400, H, DL, device=DEV)
        mla.mla_attention_noalloc(dims, qq, big, 400, 1, contiguous([8] * 400, 16)[0], oo, None)
    assert "scratch" in str(ei.value)
