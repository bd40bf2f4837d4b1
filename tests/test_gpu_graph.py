"""A whole decode step (append, q_proj, attention, out_proj) captured into a
HIP graph and replayed, against the same calls run eagerly, through the C
ABI (MI355X only): the same kernels on the same inputs, so the appended
rows, o_lat and y must agree bit for bit on every replay, with eager work
and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import head_latent_attention_13_amd as mla
from synthetic import config, make_case

from .gpu_common import DEV, dev, dims_of, i32, paged_cache, upload_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    mla.load()


@pytest.mark.parametrize("n_q", [1, 24])
def test_graph_replay_matches_eager(n_q):
    cfg = config(2).with_(batch=6, cached=(100, 900), n_q=n_q)
    case = make_case(cfg, seed=31)
    B, R, H = cfg.batch, cfg.row, cfg.n_heads
    M = B * n_q
    print(f"[graph] V2 paged shape, B={B}, n_q={n_q}", flush=True)
    layer = mla.MLALayer(dims_of(cfg), upload_weights(case), max_batch=B, max_nq=n_q)
    x = dev(case.x_new.reshape(M, cfg.d_model), cfg)
    pos, kv = i32(case.cached), i32(case.cached + n_q)
    cache, pool = paged_cache(cfg, case.rows, case.page_table, case.n_pages, case.cached + n_q)
    q = torch.empty(M, H, R, dtype=torch.bfloat16, device=DEV)
    o_lat = torch.empty(M, H, cfg.d_latent, dtype=torch.float32, device=DEV)
    y = torch.empty(M, cfg.d_model, dtype=torch.float32, device=DEV)

    def step():
        layer.append(x, pos, B, n_q, cache)
        layer.q_proj(x, kv, B, n_q, q)
        layer.attention(q, kv, B, n_q, cache, o_lat)
        layer.out_proj(o_lat, M, y)

    step()
    torch.cuda.synchronize()
    ref = (pool.clone(), o_lat.clone(), y.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        o_lat.zero_()
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("cache", "o_lat", "y"), ref, (pool, o_lat, y)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
        step()  # eager work between the replays
        torch.cuda.synchronize()
    assert layer.device_error() == 0
