"""Calls with fewer rows than the workspace was sized for, through the C
ABI (MI355X only).  At the V2 shape a 20-row call's own GEMM plans want more
split-K partial bytes than mla_workspace_size gives for 23 rows, so the
calls re-plan with fewer K splits to fit; the results must still match the
oracle (rel-L2 <= 1e-2, max-abs <= 3e-2 for bf16)."""
import numpy as np
import pytest
import torch

import head_latent_attention_13_amd as mla
from oracle import absorbed as OA
from oracle import expanded as OE
from synthetic import config, make_case

from .gpu_common import DEV, assert_close, contiguous_cache, dev, dims_of, i32, upload_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    mla.load()


def test_smaller_calls_on_a_larger_workspace():
    cfg = config(1).with_(batch=20, cached=64, n_q=1)
    case = make_case(cfg, seed=41)
    B, R, H = cfg.batch, cfg.row, cfg.n_heads
    dims = dims_of(cfg)
    assert mla.mla_workspace_size(dims, 20, 1) > mla.mla_workspace_size(dims, 23, 1), "shape no longer capped"
    print("[ws-fit] V2 shape, 20 rows on a 23-row workspace", flush=True)
    layer = mla.MLALayer(dims, upload_weights(case), max_batch=23, max_nq=1)
    x = dev(case.x_new.reshape(B, cfg.d_model), cfg)
    S = int(case.cached[0])
    cache, pool = contiguous_cache(cfg, [np.zeros((0, R), np.float32)] * B, S + 1)
    layer.append(x, i32(case.cached), B, 1, cache)
    q = torch.empty(B, H, R, dtype=torch.bfloat16, device=DEV)
    layer.q_proj(x, i32(case.cached + 1), B, 1, q)
    rng = np.random.default_rng(5)
    o_lat = (rng.standard_normal((B, H, cfg.d_latent)) * 0.05).astype(np.float32)
    y = torch.empty(B, cfg.d_model, dtype=torch.float32, device=DEV)
    layer.out_proj(torch.from_numpy(o_lat).to(DEV), B, y)
    torch.cuda.synchronize()
    assert layer.device_error() == 0

    uqk, uvo = OA.merged_weights(case.weights)
    xs = case.x_new[:, 0, :]
    pos = case.cached.astype(np.int64)
    c_ref, k_ref = OE.latent_rows(case.weights, xs, pos, cfg.rope_base)
    rows = pool.float().cpu().numpy()[:, S, :]
    assert_close(rows[:, :cfg.d_latent], c_ref, cfg, "appended latents")
    assert_close(rows[:, cfg.d_latent:], k_ref, cfg, "appended rope keys")
    q_lat, q_pe = OA.query_latent(case.weights, uqk, xs, pos, cfg.rope_base)
    qg = q.float().cpu().numpy()
    assert_close(qg[:, :, :cfg.d_latent], q_lat, cfg, "q latent part")
    assert_close(qg[:, :, cfg.d_latent:], q_pe, cfg, "q rope part")
    assert_close(y.cpu().numpy(), OA.out_proj(o_lat, uvo), cfg, "out_proj y")
