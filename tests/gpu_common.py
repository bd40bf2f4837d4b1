"""Helpers shared by the GPU parity tests: upload seeded inputs, build caches,
run one layer step through the C ABI, compare against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import head_latent_attention_13_amd as mla
from synthetic import Case

DEV = "cuda"

# Tolerances: bf16 caches with fp32 accumulation, and the fp32 config.
BF16_REL_L2, BF16_MAX_ABS = 1e-2, 3e-2
F32_REL_L2, F32_MAX_ABS = 1e-5, 1e-5


def dims_of(cfg, form="merged"):
    return mla.make_dims(cfg.d_model, cfg.n_heads, cfg.d_latent, cfg.d_q_latent, cfg.d_nope, cfg.d_rope, cfg.d_v,
                         cfg.dtype, cfg.rope_base, form=form)


def tdtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def dev(a, cfg):
    """Upload an fp32 array whose values are exactly representable in the config dtype."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(tdtype(cfg))


def upload_weights(case: Case):
    return {k: dev(v, case.cfg) for k, v in case.weights.items()}


def contiguous_cache(cfg, rows, s_max):
    B = len(rows)
    pool = torch.zeros(B, s_max, cfg.row, dtype=tdtype(cfg), device=DEV)
    for b, r in enumerate(rows):
        if len(r):
            pool[b, :len(r)] = dev(r, cfg)
    return mla.Cache(pool=pool, s_max=s_max), pool


def paged_cache(cfg, rows, table, n_pages, kv_len, poison=False):
    P = cfg.page_size
    fill = float("nan") if poison else 0.0
    pool = torch.full((n_pages, P, cfg.row), fill, dtype=tdtype(cfg), device=DEV)
    tbl = torch.from_numpy(table).to(DEV)
    for b, r in enumerate(rows):
        npg = (int(kv_len[b]) + P - 1) // P
        tmp = torch.full((npg * P, cfg.row), fill, dtype=tdtype(cfg), device=DEV)
        if len(r):
            tmp[:len(r)] = dev(r, cfg)
        pool[tbl[b, :npg].long()] = tmp.view(npg, P, cfg.row)
    cache = mla.Cache(pool=pool, page_table=tbl, page_size=P, n_pages=n_pages, max_pages_per_seq=table.shape[1])
    return cache, pool


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def run_step(layer, cfg, case: Case, cache, do_append=True):
    """append (optional) + decode + out_proj for the case's new tokens."""
    B, n_q = cfg.batch, cfg.n_q
    x = dev(case.x_new.reshape(B * n_q, cfg.d_model), cfg)
    pos = i32(case.cached)
    kv = i32(case.cached + n_q)
    o_lat = torch.empty(B * n_q, cfg.n_heads, cfg.d_latent, dtype=torch.float32, device=DEV)
    lse = torch.empty(B * n_q, cfg.n_heads, dtype=torch.float32, device=DEV)
    y = torch.empty(B * n_q, cfg.d_model, dtype=torch.float32, device=DEV)
    if do_append:
        layer.append(x, pos, B, n_q, cache)
    layer.decode(x, kv, B, n_q, cache, o_lat, lse)
    layer.out_proj(o_lat, B * n_q, y)
    torch.cuda.synchronize()
    return o_lat, lse, y


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b):
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max())


def assert_close(gpu, ref, cfg, what):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    r, m = rel_l2(gpu, ref), max_abs(gpu, ref)
    if cfg.dtype == "bf16":
        ok = r <= BF16_REL_L2 and m <= BF16_MAX_ABS
    else:
        ok = r <= F32_REL_L2 and m <= F32_MAX_ABS * max(1.0, float(np.abs(ref).max()))
    print(f"[parity] {cfg.name} {what}: rel_l2={r:.3e} max_abs={m:.3e}", flush=True)
    assert ok, f"{what}: rel_l2={r:.3e} max_abs={m:.3e}"
    return r, m


def unpack(buf: np.ndarray, K: int, N: int, bf16: bool) -> np.ndarray:
    """Packed fragment order (see include/mla.h) -> row-major [K, N]."""
    KB, KPL = (32, 8) if bf16 else (4, 1)
    Kp, Np = -(-K // KB) * KB, -(-N // 16) * 16
    a = buf.reshape(Kp // KB, Np // 16, KB // KPL, 16, KPL)      # [kb, nt, g, n16, j]
    a = a.transpose(0, 2, 4, 1, 3).reshape(Kp, Np)                # [kb, g, j, nt, n16]
    return a[:K, :N]
