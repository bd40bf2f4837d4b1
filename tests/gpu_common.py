"""Helpers shared by the GPU parity tests: upload seeded inputs, build caches,
run one layer step through the C ABI, compare against the oracle."""
from __future__ import annotations

import functools

import numpy as np
import torch

import head_latent_attention_13_amd as mla
from oracle import expanded as OE
from synthetic import Case, config, make_case, quiet_then_loud

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


# Canary guard bands: outputs are carved out of a larger buffer whose
# GUARD elements on either side hold a sentinel; a write outside the output
# changes them.
GUARD = 4096
SENTINEL = -12345.5


class Guarded:
    """An fp32 output tensor of `shape` with sentinel-filled guard bands."""

    def __init__(self, *shape):
        n = int(np.prod(shape))
        self.buf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.float32, device=DEV)
        self.t = self.buf[GUARD:GUARD + n].view(*shape)

    def check(self, what="output"):
        b = self.buf.cpu().numpy()
        assert (b[:GUARD] == SENTINEL).all() and (b[-GUARD:] == SENTINEL).all(), f"{what}: guard band overwritten"


def run_step(layer, cfg, case: Case, cache, do_append=True):
    """append (optional) + decode + out_proj for the case's new tokens.
    o_lat, lse and y sit between guard bands, checked after the step."""
    B, n_q = cfg.batch, cfg.n_q
    x = dev(case.x_new.reshape(B * n_q, cfg.d_model), cfg)
    pos = i32(case.cached)
    kv = i32(case.cached + n_q)
    o_lat = Guarded(B * n_q, cfg.n_heads, cfg.d_latent)
    lse = Guarded(B * n_q, cfg.n_heads)
    y = Guarded(B * n_q, cfg.d_model)
    if do_append:
        layer.append(x, pos, B, n_q, cache)
    layer.decode(x, kv, B, n_q, cache, o_lat.t, lse.t)
    layer.out_proj(o_lat.t, B * n_q, y.t)
    torch.cuda.synchronize()
    o_lat.check("o_lat")
    lse.check("lse")
    y.check("y")
    return o_lat.t, lse.t, y.t


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b):
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max())


def assert_close(gpu, ref, cfg, what, stress=False):
    """rel-L2 and max-abs bars of the configuration's dtype.  ``stress``:
    inputs scaled beyond the workloads' distribution (the rebase rows), for
    which the bf16 max-abs bar is taken relative to the reference's largest
    magnitude, as the fp32 bar always is (the bf16 rounding of the query
    alone moves the outputs by about 1% of their scale there)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    r, m = rel_l2(gpu, ref), max_abs(gpu, ref)
    if cfg.dtype == "bf16":
        scale = max(1.0, float(np.abs(ref).max())) if stress else 1.0
        ok = r <= BF16_REL_L2 and m <= BF16_MAX_ABS * scale
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


def oracle_for(case: Case, b, js=None, **kw):
    """Expanded oracle for sequence b of a case whose history is given as
    rows: its new tokens' rows are appended, then queries js (default: all
    new tokens) attend."""
    cfg = case.cfg
    S = int(case.cached[b])
    W = case.weights
    n_q = cfg.n_q
    js = np.arange(n_q) if js is None else np.asarray(js)
    c_new, k_new = OE.latent_rows(W, case.x_new[b], S + np.arange(n_q), cfg.rope_base)
    c = np.concatenate([case.rows[b][:, :cfg.d_latent], c_new])
    k = np.concatenate([case.rows[b][:, cfg.d_latent:], k_new])
    _, qn, qp = OE.query(W, case.x_new[b][js], S + js, cfg.rope_base)
    return OE.attention(W, qn, qp, c, k, S + js, cfg.softmax_scale, **kw)


# Queries of the V3 1024-token chunk checked against the oracle: one whole
# block of 128, the edges of later query blocks and key tiles, the last.
CHUNK_QUERIES = np.unique(np.concatenate([np.arange(128), [129, 159, 160, 161, 255, 256, 511, 512, 767, 1022, 1023]]))


@functools.lru_cache(maxsize=2)
def chunk_case(seed, loud):
    """The V3 chunked-prefill workload (seeded; ``loud``: history rows
    following synthetic.quiet_then_loud)."""
    return make_case(config(4), seed, amplitude=quiet_then_loud if loud else None)


@functools.lru_cache(maxsize=4)
def chunk_oracle(seed, loud, b):
    """Oracle outputs (o_lat, lse, y) of CHUNK_QUERIES of sequence b of
    chunk_case(seed, loud); shared by the absorbed and expanded tests."""
    return oracle_for(chunk_case(seed, loud), b, CHUNK_QUERIES)
