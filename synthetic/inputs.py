"""Seeded input draws for the MLA workloads (no attention arithmetic here).

Everything is drawn from ``numpy.random.default_rng(seed)`` (PCG64) in a
fixed order so that a (config, seed) pair names one input set:

1. the raw weights ``W_DQ, W_UQ, W_QR, W_DKV, W_KR, W_UK, W_UV, W_O``;
2. the cached lengths (when the config gives a range);
3. the page permutation (paged configs);
4. the history: either cache rows (``history="rows"``) or token activations
   (``history="x"``), one sequence after another;
5. the new tokens ``x_new``.

For bf16 configs every value is drawn in fp32 and rounded once to bf16 with
round-to-nearest-even; both sides consume exactly those values.

Synthetic cache rows stand in for rows appended from real activations: a
latent ``x @ W_DKV`` with ``x ~ N(0,1)`` and ``W ~ N(0, 0.02^2)`` has entries
distributed ``N(0, d_model * 0.02^2)``, and the RoPE key is a rotation of an
identically distributed vector, so rows are drawn i.i.d. from that normal.
Drawing them directly keeps every decode input independent of the GPU path.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

from .configs import MLAConfig

WEIGHT_ORDER = ("W_DQ", "W_UQ", "W_QR", "W_DKV", "W_KR", "W_UK", "W_UV", "W_O")


# ---------------------------------------------------------------- bf16 ----
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u  # no overflow for finite values below the largest bf16 binade
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value, returned as fp32."""
    return bf16_to_f32(bf16_bits(a))


# ------------------------------------------------------------- shapes ----
def weight_shapes(cfg: MLAConfig) -> Dict[str, tuple]:
    H = cfg.n_heads
    return {
        "W_DQ": (cfg.d_model, cfg.d_q_latent),
        "W_UQ": (cfg.d_q_latent, H, cfg.d_nope),
        "W_QR": (cfg.d_q_latent, H, cfg.d_rope),
        "W_DKV": (cfg.d_model, cfg.d_latent),
        "W_KR": (cfg.d_model, cfg.d_rope),
        "W_UK": (cfg.d_latent, H, cfg.d_nope),
        "W_UV": (cfg.d_latent, H, cfg.d_v),
        "W_O": (H, cfg.d_v, cfg.d_model),
    }


def _fan_in(name: str, cfg: MLAConfig) -> int:
    return {
        "W_DQ": cfg.d_model, "W_DKV": cfg.d_model, "W_KR": cfg.d_model,
        "W_UQ": cfg.d_q_latent, "W_QR": cfg.d_q_latent,
        "W_UK": cfg.d_latent, "W_UV": cfg.d_latent,
        "W_O": cfg.n_heads * cfg.d_v,
    }[name]


def _finish(a: np.ndarray, cfg: MLAConfig) -> np.ndarray:
    a = a.astype(np.float32, copy=False)
    return round_bf16(a) if cfg.dtype == "bf16" else a


def _x_std(cfg: MLAConfig) -> float:
    return (1.0 / cfg.d_model) ** 0.5 if cfg.init == "fanin" else 1.0


def row_std(cfg: MLAConfig) -> float:
    """Std of a latent-cache entry produced from x through W_DKV / W_KR."""
    if cfg.init == "fanin":
        return (1.0 / cfg.d_model) ** 0.5
    return 0.02 * cfg.d_model ** 0.5


# -------------------------------------------------------------- draws ----
def make_weights(cfg: MLAConfig, rng: np.random.Generator) -> Dict[str, np.ndarray]:
    out = {}
    for name, shape in weight_shapes(cfg).items():
        std = (1.0 / _fan_in(name, cfg)) ** 0.5 if cfg.init == "fanin" else 0.02
        out[name] = _finish(rng.standard_normal(shape, dtype=np.float32) * np.float32(std), cfg)
    return out


def make_lengths(cfg: MLAConfig, rng: np.random.Generator) -> np.ndarray:
    if isinstance(cfg.cached, tuple):
        lo, hi = cfg.cached
        return rng.integers(lo, hi, size=cfg.batch, endpoint=True).astype(np.int64)
    return np.full(cfg.batch, int(cfg.cached), dtype=np.int64)


def make_page_table(kv_len: np.ndarray, page_size: int, rng: np.random.Generator,
                    spare_pages: int = 0):
    """Deal a seeded permutation of the shared page pool to the sequences.

    Returns (page_table[B, max_pages] int32 with -1 in unused entries,
    n_pages).  ``spare_pages`` extra pool pages are left unowned.
    """
    pages = [(int(n) + page_size - 1) // page_size for n in kv_len]
    n_pages = sum(pages) + spare_pages
    perm = rng.permutation(n_pages).astype(np.int32)
    max_pages = max(pages) if pages else 0
    table = np.full((len(pages), max(max_pages, 1)), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[k:k + n]
        k += n
    return table, n_pages


def quiet_then_loud(n_rows: int, quiet_rows: int = 32, quiet: float = 0.05, lo: float = 5.0,
                    hi: float = 6.0) -> np.ndarray:
    """Per-row amplitude multipliers: the first ``quiet_rows`` rows scaled by
    ``quiet``, the rest by a linear ramp from ``lo`` to ``hi``.

    A cache of such rows makes every head's largest score jump by many times
    the unscaled score spread between the first 32-row block of a sequence
    and the next, and keeps growing along the sequence; it is an input
    pattern only (the amplitudes multiply i.i.d. normal draws).
    """
    a = np.empty(n_rows, dtype=np.float32)
    q = min(quiet_rows, n_rows)
    a[:q] = quiet
    if n_rows > q:
        a[q:] = np.linspace(lo, hi, n_rows - q, dtype=np.float32)
    return a


def make_rows(cfg: MLAConfig, lengths: np.ndarray, rng: np.random.Generator,
              amplitude=None) -> List[np.ndarray]:
    """Synthetic cache rows per sequence, as fp32 arrays [S_b, R].

    ``amplitude``: optional callable n -> [n] per-row multipliers (applied
    to the fp32 draws before the bf16 rounding)."""
    std = np.float32(row_std(cfg))
    out = []
    for s in lengths:
        r = rng.standard_normal((int(s), cfg.row), dtype=np.float32) * std
        if amplitude is not None:
            r *= np.asarray(amplitude(int(s)), np.float32)[:, None]
        out.append(_finish(r, cfg))
    return out


# Exponent-field weights of the synthetic E4M3 codes, fields 15 down to 8,
# then the zero code: the binade masses of a normal draw with the std of
# the bf16 rows of the V2 / V3 shapes (~1.43) at row scale 2^-6.  A row
# drawn with scale 2^k shifts its fields down by k + 6, so every row's
# values spread alike (as real rows do) whatever its scale.
_E4_FIELD_P = np.array([0.01, 0.16, 0.32, 0.24, 0.13, 0.07, 0.04, 0.02, 0.01])
_E4_K = np.array([-7, -6, -5])


def make_e4m3_rows(cfg: MLAConfig, lengths: np.ndarray, rng: np.random.Generator
                   ) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Synthetic E4M3 cache rows per sequence: (codes uint8 [S_b, R], row
    scale exponents int32 [S_b]), drawn field by field — a uniform sign
    bit, the exponent field from _E4_FIELD_P, a uniform mantissa (never the
    NaN pattern), shifted against a scale exponent drawn from _E4_K per
    row.  A row's values are code * 2^k."""
    out = []
    for s in lengths:
        n = (int(s), cfg.row)
        sign = rng.integers(0, 2, n)
        pick = rng.choice(len(_E4_FIELD_P), size=n, p=_E4_FIELD_P)
        k = rng.choice(_E4_K, size=int(s)).astype(np.int32)
        field = np.minimum(15 - pick - (k[:, None] + 6), 15)
        mant = rng.integers(0, 8, n)
        mant = np.where((field == 15) & (mant == 7), 6, mant)
        codes = (sign << 7) | (field << 3) | mant
        codes = np.where(pick == len(_E4_FIELD_P) - 1, 0, codes).astype(np.uint8)
        out.append((codes, k))
    return out


def make_x(cfg: MLAConfig, shape, rng: np.random.Generator) -> np.ndarray:
    return _finish(rng.standard_normal(shape, dtype=np.float32) * np.float32(_x_std(cfg)), cfg)


@dataclass
class Case:
    cfg: MLAConfig
    seed: int
    weights: Dict[str, np.ndarray]
    cached: np.ndarray                  # [B] cached tokens before this step
    x_new: np.ndarray                   # [B, n_q, d_model] fp32
    rows: Optional[List[np.ndarray]] = None       # history rows, history="rows"
    x_hist: Optional[List[np.ndarray]] = None     # history tokens, history="x"
    page_table: Optional[np.ndarray] = None
    n_pages: int = 0
    extra: dict = field(default_factory=dict)
    # E4M3 rows (codes [S_b, R] uint8, scale exponents [S_b]), history="e4m3"
    e4m3: Optional[List[Tuple[np.ndarray, np.ndarray]]] = None

    @property
    def kv_len(self) -> np.ndarray:
        """Visible rows per sequence after the new tokens are appended."""
        return self.cached + self.cfg.n_q

    @property
    def positions(self) -> np.ndarray:
        """[B, n_q] positions of the new tokens (0-based)."""
        return self.cached[:, None] + np.arange(self.cfg.n_q)[None, :]


def make_case(cfg: MLAConfig, seed: int, history: str = "rows",
              spare_pages: int = 0, amplitude=None) -> Case:
    """``history``: "rows" (fp32 history rows), "x" (history activations)
    or "e4m3" (E4M3 codes and scale exponents of every row a decode sees,
    the new tokens' own rows included: make_e4m3_rows over cached + n_q).
    ``amplitude``: optional per-row multipliers of the history rows
    (history="rows" only; see quiet_then_loud)."""
    rng = np.random.default_rng(seed)
    w = make_weights(cfg, rng)
    cached = make_lengths(cfg, rng)
    table, n_pages = (None, 0)
    if cfg.paged:
        table, n_pages = make_page_table(cached + cfg.n_q, cfg.page_size, rng, spare_pages)
    rows = x_hist = e4m3 = None
    if history == "rows":
        rows = make_rows(cfg, cached, rng, amplitude)
    elif history == "x":
        x_hist = [make_x(cfg, (int(s), cfg.d_model), rng) for s in cached]
    elif history == "e4m3":
        e4m3 = make_e4m3_rows(cfg, cached + cfg.n_q, rng)
    else:
        raise ValueError(history)
    x_new = make_x(cfg, (cfg.batch, cfg.n_q, cfg.d_model), rng)
    return Case(cfg=cfg, seed=seed, weights=w, cached=cached, x_new=x_new,
                rows=rows, x_hist=x_hist, page_table=table, n_pages=n_pages, e4m3=e4m3)
