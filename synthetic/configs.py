"""The five workload shapes of the MLA hot path.

Dimensions follow DeepSeek-V2/V3 as the pages give them: 128 heads of 128,
a 512-wide shared KV latent plus a 64-wide decoupled RoPE key (page
"Multi-Head Latent Attention: How DeepSeek Shrinks AI Memory", section "How
does multi-head latent attention work?"; page "How DeepSeek Rewrote the
Transformer", section 08 "The result": 576 cached numbers per token).  The
query latent width (1536), model widths (5120 / 7168) and the batch/context
mixes are the workload definitions this library is measured on.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class MLAConfig:
    name: str
    d_model: int
    n_heads: int
    d_latent: int        # d_L: shared KV latent width
    d_q_latent: int      # d_LQ: query latent width
    d_nope: int          # per-head non-positional query/key width
    d_rope: int          # decoupled RoPE key/query width (shared key)
    d_v: int             # per-head value width
    dtype: str           # "f32" or "bf16": weights, activations, cache
    batch: int
    cached: object       # int, or (lo, hi) inclusive uniform range
    n_q: int             # new tokens per sequence in this step
    paged: bool
    page_size: int = 64
    rope_base: float = 10000.0
    init: str = "std0.02"  # "fanin": N(0, 1/fan_in); "std0.02": N(0, 0.02^2)

    @property
    def row(self) -> int:
        """Elements per cached token: latent followed by the RoPE key."""
        return self.d_latent + self.d_rope

    @property
    def softmax_scale(self) -> float:
        # Scores are dot products over the concatenated nope+rope vector.
        return 1.0 / float(self.d_nope + self.d_rope) ** 0.5

    def with_batch(self, batch: int) -> "MLAConfig":
        return replace(self, batch=batch)

    def with_(self, **kw) -> "MLAConfig":
        return replace(self, **kw)


_V2 = dict(d_model=5120, n_heads=128, d_latent=512, d_q_latent=1536,
           d_nope=128, d_rope=64, d_v=128, dtype="bf16")

CONFIGS: Tuple[MLAConfig, ...] = (
    MLAConfig(name="tiny_f32", d_model=64, n_heads=4, d_latent=32,
              d_q_latent=48, d_nope=16, d_rope=8, d_v=16, dtype="f32",
              batch=1, cached=16, n_q=1, paged=False, init="fanin"),
    MLAConfig(name="v2_decode_contiguous", batch=16, cached=4096, n_q=1,
              paged=False, **_V2),
    MLAConfig(name="v2_decode_paged", batch=64, cached=(512, 16384), n_q=1,
              paged=True, **_V2),
    MLAConfig(name="v2_decode_long", batch=4, cached=100000, n_q=1,
              paged=True, **_V2),
    MLAConfig(name="v3_chunked_prefill", batch=2, cached=4096, n_q=1024,
              paged=False, **dict(_V2, d_model=7168)),
)


def config(idx_or_name) -> MLAConfig:
    if isinstance(idx_or_name, int):
        return CONFIGS[idx_or_name]
    for c in CONFIGS:
        if c.name == idx_or_name:
            return c
    raise KeyError(idx_or_name)
