"""KV-cache size accounting — oracle (test infrastructure).

Page "How DeepSeek Rewrote the Transformer", section 05 ("Four megabytes per
token"): a model with L layers, NH heads of dimension DH caches
2 x N x DH x NH x L numbers for N tokens (a key and a value per head).  With
grouped-query attention only the groups' keys and values are cached
(section 06), and MLA caches the latent plus the RoPE key, independent of
the head count (section 08: 576 per token).
"""


def mha_numbers(n_tokens: int, head_dim: int, n_heads: int, n_layers: int) -> int:
    return 2 * n_tokens * head_dim * n_heads * n_layers


def gqa_numbers(n_tokens: int, head_dim: int, n_heads: int, group: int, n_layers: int) -> int:
    return 2 * n_tokens * head_dim * (n_heads // group) * n_layers


def mla_numbers(n_tokens: int, d_latent: int, d_rope: int, n_layers: int) -> int:
    return n_tokens * (d_latent + d_rope) * n_layers


def gqa_equivalent_groups(d_latent: int, d_rope: int, head_dim: int) -> float:
    """Number of GQA key/value groups caching as many numbers as MLA."""
    return (d_latent + d_rope) / (2.0 * head_dim)
