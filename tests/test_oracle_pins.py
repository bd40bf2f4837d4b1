"""The CPU oracle against what the pages and mathematics fix (no GPU).

Tolerances: every pin compares fp64 computations that are equal in exact
arithmetic, so the bound is a small multiple of fp64 rounding (1e-12
relative); the brute force uses correctly rounded sums.
"""
import importlib.util
import json
import os
import sys
import types

import numpy as np
import pytest

import oracle
from oracle import absorbed, accounting, expanded, rope

from . import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def test_pin_mha_equivalence_without_rope():
    assert pins.pin_mha(expanded) < 1e-12


def test_pin_absorbed_equals_expanded():
    assert pins.pin_absorbed(expanded, absorbed) < 1e-12


def test_pin_softmax_rows():
    assert pins.pin_softmax(expanded) < 1e-13


def test_pin_brute_force_tiny():
    assert pins.pin_brute(expanded) < 1e-12


def test_pin_kv_cache_decode_is_last_row():
    assert pins.pin_kvcache(expanded) < 1e-13


def test_pin_rope_rotation():
    assert pins.pin_rope(rope, expanded) < 1e-9


def test_rope_pair_layout_is_a_relabelling_of_weight_columns():
    """The pages leave RoPE's pair layout open.  Any other pairing is the
    same family of functions: the half-split layout (pairs (j, j + d/2)) on
    RoPE weight columns permuted into that order gives the interleaved
    layout's output (pairs (2j, 2j + 1)) on the original columns, since a
    score sums the rotated q_pe * k_pe products over every coordinate (page
    "Multi-Head Latent Attention (MLA)", section "The RoPE problem": RoPE is
    a position rotation applied to the decoupled query and key parts)."""
    def apply_half(v, pos, base):
        v = np.asarray(v, np.float64)
        d = v.shape[-1]
        ang = rope.angles(pos, d, base)
        cos, sin = np.cos(ang), np.sin(ang)
        a, b = v[..., : d // 2], v[..., d // 2:]
        return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)

    half = types.SimpleNamespace(apply=apply_half, angles=rope.angles)
    E2 = _mutant("expanded", "from . import rope as _rope", "from . import rope as _rope", {"_rope": half})
    case = pins.make_case(pins.MID, 31, history="x")
    d = pins.MID.d_rope
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # column j <- 2j, d/2 + j <- 2j + 1
    W2 = dict(case.weights)
    W2["W_KR"] = np.asarray(case.weights["W_KR"])[..., perm]
    W2["W_QR"] = np.asarray(case.weights["W_QR"])[..., perm]
    for b in range(pins.MID.batch):
        y1 = pins._run_decode(expanded, case, b)["y"]
        y2 = pins._run_decode(E2, case, b, W=W2)["y"]
        assert np.abs(y2 - y1).max() <= 1e-12 * np.abs(y1).max()
    # and the unpermuted columns do give a different function
    y3 = pins._run_decode(E2, case, 0)["y"]
    assert np.abs(y3 - pins._run_decode(expanded, case, 0)["y"]).max() > 1e-3 * np.abs(y3).max()


def test_pin_special_cases():
    assert pins.pin_special(expanded) < 1e-12


def test_lse_merge_of_any_partition_equals_full_softmax():
    """Split-KV property used by the GPU merge: a softmax over a partition of
    the keys, recombined with log-sum-exp weights, equals the unsplit one."""
    rng = np.random.default_rng(5)
    for trial in range(20):
        m = int(rng.integers(1, 300))
        s = rng.standard_normal(m) * rng.uniform(0.1, 30)
        v = rng.standard_normal((m, 7))
        p = np.exp(s - s.max())
        full = (p / p.sum()) @ v
        cuts = np.sort(rng.choice(np.arange(1, m), size=min(m - 1, int(rng.integers(0, 6))),
                                  replace=False)) if m > 1 else np.array([], int)
        parts = np.split(np.arange(m), cuts)
        lses, outs = [], []
        for idx in parts:
            mx = s[idx].max()
            e = np.exp(s[idx] - mx)
            lses.append(mx + np.log(e.sum()))
            outs.append((e / e.sum()) @ v[idx])
        lses = np.array(lses)
        L = lses.max() + np.log(np.exp(lses - lses.max()).sum())
        merged = sum(np.exp(l - L) * o for l, o in zip(lses, outs))
        assert np.abs(merged - full).max() < 1e-12 * max(1.0, np.abs(full).max())


def test_closed_form_cache_figures():
    """Byte figures printed by the pages from the section-05 formula.

    Assumed (not printed): 61 layers and 2-byte elements."""
    g = json.load(open(GOLDEN))
    layers, elt = 61, 2
    H, D, G = g["heads"]["value"], g["head_dim"]["value"], g["gqa_group_size"]["value"]
    assert g["latent_width"]["value"] + g["rope_width"]["value"] == g["mla_numbers_per_token_per_layer"]["value"]
    mha = accounting.mha_numbers(1, D, H, layers) * elt
    gqa = accounting.gqa_numbers(1, D, H, G, layers) * elt
    mla = accounting.mla_numbers(1, g["latent_width"]["value"], g["rope_width"]["value"], layers) * elt
    assert mha == 3_997_696 and gqa == 499_712 and mla == 70_272
    # printed figures are rounded: 4 MB, 500 KB, 70 KB, 57x, ~400 GB
    assert abs(mha - g["mha_bytes_per_token"]["value"]) / g["mha_bytes_per_token"]["value"] < 0.01
    assert abs(gqa - g["gqa8_bytes_per_token"]["value"]) / g["gqa8_bytes_per_token"]["value"] < 0.01
    assert abs(mla - g["mla_bytes_per_token"]["value"]) / g["mla_bytes_per_token"]["value"] < 0.01
    assert round(mha / mla) == g["mha_over_mla"]["value"]
    n = g["mha_read_per_token_at_100k"]["context_tokens"]
    assert abs(mha * n - g["mha_read_per_token_at_100k"]["value"]) / g["mha_read_per_token_at_100k"]["value"] < 0.01
    assert accounting.gqa_equivalent_groups(512, 64, 128) == g["gqa_equivalent_groups"]["value"]


# ------------------------------------------------------ planted mistakes ----
def _mutant(modname, old, new, extra=None):
    """A copy of oracle.<modname> with ``old`` replaced by ``new`` in its source."""
    path = os.path.join(os.path.dirname(oracle.__file__), modname + ".py")
    src = open(path).read()
    assert src.count(old) >= 1, (modname, old)
    src = src.replace(old, new)
    mod = types.ModuleType("oracle._mut_" + modname)
    mod.__package__ = "oracle"
    mod.__file__ = path
    exec(compile(src, path + "[mutant]", "exec"), mod.__dict__)
    for k, v in (extra or {}).items():
        setattr(mod, k, v)
    return mod


MUTATIONS = [
    # (module, old, new): each is a plausible slip in the oracle
    ("expanded", "(qp @ k_pe.T[None])", "(0.0 * (qp @ k_pe.T[None]))"),           # dropped RoPE term
    ("expanded", "<= q_pos[:, None]", "< q_pos[:, None] + 2"),                       # causal off by one
    ("expanded", "k_nope = (c @ W_UK[:, blk, :]", "k_nope = (c @ W_UV[:, blk, :]"),  # wrong up-projection
    ("expanded", "scores = scores * scale", "scores = scores * scale * scale"),      # wrong scale
    ("expanded", "@ W_O[blk].reshape", "@ W_O[::-1][blk].reshape"),               # wrong head's W_O
    ("expanded", "W_UQ, W_QR = _f64(W[\"W_UQ\"]), _f64(W[\"W_QR\"])",
                 "W_UQ, W_QR = _f64(W[\"W_UQ\"])[:, ::-1], _f64(W[\"W_QR\"])"),          # head index
    ("expanded", "k_pe = _rope.apply(x @ _f64(W[\"W_KR\"]), np.asarray(pos), base)",
                 "k_pe = _rope.apply(x @ _f64(W[\"W_KR\"]), np.asarray(pos) + 1, base)"),  # key position
    ("expanded", "p = e / den ", "p = e / den.sum() "),                               # normalisation
    ("expanded", 'ob = p @ v ', 'ob = p.transpose(0, 1, 2)[:, :, ::-1] @ v '),        # reversed key order
    ("rope", "a * sin + b * cos", "-a * sin + b * cos"),                             # sign
    ("rope", "a, b = v[..., 0::2], v[..., 1::2]", "a, b = v[..., 1::2], v[..., 0::2]"),  # pair order
    ("rope", "-2.0 * j / d_rope", "-1.0 * j / d_rope"),                              # frequencies
    # head blocks: a block's results stored at the wrong offset, every block
    # computed for the first block's heads, the subset's head list ignored
    ("expanded", "o_lat[:, s:s + len(blk)] =", "o_lat[:, 0:len(blk)] ="),
    ("expanded", "o_h[:, s:s + len(blk)] =", "o_h[:, 0:len(blk)] ="),
    ("expanded", "lse[:, s:s + len(blk)] =", "lse[:, 0:len(blk)] ="),
    ("expanded", "blk = hs[s:s + head_block]", "blk = hs[0:head_block]"),
    ("expanded", "hs = list(range(H)) if heads is None else list(heads)", "hs = list(range(H))"),
    ("absorbed", "W_UQ[:, h, :] @ W_UK[:, h, :].T", "W_UQ[:, h, :] @ W_UK[:, -h - 1, :].T"),
    ("absorbed", "W_UV[:, h, :] @ W_O[h]", "W_UV[:, h, :] @ W_O[(h + 1) % len(W_O)]"),
]


@pytest.mark.parametrize("mod,old,new", MUTATIONS, ids=[f"{m}:{i}" for i, (m, _, _) in enumerate(MUTATIONS)])
def test_planted_mistake_fails_a_pin(mod, old, new):
    E, A, R = expanded, absorbed, rope
    if mod == "expanded":
        E = _mutant("expanded", old, new)
    elif mod == "absorbed":
        A = _mutant("absorbed", old, new)
    elif mod == "rope":
        R = _mutant("rope", old, new)
        E = _mutant("expanded", "from . import rope as _rope", "from . import rope as _rope", {"_rope": R})
        A = _mutant("absorbed", "from . import rope as _rope", "from . import rope as _rope", {"_rope": R})
    bounds = {"mha": 1e-12, "absorbed": 1e-12, "softmax": 1e-13, "brute": 1e-12,
              "kvcache": 1e-13, "rope": 1e-9, "special": 1e-12}
    failed = []
    for name in pins.ALL_PINS:
        try:
            fn = getattr(pins, "pin_" + name)
            err = {"mha": lambda: fn(E), "absorbed": lambda: fn(E, A), "softmax": lambda: fn(E),
                   "brute": lambda: fn(E), "kvcache": lambda: fn(E), "rope": lambda: fn(R, E),
                   "special": lambda: fn(E)}[name]()
        except Exception:
            failed.append(name)
            continue
        if not np.isfinite(err) or err > bounds[name]:
            failed.append(name)
    assert failed, "planted mistake passed every pin"
