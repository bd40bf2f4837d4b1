"""The oracle's E4M3 codes and row quantiser against what the format and
the mathematics fix (no GPU).

Pins:
  * decode of every one of the 256 codes equals torch.float8_e4m3fn's;
  * encode equals torch's float32 -> float8_e4m3fn cast bit for bit on
    every exact midpoint between neighbouring codes (ties), the subnormal
    range, the overflow edge, signed zeros, inf / NaN and random values;
  * encode(decode(c)) == c for every finite code (the grid is exact);
  * the row scale exponent is the smallest k >= -126 with amax <= 448 * 2^k,
    found by brute force over k;
  * round-to-nearest error bounds of the quantised rows, and the scaled
    row's largest magnitude in (224, 448] before rounding.
Planted slips in the oracle (bias, rounding mode, subnormal spacing, scale
exponent) must fail one of them.
"""
import numpy as np
import pytest
import torch

from oracle import fp8

from .test_oracle_pins import _mutant


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _probe_values():
    rng = np.random.default_rng(20)
    vals = [0.0, -0.0, 448.0, -448.0, 456.0, 464.0, -464.0, 464.5, 479.0, 480.0, 1e6, -1e6, np.inf, -np.inf, np.nan]
    # every midpoint between neighbouring positive codes, and a hair either side
    grid = np.unique(np.abs(_torch_decode(np.arange(127, dtype=np.uint8))))
    mids = (grid[:-1] + grid[1:]) / 2
    for m in mids:
        vals += [m, -m, np.nextafter(np.float32(m), np.float32(0)), np.nextafter(np.float32(m), np.float32(1e9))]
    vals += list(grid) + list(-grid)
    x = np.concatenate([np.array(vals, np.float32),
                        (rng.standard_normal(3000) * 60).astype(np.float32),
                        (rng.standard_normal(3000) * 2e-3).astype(np.float32),
                        np.exp2(rng.uniform(-12, 9, 3000)).astype(np.float32) * rng.choice([-1, 1], 3000)])
    return x.astype(np.float32)


def pin_decode(F):
    codes = np.arange(256, dtype=np.uint8)
    ref, got = _torch_decode(codes), F.decode(codes)
    same = (np.isnan(ref) & np.isnan(got)) | (ref == got)
    return int((~same).sum())


def pin_encode(F):
    x = _probe_values()
    return int((F.encode(x) != _torch_encode(x)).sum())


def pin_roundtrip(F):
    codes = np.arange(256, dtype=np.uint8)
    finite = ~np.isnan(_torch_decode(codes))
    return int((F.encode(F.decode(codes[finite])) != codes[finite]).sum())


def pin_scale_exponent(F):
    rng = np.random.default_rng(21)
    rows = (rng.standard_normal((400, 9)) * np.exp2(rng.uniform(-20, 20, (400, 1)))).astype(np.float32)
    rows[0] = 0.0
    rows[1, 3] = np.float32(448.0)       # amax exactly 448 * 2^0
    rows[2, :] = np.float32(448.0 * 2.0 ** -5)
    rows[3, 0] = np.float32(np.nextafter(np.float32(448.0), np.float32(1e9)))
    rows[4, :] = np.float32(3e-38)       # below 448 * 2^-126: the exponent stops at -126
    rows[5, :] = np.float32(448.0 * 2.0 ** -126)
    k = F.row_scale_exponents(rows)
    bad = 0
    for r, kk in zip(rows, k):
        amax = float(np.max(np.abs(r)))
        if amax == 0:
            bad += kk != 0
            continue
        ks = [j for j in range(-126, 160) if amax <= 448.0 * 2.0 ** j]
        bad += kk != min(ks)
    return int(bad)


def pin_row_bounds(F):
    """Errors of the quantised rows within half a code step, scaled amax in (224, 448]."""
    rng = np.random.default_rng(22)
    rows = (rng.standard_normal((300, 576)) * np.exp2(rng.uniform(-8, 8, (300, 1)))).astype(np.float32)
    codes, scales = F.quantize_rows(rows)
    deq = F.dequantize_rows(codes, scales)
    x = rows.astype(np.float64)
    s = scales.astype(np.float64)[:, None]
    a = np.abs(x) / s
    # half the spacing of the scaled value's binade (2^-10 below 2^-6)
    half = np.where(a < 2.0 ** -6, 2.0 ** -10, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 4)) * s
    worst = float(np.max(np.abs(deq - x) - half))
    amax = np.max(np.abs(x), axis=1) / scales      # before rounding: (224, 448]
    top = np.max(np.abs(deq), axis=1) / scales     # after: [224, 448]
    ok = worst <= 0 and np.all(amax > 224) and np.all(amax <= 448) and np.all(top >= 224) and np.all(top <= 448)
    ok = ok and np.all(np.log2(scales) == np.round(np.log2(scales)))
    return 0 if ok else 1


ALL = {"decode": pin_decode, "encode": pin_encode, "roundtrip": pin_roundtrip, "scale": pin_scale_exponent,
       "bounds": pin_row_bounds}


@pytest.mark.parametrize("name", list(ALL))
def test_pin(name):
    assert ALL[name](fp8) == 0


def test_zero_row_and_exact_grid_rows():
    codes, scales = fp8.quantize_rows(np.zeros((2, 8), np.float32))
    assert np.all(codes == 0) and np.all(scales == 1.0)
    # rows already on the grid (codes times a power of two) come back exactly
    rng = np.random.default_rng(23)
    c = rng.integers(0, 256, (50, 64)).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    c[:, 0] = 0x7E  # one 448 per row: the scale is exactly the row's
    rows = (fp8.decode(c) * np.exp2(rng.integers(-6, 6, (50, 1)))).astype(np.float32)
    codes, scales = fp8.quantize_rows(rows)
    assert np.array_equal(fp8.dequantize_rows(codes, scales), rows.astype(np.float64))


MUTATIONS = [
    ("(1.0 + m / 8.0) * np.exp2(e - 7.0)", "(1.0 + m / 8.0) * np.exp2(e - 6.0)"),     # exponent bias
    ("(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),                               # subnormal scale
    ("q = np.round(fin / step)", "q = np.floor(fin / step)"),                          # truncation
    ("q = np.round(fin / step)", "q = np.floor(fin / step + 0.5)"),                    # ties away
    ("e_unb = np.maximum(E - 1, -6)", "e_unb = np.maximum(E - 1, -7)"),                # subnormal spacing
    ("overflow = (a > 464.0)", "overflow = (a >= 464.0)"),                             # overflow edge
    ("np.where(f <= 0.875, E - 9, E - 8)", "np.where(f < 0.875, E - 9, E - 8)"),      # scale at 448 * 2^k
    ("np.where(f <= 0.875, E - 9, E - 8)", "(E - 8)"),                                 # one binade too coarse
    ("np.where(f <= 0.875, E - 9, E - 8), -126)", "np.where(f <= 0.875, E - 9, E - 8), -149)"),  # no floor
    ("return decode(codes) * np.asarray(scales", "return decode(codes) / np.asarray(scales"),  # inverse scale
]


@pytest.mark.parametrize("old,new", MUTATIONS, ids=[f"fp8:{i}" for i in range(len(MUTATIONS))])
def test_planted_mistake_fails_a_pin(old, new):
    F = _mutant("fp8", old, new)
    failed = []
    for name, pin in ALL.items():
        try:
            if pin(F) != 0:
                failed.append(name)
        except Exception:
            failed.append(name)
    assert failed, "planted mistake passed every pin"
