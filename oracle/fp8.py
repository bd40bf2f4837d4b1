"""FP8 (E4M3) latent-cache rows — TEST INFRASTRUCTURE.

The pages leave the cache's bytes per element open: the SyntaxRadar page
("Multi-Head Latent Attention: How DeepSeek Shrinks AI Memory", section
"What did DeepSeek's papers actually report?") says the served model
stored about 6 bits per cache element without saying how, and the
"Multi-Head Latent Attention (MLA)" page ("Against the alternatives")
treats cache quantisation as a separate axis that can be added to MLA.
This module is the reading the library adopts: each cache row
[c | k_pe] is stored as E4M3 codes times one power-of-two scale per row.

Format (the OCP 8-bit floating point specification, E4M3, as in
torch.float8_e4m3fn): bit 7 is the sign, bits 6-3 a biased exponent e
(bias 7), bits 2-0 a mantissa m.
  e = 0:       subnormal, value m/8 * 2^-6 (so the spacing there is 2^-9);
  1 <= e:      value (1 + m/8) * 2^(e-7);
  e = 15, m = 7: NaN (there are no infinities), so the largest finite
               magnitude is 1.75 * 2^8 = 448.
Encoding rounds to the nearest value, ties to the even mantissa; 464, the
midpoint between 448 and the step past it, rounds to 448 (even), and a
larger magnitude has no finite code and becomes NaN (sign kept).

Row quantiser: scale s = 2^k with k the smallest integer such that
amax <= 448 * 2^k (amax = the largest |value| of the fp32 row; s = 1 for a
row of zeros), but no smaller than -126 so that s and 1/s are normal fp32
numbers (rows below 448 * 2^-126 keep that scale and round towards
zero), then code = encode(value / s).  Because s is a power of two
the division is exact, every code * s is exactly representable in bf16,
and the scaled row's largest magnitude lies in (224, 448].  k is read off
the binary exponent of the fp32 amax, amax = f * 2^E with f in [0.5, 1):
k = E - 9 if f <= 0.875 (448 = 0.875 * 2^9), else E - 8 — a comparison, so
the decision needs no rounded division and is the same in any precision.

Functions: decode, encode (elementwise), quantize_rows, dequantize_rows.
Pinned in tests/test_oracle_fp8.py against torch.float8_e4m3fn casts (every
code, ties, subnormals, overflow), a brute-force search for k, and the
error bounds of round-to-nearest.
"""
import numpy as np

E4M3_MAX = 448.0
_NAN_CODE = 0x7F


def decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (uint8, any shape)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def encode(x) -> np.ndarray:
    """E4M3 codes (uint8) of real values, round to nearest, ties to even."""
    v = np.asarray(x, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    fin = np.where(np.isfinite(a), a, 0.0)  # NaN and inf are handled below
    # binade of a: a = f 2^E, f in [0.5, 1), so a lies in [2^(E-1), 2^E)
    _, E = np.frexp(fin)
    e_unb = np.maximum(E - 1, -6)          # below 2^-6 the spacing stays 2^-9
    step = np.exp2(e_unb - 3.0)            # spacing of the 8 mantissa values
    q = np.round(fin / step)               # numpy rounds halves to even
    # codes of one binade are consecutive integers (e_unb + 7) * 8 + (q - 8);
    # q = 16 carries into the next binade and a subnormal q in 0..8 lands on
    # codes 0..8 (code 8 = 2^-6, the smallest normal)
    mag_code = np.where(E - 1 < -6, q, (e_unb + 7) * 8 + (q - 8)).astype(np.int64)
    overflow = (a > 464.0) | np.isnan(a)
    mag_code = np.where(overflow, _NAN_CODE, mag_code)
    mag_code = np.where(a == 0, 0, mag_code)
    return ((sign << 7) | mag_code).astype(np.uint8)


def row_scale_exponents(rows) -> np.ndarray:
    """k per row: the smallest integer >= -126 with amax <= 448 * 2^k (0 for zero rows)."""
    r = np.asarray(rows, dtype=np.float32)
    amax = np.max(np.abs(r), axis=-1).astype(np.float64)
    f, E = np.frexp(amax)
    k = np.maximum(np.where(f <= 0.875, E - 9, E - 8), -126)
    return np.where(amax == 0, 0, k).astype(np.int64)


def quantize_rows(rows):
    """(codes uint8 [..., R], scales float32 [...]) of fp32 rows [..., R]."""
    r = np.asarray(rows, dtype=np.float32)
    k = row_scale_exponents(r)
    scales = np.exp2(k.astype(np.float64)).astype(np.float32)
    codes = encode(r.astype(np.float64) / scales[..., None].astype(np.float64))
    return codes, scales


def dequantize_rows(codes, scales) -> np.ndarray:
    """float64 rows code * scale."""
    return decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]
