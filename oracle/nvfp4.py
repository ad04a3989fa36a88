"""NVFP4 number formats and the per-32 group quantizer, in float64.

Source: model cards "Qwen3.5-397B-A17B-P48NVFP4-MoESQ" and "Qwen3-30B-A3B-P48NVFP4-MoESQ",
"Compression details" table: weights are NVFP4 (E2M1 values) with one FP8-E4M3 scale per 32 dense K
elements and an FP32 per-tensor global scale; activations are NVFP4 with dynamic per-32 group scales
and an FP32 global scale stored per expert linear.

Readings where the pages are silent:

* value = e2m1(code) * e4m3(scale) * global (the global is multiplicative);
* scale = E4M3 round-to-nearest-even of the exact real quotient amax / (6 * global), saturating at 448;
* code  = E2M1 round-to-nearest-even of the exact real quotient x / (scale * global), saturating at 6;
  a group whose scale rounds to 0 gets magnitude code 0 everywhere;
* the code's sign bit is the sign bit of x (so -0 and small negatives give 0x8);
* two codes per byte, the lower-K element in the low nibble; E4M3 is the OCP "FN" variant.
"""
from __future__ import annotations

import numpy as np

#: E2M1 magnitudes of codes 0..7 (1 sign, 2 exponent, 1 mantissa bit; bias 1; code 1 is subnormal 0.5).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e4m3fn_decode(b) -> np.ndarray:
    """OCP E4M3FN byte -> float64: sign.eeee.mmm, bias 7, subnormal m*2^-9, 0x7F/0xFF are NaN, no inf."""
    b = np.asarray(b, dtype=np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


#: Values of the finite non-negative E4M3FN bytes 0x00..0x7E (increasing with the byte).
E4M3_MAGNITUDES = e4m3fn_decode(np.arange(0x7F))
E4M3_MAX = 448.0


def e2m1_decode(c) -> np.ndarray:
    """E2M1 4-bit code -> float64 (bit 3 is the sign)."""
    c = np.asarray(c, dtype=np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def round_to_table_even(v, table: np.ndarray) -> np.ndarray:
    """Index of the entry of the increasing non-negative ``table`` nearest to ``v`` (v >= 0).

    Ties go to the even index (for E2M1 and E4M3 the index parity is the mantissa parity, so this is
    round-half-to-even); values beyond the last entry saturate to it. The comparison is against the
    exact midpoint of two neighbours (representable in float64), so for float64 ``v`` it is exact.
    """
    v = np.asarray(v, dtype=np.float64)
    n = len(table)
    hi = np.searchsorted(table, v, side="left")          # first entry >= v
    hi_c = np.clip(hi, 1, n - 1)
    lo_c = hi_c - 1
    mid = (table[lo_c] + table[hi_c]) * 0.5
    pick_hi = (v > mid) | ((v == mid) & (hi_c % 2 == 0))
    idx = np.where(pick_hi, hi_c, lo_c)
    idx = np.where(hi == 0, 0, idx)                       # v <= table[0]
    idx = np.where(hi >= n, n - 1, idx)                   # v above the top: saturate
    return idx.astype(np.int64)


def e4m3_rne_sat(v) -> np.ndarray:
    """E4M3FN byte of the non-negative real ``v``: nearest, ties to even, saturating at 448 (0x7E).
    In particular v < 2^-10 gives 0 and the tie v = 2^-10 gives 0 (the even neighbour)."""
    return round_to_table_even(v, E4M3_MAGNITUDES).astype(np.uint8)


def e2m1_rne_sat(r) -> np.ndarray:
    """E2M1 magnitude code (0..7) of the non-negative real ``r``: nearest, ties to even, saturating at 6."""
    return round_to_table_even(r, E2M1_MAGNITUDES).astype(np.uint8)


def quantize(x, g):
    """Per-32 group NVFP4 quantization of rows ``x`` [R, K] with per-row global ``g`` [R] (or scalar).

    For each row and each group of 32 consecutive K elements:
      amax = max |x_i|;  s = E4M3_RNE_sat(amax / (6 g));  code_i = sign(x_i) | E2M1_RNE_sat(|x_i| / (s g)).
    Returns (codes u8 [R, K/2] two per byte with the lower K in the low nibble, scales u8 [R, K/32]).

    Exactness: inputs are bf16 or fp32 values (<= 24 significant bits) and g is fp32. 6g and s*g are
    exact in float64, so each quotient is one correctly rounded float64 division. A rounding midpoint
    has <= 5 significant bits, so a quotient that is not exactly a midpoint lies at least ~2^-32
    (relative) from it, far beyond float64's 2^-53: the float64 comparison takes the exact decision,
    ties included. For float64 inputs carrying their own rounding (the FFN's intermediate) the decision
    is exact for the float64 value given.
    """
    x = np.asarray(x, dtype=np.float64)
    R, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    g = np.broadcast_to(np.asarray(g, dtype=np.float64).reshape(-1, 1), (R, 1))
    xg = x.reshape(R, K // 32, 32)
    ax = np.abs(xg)
    amax = ax.max(axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(g > 0, amax / (6.0 * g), 0.0)
    s_code = e4m3_rne_sat(v)
    sg = E4M3_MAGNITUDES[s_code] * g                       # [R, K/32]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(sg[..., None] > 0, ax / sg[..., None], 0.0)
    mag = e2m1_rne_sat(r)
    code = mag | (np.signbit(xg).astype(np.uint8) << 3)
    code = code.reshape(R, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_code


def unpack_codes(packed) -> np.ndarray:
    """u8 [R, K/2] -> 4-bit codes [R, K] (low nibble = even K)."""
    packed = np.asarray(packed, dtype=np.uint8)
    R, Kh = packed.shape
    c = np.empty((R, 2 * Kh), dtype=np.uint8)
    c[:, 0::2] = packed & 0xF
    c[:, 1::2] = packed >> 4
    return c


def dequantize(packed, scales, g) -> np.ndarray:
    """NVFP4 bytes -> float64 values e2m1(code) * e4m3(scale of its 32-group) * g (per row)."""
    c = unpack_codes(packed)
    R, K = c.shape
    s = e4m3fn_decode(scales)                              # [R, K/32]
    g = np.broadcast_to(np.asarray(g, dtype=np.float64).reshape(-1, 1), (R, 1))
    return e2m1_decode(c) * np.repeat(s, 32, axis=1) * g


def admissible(x, x_err, g):
    """The set of correct encodings of each 32-group when each x_i is only known to within x_err_i.

    An implementation that computes x in a lower precision (the FFN's fp32 intermediate) may land on
    either side of a rounding boundary that lies within its error bound; both results are correct.
    Returns (scale_lo, scale_hi, code_lo, code_hi) where for each group the admissible scale bytes are
    scale_lo..scale_hi and, evaluated per admissible scale inside ``check_admissible``, codes lie within
    the nearest-even roundings of the interval ends.
    """
    x = np.asarray(x, dtype=np.float64)
    err = np.asarray(x_err, dtype=np.float64)
    R, K = x.shape
    g = np.broadcast_to(np.asarray(g, dtype=np.float64).reshape(-1, 1), (R, 1))
    ax = np.abs(x).reshape(R, K // 32, 32)
    er = err.reshape(R, K // 32, 32)
    amax = ax.max(axis=2)
    aerr = er.max(axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        v_lo = np.where(g > 0, np.maximum(amax - aerr, 0.0) / (6.0 * g), 0.0)
        v_hi = np.where(g > 0, (amax + aerr) / (6.0 * g), 0.0)
    return e4m3_rne_sat(v_lo), e4m3_rne_sat(v_hi)


def check_admissible(x, x_err, g, codes, scales):
    """True per group when (scales, codes) is one of the correct encodings of x known to within x_err.

    Admissible: the scale byte is between the roundings of (amax -/+ max err)/(6g); for that scale each
    magnitude code is between the roundings of (|x_i| -/+ err_i)/(s g); the sign bit equals sign(x_i)
    unless |x_i| <= err_i (then either sign is admissible).
    """
    x = np.asarray(x, dtype=np.float64)
    err = np.asarray(x_err, dtype=np.float64)
    R, K = x.shape
    g = np.broadcast_to(np.asarray(g, dtype=np.float64).reshape(-1, 1), (R, 1))
    s_lo, s_hi = admissible(x, err, g)
    scales = np.asarray(scales, dtype=np.uint8)
    ok_s = (scales >= s_lo) & (scales <= s_hi)
    sg = E4M3_MAGNITUDES[np.minimum(scales, 0x7E)] * g
    ax = np.abs(x).reshape(R, K // 32, 32)
    er = err.reshape(R, K // 32, 32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r_lo = np.where(sg[..., None] > 0, np.maximum(ax - er, 0.0) / sg[..., None], 0.0)
        r_hi = np.where(sg[..., None] > 0, (ax + er) / sg[..., None], 0.0)
    c = unpack_codes(codes).reshape(R, K // 32, 32)
    mag = c & 7
    ok_m = (mag >= e2m1_rne_sat(r_lo)) & (mag <= e2m1_rne_sat(r_hi))
    sign = (c >> 3) & 1
    ok_sign = (sign == np.signbit(x.reshape(R, K // 32, 32))) | (ax <= er)
    return ok_s & (ok_m & ok_sign).all(axis=2)


def ambiguous_groups(x, x_err, g):
    """True per group when more than one encoding is admissible (``check_admissible``): the scale
    interval holds two bytes, or at the nearest-even scale some code interval holds two codes, or some
    |x_i| <= err_i (either sign). Groups that are not ambiguous have exactly one correct encoding."""
    x = np.asarray(x, dtype=np.float64)
    err = np.asarray(x_err, dtype=np.float64)
    R, K = x.shape
    g = np.broadcast_to(np.asarray(g, dtype=np.float64).reshape(-1, 1), (R, 1))
    s_lo, s_hi = admissible(x, err, g)
    _, s_mid = quantize(x, g)
    sg = E4M3_MAGNITUDES[s_mid] * g
    ax = np.abs(x).reshape(R, K // 32, 32)
    er = err.reshape(R, K // 32, 32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r_lo = np.where(sg[..., None] > 0, np.maximum(ax - er, 0.0) / sg[..., None], 0.0)
        r_hi = np.where(sg[..., None] > 0, (ax + er) / sg[..., None], 0.0)
    code_amb = (e2m1_rne_sat(r_lo) != e2m1_rne_sat(r_hi)).any(axis=2)
    sign_amb = (ax <= er).any(axis=2)
    return (s_lo != s_hi) | code_amb | sign_amb
