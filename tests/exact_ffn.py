"""Exact evaluation of the paired-4:8 NVFP4 MoE FFN on tiny shapes, as a pin for the float64 oracle.

Written from the number-format definitions (E2M1: 1 sign, 2 exponent, 1 mantissa bit, bias 1;
E4M3FN: bias 7, 3 mantissa bits, subnormals m * 2^-9, 0x7F NaN) and the FFN of the model cards
("Qwen3.5-397B-A17B-P48NVFP4-MoESQ", "Compression details": W4A4 gate_proj / up_proj / down_proj of
the routed experts, activations quantized per 32 with a per-expert-linear global). It shares no code
with ``oracle/``: values are enumerated from the format tables, every rounding is a nearest-value
search over the whole table with ties to the even code (not a boundary formula), every product and
sum is an exact rational (``fractions.Fraction``), and silu uses ``decimal`` at 60 significant
digits. The expert FFN is y = W2 · q(silu(g) · u) with [g | u] = W13 · q(x), the gate rows first,
each pair's output times its router weight and the k outputs of a token summed.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

PREC = 60

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
# finite non-negative E4M3FN bytes 0x00 .. 0x7E
E4M3 = [Fraction(b & 7, 512) if b >> 3 == 0 else (1 + Fraction(b & 7, 8)) * Fraction(2) ** ((b >> 3) - 7)
        for b in range(0x7F)]


def _dec(f: Fraction) -> Decimal:
    with localcontext() as c:
        c.prec = PREC
        return Decimal(f.numerator) / Decimal(f.denominator)


E2M1_D = [_dec(v) for v in E2M1]
E4M3_D = [_dec(v) for v in E4M3]


def nearest_even(v, table):
    """Index of the table entry nearest to v >= 0 by exhaustive search; equal distances go to the
    even index. Returns (index, margin) with margin = (second-best distance - best distance), so a
    caller working on an approximation of v can tell whether the decision is resolved."""
    d = [abs(t - v) for t in table]
    order = sorted(range(len(table)), key=lambda i: (d[i], i % 2, i))
    best = order[0]
    ties = [i for i in order if d[i] == d[best]]
    if len(ties) > 1:
        best = [i for i in ties if i % 2 == 0][0]
        return best, 0
    return best, d[order[1]] - d[best]


def frac(x) -> Fraction:
    return Fraction(float(x))


def quantize_group(vals, g, exact=True):
    """NVFP4 codes (4-bit, sign in bit 3) and scale byte of one 32-group for global g.
    vals: floats (exact inputs, taken as exact rationals; the sign bit of -0.0 counts) or Decimals
    (transcendental inputs known to PREC digits).
    Returns (codes, scale_byte, min_margin) where min_margin is the smallest relative decision margin
    (0 for exact ties; None when the inputs are exact, so every decision is exact)."""
    if exact:
        gq = frac(g)
        fv = [frac(v) for v in vals]
        amax = max(abs(v) for v in fv)
        sb, _ = nearest_even(amax / (6 * gq), E4M3)
        s = E4M3[sb]
        codes = []
        for v, f in zip(vals, fv):
            m = 0 if s == 0 else nearest_even(abs(f) / (s * gq), E2M1)[0]
            codes.append(m | (8 if math.copysign(1.0, float(v)) < 0 else 0))
        return codes, sb, None
    with localcontext() as c:
        c.prec = PREC
        gd = _dec(frac(g))
        amax = max(abs(v) for v in vals)
        q = amax / (6 * gd)
        sb, mg = nearest_even(q, E4M3_D)
        margin = mg / q if q else Decimal(1)
        s = E4M3_D[sb]
        codes = []
        for v in vals:
            if s == 0:
                m = 0
            else:
                r = abs(v) / (s * gd)
                m, mgc = nearest_even(r, E2M1_D)
                if r:
                    margin = min(margin, mgc / r)
            codes.append(m | (8 if v.is_signed() else 0))
        return codes, sb, margin


def decode(code: int, sb: int, g) -> Fraction:
    v = E2M1[code & 7] * E4M3[sb] * frac(g)
    return -v if code & 8 else v


def dense_weight(packed, mask, scale, gw):
    """Exact values [N][K] of one expert linear in pair-bitmask storage: chunk c of 8 K (4 bytes)
    takes mask nibble (mask[c/2] >> 4 (c % 2)) & 15; set bit i keeps byte i, the kept bytes of the
    chunk in K order; a byte holds two codes, the lower K in the low nibble. gw: 1 global, or 2
    (gate rows first, then up rows)."""
    packed, mask, scale = (np.asarray(a) for a in (packed, mask, scale))
    N, Kq = packed.shape
    K = Kq * 4
    gw = [float(v) for v in np.ravel(gw)]
    out = []
    for n in range(N):
        g = gw[0] if len(gw) == 1 or n < N // 2 else gw[1]
        row = []
        for c in range(K // 8):
            nib = (int(mask[n, c // 2]) >> (4 * (c % 2))) & 15
            kept = [i for i in range(4) if nib >> i & 1]
            assert len(kept) == 2, "a pair-bitmask nibble keeps exactly two bytes"
            bytes4 = [0, 0, 0, 0]
            bytes4[kept[0]] = int(packed[n, 2 * c])
            bytes4[kept[1]] = int(packed[n, 2 * c + 1])
            for b in bytes4:
                for code in (b & 15, b >> 4):
                    kk = len(row)
                    row.append(decode(code, int(scale[n, kk // 32]), g))
        out.append(row)
    return out


def ffn(x, ids, wts, w13, w2, g13, g2):
    """Exact MoE FFN. x [T][H] floats (bf16 values), ids/wts [T][k], w13/w2 = (packed, mask, scale,
    global) indexable by expert, g13/g2 per-expert activation globals.
    Returns (out [T][H] Fractions, mag [T][H] Fractions = sum of |terms| of the down sums,
    per-pair intermediates {(t, j): (a13 codes/scales, h Decimals, a2 codes/scales, min margin)})."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    k = np.asarray(ids).shape[1]
    W13, W2 = {}, {}
    out = [[Fraction(0)] * H for _ in range(T)]
    mag = [[Fraction(0)] * H for _ in range(T)]
    inter = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t][j])
            if e < 0:
                continue
            if e not in W13:
                W13[e] = dense_weight(w13[0][e], w13[1][e], w13[2][e], w13[3][e])
                W2[e] = dense_weight(w2[0][e], w2[1][e], w2[2][e], w2[3][e])
            I = len(W13[e]) // 2
            xs = [float(v) for v in x[t]]
            a_codes, a_scales, xhat = [], [], []
            for gi in range(H // 32):
                cs, sb, _ = quantize_group(xs[32 * gi:32 * gi + 32], g13[e])
                a_codes += cs
                a_scales.append(sb)
                xhat += [decode(c, sb, g13[e]) for c in cs]
            gu = [sum((a * w for a, w in zip(xhat, W13[e][n])), Fraction(0)) for n in range(2 * I)]
            with localcontext() as c:
                c.prec = PREC
                h = []
                for i in range(I):
                    gd, ud = _dec(gu[i]), _dec(gu[I + i])
                    h.append(gd / (1 + (-gd).exp()) * ud)
            h_codes, h_scales, margin, hhat = [], [], Decimal(1), []
            for gi in range(I // 32):
                cs, sb, mg = quantize_group(h[32 * gi:32 * gi + 32], g2[e], exact=False)
                h_codes += cs
                h_scales.append(sb)
                margin = min(margin, mg)
                hhat += [decode(c2, sb, g2[e]) for c2 in cs]
            w = frac(wts[t][j])
            for n in range(H):
                terms = [a * b for a, b in zip(hhat, W2[e][n])]
                out[t][n] += w * sum(terms, Fraction(0))
                mag[t][n] += abs(w) * sum((abs(v) for v in terms), Fraction(0))
            inter[(t, j)] = (a_codes, a_scales, h, h_codes, h_scales, margin)
    return out, mag, inter
