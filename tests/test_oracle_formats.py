"""Pins of the oracle's number formats and quantizer against textbook tables, a library cast,
exhaustive exact-rational search and hand-derived fixtures (no GPU)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_e2m1_table_is_textbook():
    # OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa; code 1 is the subnormal 0.5.
    expect = []
    for code in range(8):
        e, m = code >> 1, code & 1
        expect.append(m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))
    assert list(nvfp4.E2M1_MAGNITUDES) == expect == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(nvfp4.e2m1_decode(np.arange(16))) == expect + [-v for v in expect]


def test_e4m3fn_decode_matches_torch_cast():
    b = np.arange(256, dtype=np.uint8)
    ours = nvfp4.e4m3fn_decode(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nvfp4.e4m3fn_decode(0x7E) == 448.0 and nvfp4.e4m3fn_decode(0x01) == 2.0 ** -9
    assert nvfp4.e4m3fn_decode(0x08) == 2.0 ** -6


def test_e4m3_rounding_matches_torch_cast_in_range():
    rng = np.random.default_rng(1)
    # fp32 values spread over the whole E4M3 range, including subnormals; below 448 torch's cast is RNE
    v = (2.0 ** rng.uniform(-12, np.log2(448), 200000)).astype(np.float32)
    ours = nvfp4.e4m3_rne_sat(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_ties_and_saturation():
    cases = {1.0625: 1.0, 1.1875: 1.25, 2.0 ** -10: 0.0, 3 * 2.0 ** -11: 2.0 ** -9,
             448.0: 448.0, 464.0: 448.0, 1e6: 448.0, 0.0: 0.0, 2.0 ** -9: 2.0 ** -9}
    for v, want in cases.items():
        assert nvfp4.e4m3fn_decode(nvfp4.e4m3_rne_sat(v)) == want, v


def test_e2m1_rounding_thresholds():
    # RNE on {0,.5,1,1.5,2,3,4,6}: midpoints .25,.75,1.25,1.75,2.5,3.5,5 go to the even code
    cases = {0.25: 0, 0.2500001: 1, 0.75: 2, 0.7499999: 1, 1.25: 2, 1.2500001: 3, 1.75: 4, 2.5: 4,
             2.5000001: 5, 3.5: 6, 3.4999999: 5, 5.0: 6, 5.0000001: 7, 6.0: 7, 100.0: 7, 0.0: 0}
    for r, want in cases.items():
        assert nvfp4.e2m1_rne_sat(r) == want, r


def _nearest_even_exact(q: Fraction, table):
    """Brute force: nearest entry of a table of Fractions by exhaustive search, ties to the even index."""
    best = None
    for i, t in enumerate(table):
        d = abs(q - t)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


E2M1_F = [Fraction(v).limit_denominator() for v in nvfp4.E2M1_MAGNITUDES]
E4M3_F = [Fraction(float(v)) for v in nvfp4.E4M3_MAGNITUDES]


@pytest.mark.parametrize("s_byte,g", [(0x38, 1.0), (0x01, 2.0 ** -3), (0x4D, 0.0123), (0x7E, 3.1e-4)])
def test_codes_exhaustive_bf16_vs_rational_search(s_byte, g):
    """All 65,536 bf16 inputs: code decision vs exhaustive exact-rational nearest-value search."""
    g = float(np.float32(g))
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32).astype(np.float64)
    x = x[np.isfinite(x)]
    s = float(nvfp4.e4m3fn_decode(s_byte))
    sg = s * g
    r = np.abs(x) / sg
    ours = nvfp4.e2m1_rne_sat(r)
    # exact check on the values near a boundary (and a random sample of the rest)
    sgF = Fraction(s) * Fraction(g)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    near = np.min(np.abs(r[:, None] - mids[None, :]), axis=1) < 1e-2
    rng = np.random.default_rng(0)
    pick = np.nonzero(near | (rng.random(r.shape[0]) < 0.02))[0]
    for i in pick:
        q = abs(Fraction(float(x[i]))) / sgF
        if q > 6:
            want = 7
        else:
            want = _nearest_even_exact(q, E2M1_F)
        assert ours[i] == want, (x[i], s, g)


def test_scale_decision_vs_rational_search():
    rng = np.random.default_rng(3)
    for _ in range(3000):
        g = float(np.float32(2.0 ** rng.uniform(-14, 2)))
        # amax: a bf16 value, often constructed to sit on or next to an E4M3 midpoint * 6g
        if rng.random() < 0.5:
            amax = float(torch.tensor(2.0 ** rng.uniform(-20, 12)).to(torch.bfloat16).float())
        else:
            i = rng.integers(0, 126)
            mid = (float(nvfp4.E4M3_MAGNITUDES[i]) + float(nvfp4.E4M3_MAGNITUDES[i + 1])) / 2
            amax = float(np.float32(mid * 6 * g))
            amax = float(np.nextafter(np.float32(amax), np.float32(rng.choice([-1, 1]) * np.inf))) \
                if rng.random() < 0.5 else amax
        got = int(nvfp4.e4m3_rne_sat(amax / (6 * g)))
        q = Fraction(amax) / (6 * Fraction(g))
        want = 0x7E if q >= 448 else _nearest_even_exact(q, E4M3_F)
        assert got == want, (amax, g)


def test_quantize_round_trip_of_representable_groups():
    """x = code * s * g exactly (bf16), with a +-6 in each group, must quantize back to (codes, s)."""
    rng = np.random.default_rng(5)
    R, K = 64, 256
    for g in [1.0, 2.0 ** -7, 2.0 ** 3]:
        codes = rng.integers(0, 16, size=(R, K), dtype=np.uint8)
        codes[:, ::32] = rng.choice([7, 15], size=(R, K // 32))       # one +-6 per group
        s = rng.integers(0x08, 0x70, size=(R, K // 32), dtype=np.uint8)
        x = nvfp4.e2m1_decode(codes) * np.repeat(nvfp4.e4m3fn_decode(s), 32, axis=1) * g
        assert np.array_equal(torch.tensor(x).to(torch.bfloat16).double().numpy(), x)  # exact in bf16
        pc, ps = nvfp4.quantize(x, g)
        assert np.array_equal(ps, s)
        assert np.array_equal(nvfp4.unpack_codes(pc), codes)


def test_quantize_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "pair_bitmask_example.json")))
    vals = np.array(ex["values"], dtype=np.float64)[None, :]
    vals[0, 24] = -0.0
    vals[0, 25] = -0.0
    codes, scales = nvfp4.quantize(vals, ex["global"])
    assert scales.tolist() == [[ex["scale_byte"]]]
    assert codes[0].tolist() == ex["dense_bytes"]
    back = nvfp4.dequantize(codes, scales, ex["global"])
    assert np.array_equal(back, vals)


def test_quantize_degenerate_groups():
    x = np.zeros((2, 64))
    x[1, :32] = -0.0
    x[1, 32:] = 1e-30                    # amax/(6g) below 2^-10: scale 0, magnitude codes 0
    c, s = nvfp4.quantize(x, 1.0)
    assert (s == 0).all()
    cc = nvfp4.unpack_codes(c)
    assert (cc[0] == 0).all() and (cc[1, :32] == 8).all() and (cc[1, 32:] == 0).all()
    # saturation: global 1/2688 and N(0,1)-sized values -> scale 448, codes clipped at 6
    g = float(np.float32(1) / np.float32(2688))
    x = np.full((1, 32), 3.0)
    x[0, 0] = -5.0
    c, s = nvfp4.quantize(x, g)
    assert s[0, 0] == 0x7E
    assert (nvfp4.unpack_codes(c)[0] == np.array([15] + [7] * 31)).all()


def test_admissible_contains_exact_and_rejects_far():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((8, 128))
    c, s = nvfp4.quantize(x, 0.01)
    err = np.full_like(x, 1e-9)
    assert nvfp4.check_admissible(x, err, 0.01, c, s).all()
    c2 = c.copy()
    c2[0, 0] ^= 0x3                      # move a code by more than the error allows
    ok = nvfp4.check_admissible(x, err, 0.01, c2, s)
    assert not ok[0, 0] and ok[1:].all()
