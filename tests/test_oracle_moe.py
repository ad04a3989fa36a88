"""Pins of the oracle's permutation, grouped GEMM and FFN (no GPU): brute force, exact rationals,
library reductions and metamorphic relations."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import compress, moe, nvfp4, pairbitmask
import synth


def test_permute_vs_brute_force():
    rng = np.random.default_rng(0)
    T, k, E = 37, 4, 9
    ids = rng.integers(-1, E, size=(T, k))
    ids[3, :] = [2, 2, 5, -1]                       # a duplicate id counts twice; -1 is dropped
    counts, offsets, sorted_pairs, inv = moe.permute(ids, E)
    brute = [t * k + j for e in range(E) for t in range(T) for j in range(k) if ids[t, j] == e]
    assert sorted_pairs.tolist() == brute
    assert counts.tolist() == [int((ids == e).sum()) for e in range(E)]
    assert offsets[0] == 0 and offsets[-1] == len(brute) and (np.diff(offsets) == counts).all()
    for p in range(T * k):
        assert (inv[p] == -1) == (ids.ravel()[p] == -1)
        if inv[p] >= 0:
            assert sorted_pairs[inv[p]] == p
    with pytest.raises(ValueError):
        moe.permute(np.array([[E]]), E)


def _exact_value(code, sbyte, g):
    return Fraction(float(nvfp4.e2m1_decode(code))) * Fraction(float(nvfp4.e4m3fn_decode(sbyte))) * Fraction(float(g))


def test_grouped_gemm_vs_exact_rationals():
    """Two experts, tiny shapes: every output against an exact rational sum."""
    E, N, K = 2, 6, 64
    packed, mask, scale, gw = synth.random_sparse_weights(3, E, N, K, G=2)
    a_codes, a_scales = synth.random_act_codes(4, 5, K)
    a_scales = np.clip(a_scales, 0x20, 0x5F)
    a_global = np.array([0.011, 0.37], np.float32)
    offsets = np.array([0, 2, 5])
    out = moe.grouped_gemm(a_codes, a_scales, a_global, offsets, packed, mask, scale, gw)
    ac = nvfp4.unpack_codes(a_codes)
    for e in range(E):
        dense = pairbitmask.unpack(packed[e], mask[e])
        wc = nvfp4.unpack_codes(dense)
        for r in range(offsets[e], offsets[e + 1]):
            for n in range(N):
                g_w = gw[e, 0] if n < N // 2 else gw[e, 1]
                acc = Fraction(0)
                mag = Fraction(0)
                for kk in range(K):
                    term = _exact_value(ac[r, kk], a_scales[r, kk // 32], a_global[e]) * \
                        _exact_value(wc[n, kk], scale[e, n, kk // 32], g_w)
                    acc += term
                    mag += abs(term)
                # float64 summation of K exact-ish products: error <= K * 2^-53 * sum|terms|
                assert abs(Fraction(float(out[r, n])) - acc) <= Fraction(K, 2 ** 53) * mag, (e, r, n)


def test_grouped_gemm_single_expert_is_matmul_of_dequantized():
    N, K, M = 16, 128, 9
    packed, mask, scale, gw = synth.random_sparse_weights(5, 1, N, K)
    a_codes, a_scales = synth.random_act_codes(6, M, K)
    out = moe.grouped_gemm(a_codes, a_scales, [0.5], [0, M], packed, mask, scale, gw)
    W = compress.decompress(packed[0], mask[0], scale[0], gw[0, 0])
    X = nvfp4.dequantize(a_codes, a_scales, 0.5)
    assert np.allclose(out, np.matmul(X, W.T), rtol=1e-13, atol=0)


def _tiny_layer(seed, E, H, I):
    w13 = [[], [], [], []]
    w2 = [[], [], [], []]
    for e in range(E):
        g, u, d = synth.expert_dense_weights(seed, e, H, I)
        pg, mg, sg, gg = compress.compress(g.numpy())
        pu, mu, su, gu = compress.compress(u.numpy())
        for lst, vals in zip(w13, [np.concatenate([pg, pu]), np.concatenate([mg, mu]),
                                   np.concatenate([sg, su]), np.array([gg, gu], np.float32)]):
            lst.append(vals)
        for lst, vals in zip(w2, compress.compress(d.numpy())):
            lst.append(vals if np.ndim(vals) else np.array([vals], np.float32))
    return [np.stack(v) for v in w13], [np.stack(v) for v in w2]


def test_ffn_top1_equals_single_expert_and_is_equivariant():
    E, H, I, T = 3, 64, 32, 12
    w13, w2 = _tiny_layer(9, E, H, I)
    x = synth.activations(1, T, H).float().numpy()
    g13 = np.full(E, np.float32(0.002), np.float32)
    g2 = np.full(E, np.float32(0.0005), np.float32)
    ids = np.array([[t % E] for t in range(T)], np.int32)
    wts = np.ones((T, 1), np.float32)
    out = moe.moe_ffn(x, ids, wts, w13, w2, g13, g2)
    # single-expert FFN of token t through its expert, written out stage by stage
    for t in range(T):
        e = t % E
        c, s = nvfp4.quantize(x[t:t + 1], g13[e])
        W13 = moe.dequant_weight(w13[0][e], w13[1][e], w13[2][e], w13[3][e])
        gu = nvfp4.dequantize(c, s, g13[e]) @ W13.T
        h = gu[:, :I] / (1 + np.exp(-gu[:, :I])) * gu[:, I:]
        c2, s2 = nvfp4.quantize(h, g2[e])
        y = nvfp4.dequantize(c2, s2, g2[e]) @ moe.dequant_weight(w2[0][e], w2[1][e], w2[2][e], w2[3][e]).T
        assert np.allclose(out[t], y[0], rtol=1e-12, atol=1e-15)
    # shuffling tokens permutes the output rows
    perm = np.random.default_rng(0).permutation(T)
    out_p = moe.moe_ffn(x[perm], ids[perm], wts[perm], w13, w2, g13, g2)
    assert np.allclose(out_p, out[perm], rtol=1e-13, atol=1e-16)


def test_ffn_topk_is_weighted_sum_of_top1():
    E, H, I, T, k = 4, 64, 32, 6, 3
    w13, w2 = _tiny_layer(10, E, H, I)
    x = synth.activations(2, T, H).float().numpy()
    ids, wts = synth.routing(3, T, E, k)
    g13 = np.full(E, np.float32(0.002), np.float32)
    g2 = np.full(E, np.float32(0.0005), np.float32)
    out = moe.moe_ffn(x, ids, wts, w13, w2, g13, g2)
    acc = np.zeros_like(out)
    for j in range(k):
        acc += moe.moe_ffn(x, ids[:, j:j + 1], wts[:, j:j + 1], w13, w2, g13, g2)
    assert np.allclose(out, acc, rtol=1e-12, atol=1e-15)
    # dropping a pair (-1) removes exactly its term
    ids2 = ids.copy()
    ids2[:, 2] = -1
    out2 = moe.moe_ffn(x, ids2, wts, w13, w2, g13, g2)
    out_j2 = moe.moe_ffn(x, ids[:, 2:3], wts[:, 2:3], w13, w2, g13, g2)
    assert np.allclose(out2 + out_j2, out, rtol=1e-12, atol=1e-15)


def test_synth_routing_shapes():
    w = synth.WORKLOADS["qwen3_30b_prefill"]
    ids, wts = synth.routing(0, w.T, w.E, w.k, w.routing, w.zipf_s, w.zipf_beta)
    counts = np.bincount(ids.ravel(), minlength=128)
    assert counts.max() > 5 * counts.mean() and (counts == 0).sum() >= 1
    assert np.allclose(wts.sum(axis=1), 1, atol=1e-6)
    assert (np.diff(np.sort(ids, axis=1), axis=1) > 0).all()        # distinct experts per token


# ---- router (route_topk) pins: the selection against a rank definition counted pair by pair, the
# weights against closed forms

def _rank_select(l, k):
    """Experts of one token by a counting definition: rank_i = #{j : l_j > l_i, or l_j == l_i and j < i}."""
    E = len(l)
    rank = [sum(1 for j in range(E) if l[j] > l[i] or (l[j] == l[i] and j < i)) for i in range(E)]
    return [i for r in range(k) for i in range(E) if rank[i] == r]


def test_route_topk_selection_vs_rank_count():
    rng = np.random.default_rng(5)
    for E, k in ((6, 2), (9, 4), (16, 16), (33, 8)):
        l = rng.integers(-3, 4, size=(20, E)).astype(np.float64)      # many equal logits
        ids, w = moe.route_topk(l, k)
        for t in range(20):
            assert ids[t].tolist() == _rank_select(l[t].tolist(), k)
        assert np.all(np.diff(w, axis=1) <= 0)                         # listed by decreasing weight


def test_route_topk_weights_closed_forms():
    rng = np.random.default_rng(6)
    l = rng.standard_normal((50, 12))
    ids, w = moe.route_topk(l, 4)
    sel = np.take_along_axis(l, ids, axis=1)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    # ratios of weights are exp(differences of logits), whatever the normalization
    assert np.allclose(w[:, 1:] / w[:, :1], np.exp(sel[:, 1:] - sel[:, :1]), rtol=1e-13)
    # without renormalization the weights are the softmax probabilities: all of them sum to 1
    ids_all, p_all = moe.route_topk(l, 12, renormalize=False)
    assert np.allclose(p_all.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    _, p4 = moe.route_topk(l, 4, renormalize=False)
    assert np.allclose(p4, p_all[:, :4], rtol=0, atol=0)
    # equal logits: the first k ids, weight 1/k each
    ids_eq, w_eq = moe.route_topk(np.full((3, 10), 0.7), 3)
    assert ids_eq.tolist() == [[0, 1, 2]] * 3 and np.allclose(w_eq, 1.0 / 3, rtol=0, atol=1e-16)
    # a shift of all logits of a token changes nothing
    ids_s, w_s = moe.route_topk(l + 123.25, 4)
    assert np.array_equal(ids_s, ids) and np.allclose(w_s, w, rtol=1e-12)


def _nearest_e4m3_brute(v: Fraction) -> int:
    """The finite E4M3FN byte (0x00..0x7E) nearest to v >= 0 by exact rational distance, ties to the
    even byte (the byte's low bit is the mantissa's)."""
    best = None
    for c in range(0x7F):
        d = abs(Fraction(float(nvfp4.e4m3fn_decode(np.uint8(c)))) - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def _fp32_nearest(q: Fraction) -> np.float32:
    """The fp32 nearest to the positive rational q (ties to even), found among neighbours."""
    c = np.float32(float(q))
    cands = [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))]
    dist = [abs(Fraction(float(x)) - q) for x in cands]
    best = min(dist)
    picks = [x for x, d in zip(cands, dist) if d == best]
    return picks[0] if len(picks) == 1 else [x for x in picks if int(x.view(np.uint32)) % 2 == 0][0]


@pytest.mark.parametrize("gg,gu", [(1.0, 3.0), (3.0, 1.0), (1e-3, 7.3e-1), (0.37, 0.0021), (2.5e-4, 2.5e-4 * 1.0001)])
def test_fold_gate_up_globals_vs_brute_force(gg, gu):
    """Every folded up scale is the nearest E4M3 to e4m3(s) * fp32(g_up / g_gate), by exact rationals
    over all finite codes (ratios far from 1 reach both saturation at 448 and underflow to 0)."""
    rng = np.random.default_rng(int(gu * 1e6) % 1000)
    I, G = 16, 8
    scale = rng.integers(0, 0x7F, size=(2 * I, G), dtype=np.uint8)
    scale[I, :4] = [0x00, 0x01, 0x7E, 0x08]                   # zero, smallest subnormal, 448, 2^-6
    scale[I + 1, :3] = [0x7F, 0x80, 0xC5]                     # NaN and negative bytes: not scales
    gw = np.array([gg, gu], np.float32)
    out, gw2 = moe.fold_gate_up_globals(scale, gw)
    assert np.array_equal(out[:I], scale[:I])                 # gate rows untouched
    assert gw2.dtype == np.float32 and gw2[0] == gw[0] and gw2[1] == gw[0]
    r = _fp32_nearest(Fraction(float(gw[1])) / Fraction(float(gw[0])))
    for (i, j), s in np.ndenumerate(scale[I:]):
        if s == 0 or s >= 0x7F:
            assert out[I + i, j] == s                         # zero, and bytes that are not scales
            continue
        v = Fraction(float(nvfp4.e4m3fn_decode(s))) * Fraction(float(r))
        want = _nearest_e4m3_brute(v)
        assert out[I + i, j] == want, (i, j, int(s), float(v))


def test_fold_gate_up_globals_identities():
    """Equal globals: nothing changes. A power-of-two ratio keeping every scale in E4M3's normal range:
    the dequantized weights, and so the FFN, are exactly those of the unfolded layer."""
    E, H, I, T, k = 3, 64, 32, 8, 2
    w13, w2 = _tiny_layer(11, E, H, I)
    for e in range(E):
        same = np.array([w13[3][e][0], w13[3][e][0]], np.float32)
        out, gw = moe.fold_gate_up_globals(w13[2][e], same)
        assert np.array_equal(out, w13[2][e]) and np.array_equal(gw, same)
    # rebuild the up half with globals 4x the gate's and scales in [2^-4, 112] (no saturation or
    # subnormals after a x4 fold)
    rng = np.random.default_rng(12)
    f13 = [a.copy() for a in w13]
    for e in range(E):
        up = f13[2][e][I:]
        up[...] = rng.integers(0x18, 0x6E, size=up.shape, dtype=np.uint8)   # 2^-4 .. 112
        f13[3][e] = np.array([w13[3][e][0], w13[3][e][0] * 4], np.float32)
    g13 = np.full(E, np.float32(0.002), np.float32)
    g2 = np.full(E, np.float32(0.0005), np.float32)
    x = synth.activations(4, T, H).float().numpy()
    ids, wts = synth.routing(5, T, E, k)
    ref = moe.moe_ffn(x, ids, wts, f13, w2, g13, g2)
    folded = [a.copy() for a in f13]
    for e in range(E):
        folded[2][e], folded[3][e] = moe.fold_gate_up_globals(f13[2][e], f13[3][e])
        assert np.array_equal(moe.dequant_weight(*(a[e] for a in folded)),
                              moe.dequant_weight(*(a[e] for a in f13)))
    assert np.array_equal(moe.moe_ffn(x, ids, wts, folded, w2, g13, g2), ref)
