"""Token->expert permutation, grouped sparse GEMM and MoE FFN, in float64.

Sources: model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ" (header: 512 routed experts with 10 active;
"Compression details": the routed experts' gate_proj, up_proj and down_proj are W4A4 NVFP4 with
paired-4:8 weights, activations quantized per 32 with a global stored per expert linear; the kernel is
a paired-4:8 sparse NVFP4 *grouped* GEMM); model cards "Qwen3.8-Flash-Next-P48NVFP4-MoESQ" and
"Qwen3-30B-A3B-P48NVFP4-MoESQ" (gate and up projections carry separate global scales).

Readings where the pages are silent: the expert FFN is down(quant(silu(gate) * up)) with
silu(v) = v / (1 + exp(-v)); gate rows come first in the fused gate|up weight; each expert's gate and
up outputs take their own weight global; activations are quantized per (token, expert) row with that
expert's global; the intermediate is kept unrounded before its quantization; each expert's down
output is multiplied by its router weight and the k results of a token are summed; the permutation is
stable by (expert, flattened pair index t*k + j); an expert id of -1 drops the pair.
"""
from __future__ import annotations

import numpy as np

from . import nvfp4, pairbitmask


def permute(topk_ids, E: int):
    """Stable grouping of the pairs p = t*k + j by expert.

    Returns counts [E], offsets [E+1] (exclusive prefix of counts), sorted_pairs [P'] (pair ids in
    (expert, p) order) and inv [T*k] (row of pair p in the sorted order, -1 for a dropped pair).
    """
    flat = np.asarray(topk_ids, dtype=np.int64).ravel()
    if ((flat < -1) | (flat >= E)).any():
        raise ValueError("expert id outside [-1, E)")
    live = np.nonzero(flat >= 0)[0]
    sorted_pairs = live[np.argsort(flat[live], kind="stable")]
    counts = np.bincount(flat[live], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    inv = np.full(flat.shape[0], -1, dtype=np.int64)
    inv[sorted_pairs] = np.arange(sorted_pairs.shape[0])
    return counts.astype(np.int64), offsets.astype(np.int64), sorted_pairs.astype(np.int64), inv


def route_topk(logits, k: int, renormalize: bool = True):
    """Router of a MoE layer (the BF16 `mlp.gate` the model cards leave uncompressed; the pages do not
    spell its rule, the reading taken is the usual softmax top-k): probabilities p = softmax(logits)
    over the E experts in float64, the k largest p per token, equal p going to the lower expert id,
    listed by decreasing p; their weights are p renormalized over the k picks when ``renormalize``,
    else p itself.

    logits [T, E] -> ids int64 [T, k], weights float64 [T, k].
    """
    z = np.asarray(logits, dtype=np.float64)
    if z.ndim != 2 or not 1 <= k <= z.shape[1]:
        raise ValueError("logits [T, E] with 1 <= k <= E")
    e = np.exp(z - z.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :k]        # stable: equal p keep id order
    w = np.take_along_axis(p, ids, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int64), w


def weight_rows_global(gw_e, N: int) -> np.ndarray:
    """Per-row weight global of one expert linear: G=1 -> all rows; G=2 -> rows [0,N/2) take gw[0]
    (gate), rows [N/2,N) take gw[1] (up)."""
    gw_e = np.asarray(gw_e, dtype=np.float64).ravel()
    if gw_e.shape[0] == 1:
        return np.full(N, gw_e[0])
    if gw_e.shape[0] == 2 and N % 2 == 0:
        return np.repeat(gw_e, N // 2)
    raise ValueError("G must be 1, or 2 with N even")


def fold_gate_up_globals(scale13, gw13):
    """Load-time fold of the gate/up global ratio into the block scales (model card
    "Qwen3.8-Flash-Next-P48NVFP4-MoESQ", the note under "Compression details", and model card
    "Qwen3-30B-A3B-P48NVFP4-MoESQ", the note after the evaluation table: the two projections carry
    separate globals, and the serving loader folds their ratio into the block scales so that one
    global serves both). Reading: the gate's global is the one kept for both halves (the one a loader
    without the fold would apply to both), and each up block scale s becomes the E4M3 code nearest to
    e4m3(s) * r (ties to even, saturating at 448), r = the fp32 quotient g_up / g_gate; a zero scale
    stays zero, and a byte that is not a finite non-negative scale (0x7F and above) is left as it is.
    e4m3(s) has 4 significant bits and r 24, so the product is exact in float64.

    scale13 u8 [2I, K/32] (gate rows, then up rows), gw13 [2] -> (scale u8 [2I, K/32], gw float32 [2]).
    """
    scale13 = np.asarray(scale13, dtype=np.uint8)
    gw13 = np.asarray(gw13, dtype=np.float32).ravel()
    N = scale13.shape[0]
    if gw13.shape[0] != 2 or N % 2:
        raise ValueError("a fused gate|up linear: 2 globals and an even number of rows")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.float64(np.float32(np.float64(gw13[1]) / np.float64(gw13[0])))
    up = scale13[N // 2:]
    keep = (up == 0) | (up >= 0x7F)
    with np.errstate(invalid="ignore"):
        v = nvfp4.e4m3fn_decode(np.where(keep, 0, up)) * r
    folded = np.where(keep, up, nvfp4.e4m3_rne_sat(np.where(keep, 0.0, v)))
    out = scale13.copy()
    out[N // 2:] = folded
    return out, np.array([gw13[0], gw13[0]], dtype=np.float32)


def dequant_weight(packed, mask, scale, gw_e) -> np.ndarray:
    """One expert linear in pair-bitmask NVFP4 -> dense float64 [N, K]."""
    dense = pairbitmask.unpack(packed, mask)
    N = dense.shape[0]
    return nvfp4.dequantize(dense, scale, weight_rows_global(gw_e, N))


def grouped_gemm(a_codes, a_scales, a_global, offsets, w_packed, w_mask, w_scale, w_global):
    """out[r, n] = sum_K xhat[r, K] * what_e[n, K] for the rows r of each expert e.

    xhat = NVFP4 dequant of row r with a_global[e]; what_e = dequant of expert e's weight with its
    per-row global. ``w_*`` are indexable by expert (arrays [E, ...] or dicts of the touched experts).
    Rows outside every expert's range stay 0.
    """
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    R = a_codes.shape[0]
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.shape[0] - 1
    out = None
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 <= r0:
            continue
        W = dequant_weight(w_packed[e], w_mask[e], w_scale[e], w_global[e])
        if out is None:
            out = np.zeros((R, W.shape[0]))
        X = nvfp4.dequantize(a_codes[r0:r1], a_scales[r0:r1], np.float64(a_global[e]))
        out[r0:r1] = X @ W.T
    if out is None:
        out = np.zeros((R, np.asarray(w_packed[0]).shape[0] if R else 0))
    return out


def silu(v):
    return v / (1.0 + np.exp(-v))


def moe_ffn(x, topk_ids, topk_weights, w13, w2, g13, g2, want=False):
    """MoE FFN of tokens x [T, H] (bf16 values as floats) through paired-4:8 NVFP4 experts.

    w13 = (packed, mask, scale, global) of the fused gate|up linear, per expert [2I, H/4] ... with
    global [2]; w2 = the same for down, [H, I/4] ... with global [1]; each indexable by expert.
    g13, g2: per-expert activation globals of gate/up and of down.

    For each pair (t, j) with expert e = topk_ids[t, j]:
      a13 = quant(x[t], g13[e]);  [gate | up] = dq(a13) @ W13_e^T;  h = silu(gate) * up;
      a2 = quant(h, g2[e]);  y = dq(a2) @ W2_e^T;  out[t] += topk_weights[t, j] * y.
    Returns out float64 [T, H] and, with ``want``, a dict of the intermediates in sorted-row order.
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids)
    k = ids.shape[1]
    E = len(g13)
    counts, offsets, sorted_pairs, inv = permute(ids, E)
    P = sorted_pairs.shape[0]
    tok = sorted_pairs // k
    inter = {}
    a13c = np.zeros((P, H // 2), np.uint8)
    a13s = np.zeros((P, H // 32), np.uint8)
    I = None
    h_all = None
    a2c = a2s = None
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 <= r0:
            continue
        c, s = nvfp4.quantize(x[tok[r0:r1]], np.float64(g13[e]))
        a13c[r0:r1], a13s[r0:r1] = c, s
        W13 = dequant_weight(w13[0][e], w13[1][e], w13[2][e], w13[3][e])
        if I is None:
            I = W13.shape[0] // 2
            h_all = np.zeros((P, I))
            a2c = np.zeros((P, I // 2), np.uint8)
            a2s = np.zeros((P, I // 32), np.uint8)
        gu = nvfp4.dequantize(c, s, np.float64(g13[e])) @ W13.T
        h = silu(gu[:, :I]) * gu[:, I:]
        h_all[r0:r1] = h
        c2, s2 = nvfp4.quantize(h, np.float64(g2[e]))
        a2c[r0:r1], a2s[r0:r1] = c2, s2
    out = down_combine(a2c, a2s, g2, offsets, sorted_pairs, topk_weights, w2, T, H) if P else np.zeros((T, H))
    if want:
        inter.update(counts=counts, offsets=offsets, sorted_pairs=sorted_pairs, inv=inv,
                     a13_codes=a13c, a13_scales=a13s, h=h_all, a2_codes=a2c, a2_scales=a2s)
        return out, inter
    return out


def down_combine(a2_codes, a2_scales, g2, offsets, sorted_pairs, topk_weights, w2, T: int, H: int):
    """The down projection of each sorted row, times its router weight, summed into its token."""
    wts = np.asarray(topk_weights, dtype=np.float64).ravel()
    k = np.asarray(topk_weights).shape[1]
    out = np.zeros((T, H))
    y = grouped_gemm(a2_codes, a2_scales, g2, offsets, w2[0], w2[1], w2[2], w2[3])
    y = y * wts[sorted_pairs][:, None]
    np.add.at(out, sorted_pairs // k, y)
    return out


def h_error_bound(x, topk_ids, w13, g13, g2, gamma: float, unit: float = 2.0 ** -24):
    """Per-element bound on |h_fp32 - h| for an implementation that accumulates gate/up in fp32.

    With S = sum_K |xhat_K * what_K| (per output), an fp32 accumulation of exactly-representable
    products whose error is at most gamma * unit * S, followed by fp32 global-scale products, silu and
    the gate*up product (each a few units of rounding), deviates from the float64 value by at most
    B = 1.1 * dG * |up| + |silu(gate)| * dU + dG * dU + 16 * unit * |h|, with dG = gamma*unit*S_gate*(1+...)
    (|silu'| <= 1.1). Returned in sorted-row order, like ``moe_ffn``'s ``h``.
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids)
    k = ids.shape[1]
    E = len(g13)
    counts, offsets, sorted_pairs, inv = permute(ids, E)
    tok = sorted_pairs // k
    B = None
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 <= r0:
            continue
        W13 = dequant_weight(w13[0][e], w13[1][e], w13[2][e], w13[3][e])
        I = W13.shape[0] // 2
        if B is None:
            B = np.zeros((sorted_pairs.shape[0], I))
        c, s = nvfp4.quantize(x[tok[r0:r1]], np.float64(g13[e]))
        X = nvfp4.dequantize(c, s, np.float64(g13[e]))
        gu = X @ W13.T
        S = np.abs(X) @ np.abs(W13).T
        d = gamma * unit * S + 4 * unit * np.abs(gu)
        gate, up = gu[:, :I], gu[:, I:]
        dG, dU = d[:, :I], d[:, I:]
        h = silu(gate) * up
        B[r0:r1] = 1.1 * dG * np.abs(up) + np.abs(silu(gate)) * dU + 1.1 * dG * dU + 16 * unit * np.abs(h)
    return B
