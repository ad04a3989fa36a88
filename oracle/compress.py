"""Compression of a dense fp32 weight into paired-4:8 NVFP4 pair-bitmask storage (synthetic layers).

Source: model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ", "Compression details" (paired 4:8 along K:
in every 8 consecutive elements, i.e. 4 pairs, exactly 2 pairs are kept; NVFP4 weights with an E4M3
scale per 32 K and an FP32 per-tensor global scale) and "Sparse storage layout"; the mask choice
follows the synthetic recipe (keep the two largest-magnitude pairs, then quantize with
global = amax/(6*448)) since the trained masks of the pages are not available.

Readings where the pages are silent: a pair's magnitude is a^2 + b^2, computed in float64 as a*a + b*b
(no fused multiply-add) from the fp32 values, ties to the lower pair index; the global is the fp32
quotient fp32(amax of the pruned tensor) / 2688; pruned pairs are the byte 0x00; the kept pairs are
named by the prune, also where their NVFP4 byte is 0x00.
"""
from __future__ import annotations

import numpy as np

from . import nvfp4, pairbitmask


def prune_pairs(w) -> np.ndarray:
    """Keep flags [N, K/2] (one per pair): in every chunk of 4 pairs, the 2 with the largest a^2 + b^2."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    a = w[:, 0::2].astype(np.float64)
    b = w[:, 1::2].astype(np.float64)
    score = (a * a + b * b).reshape(N, K // 8, 4)
    order = np.argsort(-score, axis=2, kind="stable")       # stable: equal scores keep lower index first
    keep = np.zeros_like(score, dtype=bool)
    np.put_along_axis(keep, order[..., :2], True, axis=2)
    return keep.reshape(N, K // 2)


def global_scale(w_pruned) -> np.float32:
    """fp32(amax |w_pruned|) / fp32(2688), an IEEE fp32 division (2688 = 6 * 448)."""
    amax = np.float32(np.abs(np.asarray(w_pruned, dtype=np.float32)).max())
    return np.float32(amax) / np.float32(2688.0)


def compress(w):
    """Dense fp32 [N, K] -> (packed u8 [N,K/4], mask u8 [N,K/16], scale u8 [N,K/32], global fp32)."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    keep = prune_pairs(w)                                    # [N, K/2]
    keep_el = np.repeat(keep, 2, axis=1)                     # [N, K]
    wp = np.where(keep_el, w, np.float32(0.0))
    gw = global_scale(wp)
    codes, scales = nvfp4.quantize(wp.astype(np.float64), np.float64(gw))
    dense = np.where(keep, codes, 0).astype(np.uint8)        # pruned pair -> byte 0x00
    packed, mask = pairbitmask.pack(dense, keep=keep)
    return packed, mask, scales, gw


def decompress(packed, mask, scale, gw) -> np.ndarray:
    """Pair-bitmask NVFP4 -> dense float64 weight [N, K] (pruned elements 0)."""
    dense = pairbitmask.unpack(packed, mask)
    return nvfp4.dequantize(dense, scale, np.float64(gw))
