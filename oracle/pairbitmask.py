"""Pair-bitmask storage codec (``paired48_sparse``, layout "pair-bitmask", version 1), on NVFP4 bytes.

Source: model card "Qwen3.5-397B-A17B-P48NVFP4-MoESQ", section "Sparse storage layout" and its table
(the same text on the Qwen3-30B-A3B card): packed NVFP4 holds two adjacent K elements per byte, so a
pair is a byte and a paired-4:8 weight has exactly two nonzero bytes in every 4-byte chunk.

* ``weight_sparse_packed`` u8 [out, K/4]: the two kept bytes of every 4-byte chunk, in K order;
* ``weight_sparse_mask``   u8 [out, K/16]: one 4-bit mask per chunk with exactly two bits set, bit i
  meaning byte i of the chunk is kept, the lower-K chunk in the low nibble;
* the encoding is lossless: dense NVFP4 -> sparse -> dense is exact.

Reading (pages silent): byte i of a chunk is the i-th lowest-K byte; bit i is counted from the LSB.
"""
from __future__ import annotations

import numpy as np

#: quantization_config marker: "paired48_sparse": {"layout": "pair-bitmask", "version": 1}
LAYOUT = "pair-bitmask"
VERSION = 1


def nibbles(mask) -> np.ndarray:
    """u8 [N, K/16] -> chunk nibbles [N, K/8] (chunk 2j in the low nibble of byte j)."""
    mask = np.asarray(mask, dtype=np.uint8)
    N, M = mask.shape
    nib = np.empty((N, 2 * M), dtype=np.uint8)
    nib[:, 0::2] = mask & 0xF
    nib[:, 1::2] = mask >> 4
    return nib


def popcount4(n) -> np.ndarray:
    n = np.asarray(n, dtype=np.uint8)
    return ((n >> 0) & 1) + ((n >> 1) & 1) + ((n >> 2) & 1) + ((n >> 3) & 1)


def invalid_nibbles(mask) -> int:
    """Number of chunk masks that do not have exactly two bits set."""
    return int((popcount4(nibbles(mask)) != 2).sum())


def unpack(packed, mask) -> np.ndarray:
    """Sparse (packed [N, K/4], mask [N, K/16]) -> dense packed NVFP4 [N, K/2] with pruned bytes 0x00."""
    packed = np.asarray(packed, dtype=np.uint8)
    nib = nibbles(mask)
    N, C = nib.shape
    if packed.shape != (N, 2 * C):
        raise ValueError("packed/mask shapes disagree")
    if (popcount4(nib) != 2).any():
        raise ValueError("a chunk mask does not have exactly two bits set")
    bits = (nib[..., None] >> np.arange(4, dtype=np.uint8)) & 1          # [N, C, 4]
    # position of the first and second kept byte of each chunk
    first = np.argmax(bits, axis=2)
    second = 3 - np.argmax(bits[..., ::-1], axis=2)
    dense = np.zeros((N, C, 4), dtype=np.uint8)
    kept = packed.reshape(N, C, 2)
    n_idx, c_idx = np.indices((N, C))
    dense[n_idx, c_idx, first] = kept[..., 0]
    dense[n_idx, c_idx, second] = kept[..., 1]
    return dense.reshape(N, 4 * C)


def pack(dense, keep=None):
    """Dense packed NVFP4 [N, K/2] -> (packed [N, K/4], mask [N, K/16]).

    ``keep`` (bool [N, K/2], optional) names the kept bytes explicitly, exactly two per 4-byte chunk;
    the other bytes must be 0x00. Without it the kept bytes are the nonzero ones; a chunk with more than
    two is an error and a chunk with fewer is completed with its lowest-index zero bytes.
    """
    dense = np.asarray(dense, dtype=np.uint8)
    N, Kh = dense.shape
    if Kh % 8:
        raise ValueError("K must be a multiple of 16 (K/2 bytes a multiple of 8)")
    C = Kh // 4
    ch = dense.reshape(N, C, 4)
    if keep is None:
        k = ch != 0
        cnt = k.sum(axis=2)
        if (cnt > 2).any():
            raise ValueError("a 4-byte chunk has more than two nonzero bytes")
        for i in range(4):                      # complete with the lowest-index zero bytes
            need = k.sum(axis=2) < 2
            k[..., i] |= need & ~k[..., i]
    else:
        k = np.asarray(keep, dtype=bool).reshape(N, C, 4)
        if (k.sum(axis=2) != 2).any():
            raise ValueError("keep must mark exactly two bytes per chunk")
        if (ch[~k] != 0).any():
            raise ValueError("a byte outside keep is nonzero")
    order = np.argsort(~k, axis=2, kind="stable")[..., :2]              # kept byte indices, in K order
    packed = np.take_along_axis(ch, order, axis=2).reshape(N, 2 * C)
    nib = (k * (1 << np.arange(4))).sum(axis=2).astype(np.uint8)        # [N, C]
    mask = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed.astype(np.uint8), mask


def stored_bytes(out: int, K: int) -> int:
    """Bytes of one linear in sparse storage: packed K/4 + mask K/16 + scales K/32 per output row."""
    return out * (K // 4 + K // 16 + K // 32)


def dense_nvfp4_bytes(out: int, K: int) -> int:
    """Bytes of the same linear as dense packed NVFP4 with per-32 E4M3 scales: K/2 + K/32 per row."""
    return out * (K // 2 + K // 32)
