"""Pins of the pair-bitmask codec and the synthetic weight compression (no GPU)."""
import json
import os
from itertools import combinations

import numpy as np
import pytest

from oracle import compress, nvfp4, pairbitmask
import synth


def test_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "pair_bitmask_example.json")))
    dense = np.array([ex["dense_bytes"]], dtype=np.uint8)
    packed, mask = pairbitmask.pack(dense)
    assert packed[0].tolist() == ex["packed"]
    assert mask[0].tolist() == ex["mask"]
    assert pairbitmask.nibbles(mask)[0].tolist() == ex["chunk_nibbles"]
    assert pairbitmask.unpack(packed, mask)[0].tolist() == ex["dense_bytes"]
    vals = nvfp4.dequantize(pairbitmask.unpack(packed, mask), np.array([[ex["scale_byte"]]]), ex["global"])
    assert vals[0].tolist() == ex["values"]


def _random_dense(rng, N, K, zero_kept=False):
    nib = synth.VALID_NIBBLES[rng.integers(0, 6, size=(N, K // 8))]
    keep = ((nib[..., None] >> np.arange(4)) & 1).astype(bool).reshape(N, K // 2)
    vals = rng.integers(1 if not zero_kept else 0, 256, size=(N, K // 2), dtype=np.uint8)
    dense = np.where(keep, vals, 0).astype(np.uint8)
    return dense, keep


def test_round_trips_and_invariants():
    rng = np.random.default_rng(0)
    for N, K in [(1, 32), (7, 64), (33, 512)]:
        dense, keep = _random_dense(rng, N, K)
        packed, mask = pairbitmask.pack(dense)
        assert packed.shape == (N, K // 4) and mask.shape == (N, K // 16)
        assert pairbitmask.invalid_nibbles(mask) == 0
        assert np.array_equal(pairbitmask.unpack(packed, mask), dense)           # dense -> sparse -> dense
        p2, m2 = pairbitmask.pack(pairbitmask.unpack(packed, mask))
        assert np.array_equal(p2, packed) and np.array_equal(m2, mask)           # sparse -> dense -> sparse
        # exactly two nonzero bytes per chunk -> 8 kept bytes (16 survivors) per 32-K scale group
        nz = (pairbitmask.unpack(packed, mask).reshape(N, K // 32, 16) != 0).sum(axis=2)
        assert (nz == 8).all()


def test_explicit_keep_preserves_zero_kept_bytes():
    rng = np.random.default_rng(1)
    dense, keep = _random_dense(rng, 16, 128, zero_kept=True)
    dense[0, :4] = 0                         # a whole chunk of zero bytes, 2 of them kept
    packed, mask = pairbitmask.pack(dense, keep=keep)
    assert np.array_equal(pairbitmask.unpack(packed, mask), dense)
    kept_from_mask = ((pairbitmask.nibbles(mask)[..., None] >> np.arange(4)) & 1).astype(bool)
    assert np.array_equal(kept_from_mask.reshape(16, 64), keep)


def test_pack_rejects_three_nonzero_and_unpack_rejects_bad_mask():
    d = np.zeros((1, 16), np.uint8)
    d[0, :3] = 1
    with pytest.raises(ValueError):
        pairbitmask.pack(d)
    with pytest.raises(ValueError):
        pairbitmask.unpack(np.zeros((1, 8), np.uint8), np.array([[0x37, 0x33]], np.uint8))
    assert pairbitmask.invalid_nibbles(np.array([[0x37, 0x33]], np.uint8)) == 1


def test_storage_byte_accounting_reproduces_page_figures(golden_dir):
    fig = json.load(open(os.path.join(golden_dir, "storage_figures.json")))
    GiB = 2.0 ** 30
    f = fig["flash_next_routed_experts"]
    n = f["params"]
    # per dense weight: sparse = 1/4 + 1/16 + 1/32 = 11/32 byte, dense NVFP4 = 1/2 + 1/32 = 17/32, BF16 = 2
    assert pairbitmask.stored_bytes(1, 32) == 11 and pairbitmask.dense_nvfp4_bytes(1, 32) == 17
    assert abs(n * 2 / GiB - f["bf16_gib"]) <= f["printed_precision_gib"]
    assert abs(n * 11 / 32 / GiB - f["sparse_gib"]) <= f["printed_precision_gib"]
    assert abs(n * 17 / 32 / GiB - f["dense_nvfp4_gib"]) <= f["printed_precision_gib"]
    r = fig["sparse_vs_dense_ratio"]
    assert abs(11 / 17 - r["ratio"]) <= r["printed_precision"]
    q = fig["qwen35_397b_checkpoint"]
    per_expert_dense = 3 * pairbitmask.dense_nvfp4_bytes(q["moe_intermediate"], q["hidden"])
    per_expert_sparse = 3 * pairbitmask.stored_bytes(q["moe_intermediate"], q["hidden"])
    diff = q["layers"] * q["experts"] * (per_expert_dense - per_expert_sparse) / GiB
    assert abs(diff - (q["dense_ckpt_gib"] - q["sparse_ckpt_gib"])) <= 2 * q["printed_precision_gib"]
    # kept values: 4 bits for half the elements = 2 bits per dense weight
    assert 4 * 0.5 == fig["effective_bits"]["bits_per_weight"]


def _prune_brute(w):
    N, K = w.shape
    keep = np.zeros((N, K // 2), bool)
    for n in range(N):
        for c in range(K // 8):
            sc = [float(w[n, 8 * c + 2 * i]) ** 2 + float(w[n, 8 * c + 2 * i + 1]) ** 2 for i in range(4)]
            best = max(combinations(range(4), 2), key=lambda p: (sc[p[0]] + sc[p[1]], -p[0], -p[1]))
            for i in best:
                keep[n, 4 * c + i] = True
    return keep


def test_prune_vs_brute_force_and_ties():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((6, 64)) * 0.02).astype(np.float32)
    assert np.array_equal(compress.prune_pairs(w), _prune_brute(w))
    t = np.array([[1, 0, 0, 1, -1, 0, 0.5, 0.5] * 4], np.float32)   # pair scores 1, 1, 1, 0.5
    assert compress.prune_pairs(t)[0, :4].tolist() == [True, True, False, False]


def test_compress_invariants_and_decode():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((48, 256)) * 0.02).astype(np.float32)
    packed, mask, scale, gw = compress.compress(w)
    assert pairbitmask.invalid_nibbles(mask) == 0
    assert scale.max() <= 0x7E
    keep = compress.prune_pairs(w)
    kept_from_mask = ((pairbitmask.nibbles(mask)[..., None] >> np.arange(4)) & 1).astype(bool)
    assert np.array_equal(kept_from_mask.reshape(keep.shape), keep)
    wp = np.where(np.repeat(keep, 2, axis=1), w, 0).astype(np.float64)
    assert gw == np.float32(np.float32(np.abs(wp).max()) / np.float32(2688))
    deq = compress.decompress(packed, mask, scale, gw)
    assert (deq[~np.repeat(keep, 2, axis=1)] == 0).all()
    # NVFP4 error: within one E2M1 step at the group's scale plus the saturation gap of the scale
    amax_g = np.abs(wp).reshape(48, 8, 32).max(axis=2)
    bound = np.repeat(0.2 * amax_g, 32, axis=1)
    assert (np.abs(deq - wp) <= bound + 1e-12).all()
    # the tensor's largest block takes (close to) the largest scale
    assert scale.max() >= 0x7D
