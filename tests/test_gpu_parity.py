"""Parity of the HIP library (through its C ABI) with the CPU oracle on MI355X.

Integer work is compared bit-exactly (permutation, quantized codes and scales, compressed weights,
storage codec); fp32 outputs row by row within 1e-3 (max |y - yref| / max |yref| per row).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import compress, moe, nvfp4, pairbitmask

pytestmark = pytest.mark.gpu

moesq = pytest.importorskip("sparse_quantized_moe_amd")
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(autouse=True)
def _gpu():
    _need_gpu()
    yield
    torch.cuda.synchronize()


def rowwise(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    return float((np.abs(y - ref).max(axis=1) / den).max())


# ------------------------------------------------------------------------------------------------
# activation quantizer
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,outliers,gmode", [
    (16, 512, 0.0, "amax"), (256, 2048, 0.0, "amax"), (64, 4096, 0.0, "fixed"),
    (333, 7168, 0.001, "amax"), (5, 96, 0.0, "tiny"), (7, 64, 0.0, "huge")])
def test_quantize_bf16_bit_exact(T, H, outliers, gmode):
    x = synth.activations(3, T, H, device=DEV, outlier_frac=outliers, outlier_scale=50.0)
    amax = np.float32(x.float().abs().max().item())
    g = {"amax": amax / np.float32(2688), "fixed": synth.ACT_GLOBAL_FIXED,
         "tiny": np.float32(2.0 ** -40), "huge": np.float32(100.0)}[gmode]
    gt = torch.tensor([g], dtype=torch.float32, device=DEV)
    codes, scales = moesq.quantize_act(x, gt)
    rc, rs = nvfp4.quantize(x.float().cpu().numpy(), np.float64(g))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("spread", [1, 48])
def test_quantize_f32_boundaries_bit_exact(spread):
    """fp32 inputs placed on and next to every E2M1 and E4M3 rounding boundary: one ulp either side,
    or up to `spread` ulps either side (across the window where the kernel switches from the hardware
    conversion to the exact comparisons)."""
    rng = np.random.default_rng(11 + spread)
    R = 512
    g = np.float32(0.0371)
    x = np.zeros((R, 64), np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for r in range(R):
        s = float(nvfp4.E4M3_MAGNITUDES[rng.integers(8, 0x7E)])
        for gi in range(2):
            # make the group amax give exactly scale s (amax = 6 s g, a +-6 code)
            v = (rng.choice(mids, 32) * s * float(g)).astype(np.float32)
            if spread == 1:
                v = np.where(rng.random(32) < 0.3, np.nextafter(v, np.float32(np.inf)), v)
                v = np.where(rng.random(32) < 0.3, np.nextafter(v, np.float32(0)), v)
            else:   # shift the bit pattern by a whole number of ulps (all values are positive here)
                v = (v.view(np.int32) + rng.integers(-spread, spread + 1, 32).astype(np.int32)).view(np.float32)
            v[0] = np.float32(6 * s * float(g))
            if rng.random() < 0.3:   # amax on an E4M3 midpoint instead
                i = rng.integers(8, 0x7D)
                m = (nvfp4.E4M3_MAGNITUDES[i] + nvfp4.E4M3_MAGNITUDES[i + 1]) / 2
                v[0] = np.float32(6 * m * float(g))
            v *= np.where(rng.random(32) < 0.5, -1, 1).astype(np.float32)
            x[r, 32 * gi:32 * gi + 32] = v
    xt = torch.from_numpy(x).to(DEV)
    codes, scales = moesq.quantize_act(xt, torch.tensor([g], device=DEV))
    rc, rs = nvfp4.quantize(x.astype(np.float64), np.float64(g))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_bf16_boundaries_bit_exact():
    """bf16 inputs on every E2M1 rounding boundary and one bf16 ulp either side. With a power-of-two
    global, B·s·g has at most 7 significant bits and is itself a bf16 value, so exact ties occur (the
    case where the bf16 encoder relies on the conversion's nearest-even)."""
    rng = np.random.default_rng(29)
    R = 512
    g = np.float32(2.0 ** -5)
    x = np.zeros((R, 64), np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for r in range(R):
        s = float(nvfp4.E4M3_MAGNITUDES[rng.integers(8, 0x7E)])
        for gi in range(2):
            v = (rng.choice(mids, 32) * s * float(g)).astype(np.float32)
            b = (v.view(np.uint32) >> 16).astype(np.int64) + rng.integers(-1, 2, 32)
            v = (b.astype(np.uint32) << 16).view(np.float32)
            v[0] = np.float32(6 * s * float(g))   # amax = 6 s g: the group's scale is s
            v *= np.where(rng.random(32) < 0.5, -1, 1).astype(np.float32)
            x[r, 32 * gi:32 * gi + 32] = v
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xt.float().numpy(), x)   # every input is a bf16 value
    codes, scales = moesq.quantize_act(xt.to(DEV), torch.tensor([g], device=DEV))
    rc, rs = nvfp4.quantize(x.astype(np.float64), np.float64(g))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_gather_with_expert_globals():
    T, H, E = 40, 256, 5
    x = synth.activations(4, T, H, device=DEV)
    src = torch.tensor(np.random.default_rng(0).integers(0, T, 70), dtype=torch.int32, device=DEV)
    offs = torch.tensor([0, 10, 10, 33, 50, 66], dtype=torch.int32, device=DEV)
    g = torch.tensor([0.001, 0.002, 0.0005, 0.004, 0.0011], dtype=torch.float32, device=DEV)
    codes = torch.zeros((70, H // 2), dtype=torch.uint8, device=DEV)
    codes, scales = moesq.quantize_act(x, g, src_row=src, expert_offsets=offs)
    xs = x.float().cpu().numpy()[src.cpu().numpy()]
    o = offs.cpu().numpy()
    for e in range(E):
        if o[e + 1] > o[e]:
            rc, rs = nvfp4.quantize(xs[o[e]:o[e + 1]], np.float64(g[e].item()))
            assert np.array_equal(codes[o[e]:o[e + 1]].cpu().numpy(), rc)
            assert np.array_equal(scales[o[e]:o[e + 1]].cpu().numpy(), rs)


# ------------------------------------------------------------------------------------------------
# permutation
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,k,E,kind", [(256, 8, 128, "softmax"), (8192, 8, 128, "zipf"), (1, 1, 1, "softmax"),
                                        (1000, 10, 512, "softmax"), (16384, 8, 384, "zipf"), (3, 2, 1024, "softmax")])
def test_permute_bit_exact(T, k, E, kind):
    ids, _ = synth.routing(5, T, E, k, kind, 1.0, 1.0)
    ids = ids.copy()
    if T > 4:
        ids[1, 0] = -1
        ids[2, :] = -1
    counts, offsets, sorted_, inv, status = moesq.permute(torch.from_numpy(ids).to(DEV), E)
    rc, ro, rs, ri = moe.permute(ids, E)
    n = int(ro[-1])
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(sorted_.cpu().numpy()[:n], rs)
    assert np.array_equal(inv.cpu().numpy(), ri)
    assert status.item() == 0


def test_permute_duplicates_and_invalid_ids():
    rng = np.random.default_rng(8)
    T, k, E = 700, 4, 16
    ids = rng.integers(-1, E, size=(T, k)).astype(np.int32)     # many duplicate ids inside rows
    bad = ids.copy()
    bad[5, 1] = E + 3
    bad[600, 0] = -7
    counts, offsets, sorted_, inv, status = moesq.permute(torch.from_numpy(bad).to(DEV), E)
    ref_ids = bad.copy()
    ref_ids[(ref_ids >= E) | (ref_ids < -1)] = -1
    rc, ro, rs, ri = moe.permute(ref_ids, E)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(sorted_.cpu().numpy()[:int(ro[-1])], rs)
    assert np.array_equal(inv.cpu().numpy(), ri)
    assert status.item() == 2


def test_permute_one_tile_with_duplicates_among_clean_tiles():
    # tiles of 512 tokens: only the second holds a token naming an expert twice
    ids, _ = synth.routing(9, 1500, 64, 6)
    ids = ids.copy()
    ids[900, 3] = ids[900, 1]
    counts, offsets, sorted_, inv, status = moesq.permute(torch.from_numpy(ids).to(DEV), 64)
    rc, ro, rs, ri = moe.permute(ids, 64)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(sorted_.cpu().numpy()[:int(ro[-1])], rs)
    assert np.array_equal(inv.cpu().numpy(), ri)
    assert status.item() == 0


def test_permute_no_tokens():
    counts, offsets, sorted_, inv, status = moesq.permute(torch.zeros((0, 4), dtype=torch.int32, device=DEV), 8)
    assert counts.cpu().numpy().tolist() == [0] * 8
    assert offsets.cpu().numpy().tolist() == [0] * 9
    assert status.item() == 0


# ------------------------------------------------------------------------------------------------
# weight compression and storage codec
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("N,K", [(256, 512), (768, 2048), (64, 7168), (3, 32)])
def test_compress_bit_exact(N, K):
    w = synth.dense_weight(6, 0, 0, N, K, device=DEV)
    if N == 3:                                   # ties between pair magnitudes and an all-zero chunk
        w[0, :8] = torch.tensor([0.5, 0, 0, 0.5, -0.5, 0, 0.3, 0.4], device=DEV)
        w[1, 8:16] = 0
    packed, mask, scale, gw = moesq.compress_weights(w)
    rp, rm, rs, rg = compress.compress(w.cpu().numpy())
    assert gw.item() == rg
    assert np.array_equal(scale.cpu().numpy(), rs)
    assert np.array_equal(mask.cpu().numpy(), rm)
    assert np.array_equal(packed.cpu().numpy(), rp)


def test_storage_codec_bit_exact():
    rng = np.random.default_rng(9)
    N, K = 200, 1024
    packed, mask, _, _ = synth.random_sparse_weights(10, 1, N, K)
    p, m = torch.from_numpy(packed[0]).to(DEV), torch.from_numpy(mask[0]).to(DEV)
    dense, bad = moesq.unpack_pair_bitmask(p, m, K)
    assert bad.item() == 0
    assert np.array_equal(dense.cpu().numpy(), pairbitmask.unpack(packed[0], mask[0]))
    # pack of a dense tensor whose kept bytes are nonzero: round trip
    d2 = pairbitmask.unpack(packed[0] | 1, mask[0])
    p2, m2, bad2 = moesq.pack_pair_bitmask(torch.from_numpy(d2).to(DEV), K)
    rp, rm = pairbitmask.pack(d2)
    assert bad2.item() == 0 and np.array_equal(p2.cpu().numpy(), rp) and np.array_equal(m2.cpu().numpy(), rm)
    # canonical completion of chunks with fewer than two nonzero bytes, and validation
    d3 = d2.copy()
    d3[0, :4] = 0
    d3[1, 4:8] = [0, 0, 9, 0]
    p3, m3, _ = moesq.pack_pair_bitmask(torch.from_numpy(d3).to(DEV), K)
    rp3, rm3 = pairbitmask.pack(d3)
    assert np.array_equal(p3.cpu().numpy(), rp3) and np.array_equal(m3.cpu().numpy(), rm3)
    mbad = mask[0].copy()
    mbad[3, 2] = 0x37
    mbad[9, 0] = 0xFF
    assert moesq.validate_weights(torch.from_numpy(mbad).to(DEV), K) == pairbitmask.invalid_nibbles(mbad) == 3


def _tiled_reference(packed, mask, scale):
    """The tiled record bytes, written out from the layout's definition in include/moesq.h."""
    E, N, Kq = packed.shape
    K = Kq * 4
    steps = K // 256
    out = np.zeros((E, N // 16, steps, 1408), np.uint8)
    lo, hi = packed & 0x0F, packed >> 4
    for e in range(E):
        for tile in range(N // 16):
            for ss in range(steps):
                for lane in range(64):
                    row, q = tile * 16 + lane % 16, lane // 16
                    kb = (ss * 256 + 64 * q) // 4                    # packed byte offset of the lane's 64 K
                    for t in range(4):                               # smfmac t: bytes (b0 b1)(b0' b1')
                        b = kb + 4 * t
                        rec = out[e, tile, ss]
                        rec[16 * lane + 4 * t + 0] = lo[e, row, b] | (lo[e, row, b + 1] << 4)
                        rec[16 * lane + 4 * t + 1] = lo[e, row, b + 2] | (lo[e, row, b + 3] << 4)
                        rec[16 * lane + 4 * t + 2] = hi[e, row, b] | (hi[e, row, b + 1] << 4)
                        rec[16 * lane + 4 * t + 3] = hi[e, row, b + 2] | (hi[e, row, b + 3] << 4)
                    m0 = (ss * 256 + 64 * q) // 16
                    for j in range(4):                               # mask byte -> two position codes
                        mb = int(mask[e, row, m0 + j])
                        codes = []
                        for nib in (mb & 15, mb >> 4):
                            bits = [i for i in range(4) if nib >> i & 1]
                            codes.append(bits[0] | (bits[-1] << 2))
                        out[e, tile, ss, 1024 + 4 * lane + j] = codes[0] | (codes[1] << 4)
                    s0 = (ss * 256 + 64 * q) // 32
                    out[e, tile, ss, 1280 + 2 * lane: 1282 + 2 * lane] = scale[e, row, s0:s0 + 2]
    return out.reshape(-1)


def test_prepare_layout_and_round_trip():
    E, N, K = 2, 32, 512
    packed, mask, scale, gw = synth.random_sparse_weights(30, E, N, K, 1)
    w = moesq.SparseWeights(*(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in (packed, mask, scale, gw)))
    wt = moesq.prepare_weights(w)
    assert np.array_equal(wt.packed.cpu().numpy(), _tiled_reference(packed, mask, scale))
    back = moesq.unprepare_weights(wt)
    for a, b in ((back.packed, packed), (back.mask, mask), (back.scale, scale)):
        assert np.array_equal(a.cpu().numpy(), b)


# ------------------------------------------------------------------------------------------------
# grouped GEMM
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("E,N,K,G,counts", [
    (1, 256, 512, 1, [16]),                                       # one expert linear
    (4, 256, 512, 2, [0, 5, 33, 17]),                             # ragged, an empty expert, decode tactic
    (3, 320, 768, 1, [200, 0, 130]),                              # prefill tactic, N not a multiple of 256
    (2, 64, 2048, 2, [1, 129]),
    (9, 256, 512, 1, [13, 29, 45, 61, 77, 93, 109, 125, 135]),    # prefill, last m-blocks of 1 .. 8 token tiles
    (5, 128, 1280, 1, [40, 3, 0, 31, 64]),                        # decode, K-chunks of 512 with a short last one
    (6, 576, 768, 1, [7, 0, 40, 16, 1, 33]),                      # decode, K in one chunk: n-block loop, ragged
                                                                  # last n-block, several m-blocks
    (3, 1024, 768, 2, [20, 5, 64]),                               # the same with two global scales
])
def test_grouped_gemm_random_bytes(E, N, K, G, counts, layout):
    packed, mask, scale, gw = synth.random_sparse_weights(12, E, N, K, G)
    scale = np.clip(scale, 0x18, 0x60).astype(np.uint8)            # keep products in a sane exponent range
    rows = sum(counts)
    a_codes, a_scales = synth.random_act_codes(13, rows, K)
    a_scales = np.clip(a_scales, 0x18, 0x60).astype(np.uint8)
    a_global = (2.0 ** np.random.default_rng(1).uniform(-6, -2, E)).astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    w = moesq.SparseWeights(*(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in (packed, mask, scale, gw)))
    if layout == 1:
        w = moesq.prepare_weights(w)
    out = moesq.grouped_gemm(torch.from_numpy(a_codes).to(DEV), torch.from_numpy(a_scales).to(DEV),
                             torch.from_numpy(a_global).to(DEV), torch.from_numpy(offsets).to(DEV), w)
    ref = moe.grouped_gemm(a_codes, a_scales, a_global, offsets, packed, mask, scale, gw)
    err = rowwise(out.cpu().numpy(), ref)
    assert err <= 1e-3, err


def test_linear_workload():
    """One expert linear, M=16, N=256, K=512, compressed from N(0, 0.02) and quantized from N(0, 1)."""
    wl = synth.WORKLOADS["linear"]
    w = synth.dense_weight(0, 0, 0, wl.I, wl.H, device=DEV)
    packed, mask, scale, gw = moesq.compress_weights(w)
    rp, rm, rs, rg = compress.compress(w.cpu().numpy())
    assert np.array_equal(packed.cpu().numpy(), rp) and np.array_equal(mask.cpu().numpy(), rm)
    assert np.array_equal(scale.cpu().numpy(), rs) and gw.item() == rg
    x = synth.activations(0, wl.T, wl.H, device=DEV)
    g = np.float32(x.float().abs().max().item()) / np.float32(2688)
    codes, scales = moesq.quantize_act(x, torch.tensor([g], device=DEV))
    rc, rsc = nvfp4.quantize(x.float().cpu().numpy(), np.float64(g))
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rsc)
    sw = moesq.SparseWeights(packed[None], mask[None], scale[None], gw.view(1, 1))
    offs = torch.tensor([0, wl.T], dtype=torch.int32, device=DEV)
    out = moesq.grouped_gemm(codes, scales, torch.tensor([g], device=DEV), offs, sw)
    ref = moe.grouped_gemm(rc, rsc, [g], [0, wl.T], rp[None], rm[None], rs[None], np.array([[rg]]))
    assert rowwise(out.cpu().numpy(), ref) <= 1e-3


# ------------------------------------------------------------------------------------------------
# MoE FFN
# ------------------------------------------------------------------------------------------------
def _layer(seed, E, H, I, tiled=True):
    def dense_expert(e):       # regenerated on demand (deterministic), not cached
        return synth.expert_dense_weights(seed, e, H, I, device=DEV)
    w13, w2 = moesq.compress_moe_layer(E, H, I, dense_expert, device=DEV)
    if tiled:
        w13, w2 = moesq.prepare_weights(w13), moesq.prepare_weights(w2)
    return w13, w2, dense_expert


def _globals(x, ids, E, dense_expert, fixed=False):
    if fixed:
        return (np.full(E, synth.ACT_GLOBAL_FIXED, np.float32),) * 2
    g13 = synth.act_globals_from_x(x, ids, E)
    g2 = np.full(E, synth.ACT_GLOBAL_FIXED, np.float32)
    T = x.shape[0]
    for e in range(E):
        rows = np.nonzero((ids == e).any(axis=1))[0]
        if len(rows):
            g, u, _ = dense_expert(e)
            g2[e] = synth.down_global_from_dense(x[torch.from_numpy(rows).to(x.device)], g, u)
    return g13, g2


def _run_ffn(x, ids, wts, w13, w2, g13, g2):
    T, H = x.shape
    k = ids.shape[1]
    E, I = w13.E, w2.K
    ws = torch.empty(moesq.lib().moesq_moe_ffn_workspace_size(T, H, I, k, E, 0), dtype=torch.uint8, device=DEV)
    out = moesq.moe_ffn(x, torch.from_numpy(ids).to(DEV), torch.from_numpy(wts).to(DEV), w13, w2,
                        torch.from_numpy(g13).to(DEV), torch.from_numpy(g2).to(DEV), workspace=ws)
    inter = {kk: v.cpu().numpy() for kk, v in moesq.ffn_intermediates(ws, T, H, I, k, E).items()}
    return out.cpu().numpy(), inter


@pytest.mark.parametrize("E,H,I,T,k,fixed,tiled", [(8, 512, 256, 64, 4, False, True),     # decode tactic
                                                    (8, 512, 256, 64, 4, False, False),    # stored layout
                                                    (8, 512, 256, 512, 4, False, True),    # prefill tactic
                                                    (8, 512, 256, 512, 4, False, False),
                                                    (6, 256, 512, 40, 3, True, True),      # 1/2688 globals
                                                    (6, 768, 256, 384, 4, False, True),    # prefill, 3 gate/up steps
                                                    (4, 1280, 512, 256, 2, False, True)])  # prefill, 5 gate/up steps
def test_moe_ffn_small(E, H, I, T, k, fixed, tiled):
    from ffn_check import compare_ffn, oracle_layer
    w13, w2, dense_expert = _layer(21, E, H, I, tiled)
    x = synth.activations(22, T, H, device=DEV)
    ids, wts = synth.routing(23, T, E, k)
    g13, g2 = _globals(x, ids, E, dense_expert, fixed)
    out, inter = _run_ffn(x, ids, wts, w13, w2, g13, g2)
    rc, ro, rs, ri = moe.permute(ids, E)
    assert np.array_equal(inter["offsets"], ro) and np.array_equal(inter["inv"], ri)
    assert np.array_equal(inter["sorted"][:int(ro[-1])], rs)
    ow13, ow2 = oracle_layer(dense_expert, range(E))
    st = compare_ffn(x.float().cpu().numpy(), ids, wts, ow13, ow2, g13, g2, out, inter)
    print("ffn small", E, H, I, T, k, st)


@pytest.mark.parametrize("E,H,I,T,k,zipf_beta", [
    (1, 256, 256, 300, 1, 0.0),             # one expert, top-1: m-blocks of 8, 8 and 3 token tiles
    (3, 768, 512, 700, 2, 1.0),             # skewed, I < H, three gate/up steps
    (17, 1280, 768, 1000, 5, 0.0),          # odd expert count, k = 5, a partial 512-row n-block
    (5, 256, 1024, 400, 3, 1.0),            # I > H: the down GEMM's K is four times the gate/up one's
    (40, 512, 256, 600, 10, 0.0),           # top-10 (the 16-wide routing variant) at the prefill tactic
    (64, 512, 256, 3000, 8, 2.0),           # 15 empty experts, every tile count, a claimed item tail
])
def test_moe_ffn_odd_shapes(E, H, I, T, k, zipf_beta):
    """Shapes off the beaten track through the large-batch path: every m-block tile count, a claimed
    tail of the item list, experts with no rows, k not a power of two, I above H."""
    from ffn_check import compare_ffn, oracle_layer
    w13, w2, dense_expert = _layer(31, E, H, I, True)
    x = synth.activations(32, T, H, device=DEV)
    ids, wts = synth.routing(33, T, E, k, "zipf" if zipf_beta else "softmax", 1.0, zipf_beta)
    g13, g2 = _globals(x, ids, E, dense_expert)
    out, inter = _run_ffn(x, ids, wts, w13, w2, g13, g2)
    rc, ro, rs, ri = moe.permute(ids, E)
    assert np.array_equal(inter["offsets"], ro) and np.array_equal(inter["inv"], ri)
    assert np.array_equal(inter["sorted"][:int(ro[-1])], rs)
    ow13, ow2 = oracle_layer(dense_expert, range(E))
    st = compare_ffn(x.float().cpu().numpy(), ids, wts, ow13, ow2, g13, g2, out, inter)
    print("ffn odd shape", E, H, I, T, k, zipf_beta, st)


_RUNS = {}


def _full_run(name):
    """The full-size layer ``name`` through moesq_moe_ffn in the bench's launch configuration (tiled
    weights, default flags), kept on the host for the tests of this workload (one workload at a time)."""
    if name in _RUNS:
        return _RUNS[name]
    _RUNS.clear()
    wl = synth.WORKLOADS[name]
    w13, w2, dense_expert = _layer(0, wl.E, wl.H, wl.I)
    x = synth.activations(0, wl.T, wl.H, device=DEV, outlier_frac=wl.outlier_frac, outlier_scale=wl.outlier_scale)
    ids, wts = synth.routing(0, wl.T, wl.E, wl.k, wl.routing, wl.zipf_s, wl.zipf_beta)
    g13, g2 = _globals(x, ids, wl.E, dense_expert, wl.fixed_act_global)
    out, inter = _run_ffn(x, ids, wts, w13, w2, g13, g2)
    del w13, w2
    torch.cuda.empty_cache()
    run = {"wl": wl, "x": x.float().cpu().numpy(), "ids": ids, "wts": wts, "g13": g13, "g2": g2, "out": out,
           "inter": inter, "dense_expert": dense_expert}
    _RUNS[name] = run
    return run


# tokens checked per layer; at 384 experts only tokens whose 8 experts all lie among the 48 busiest
# (the oracle compresses and dequantizes every expert a checked token names)
_SAMPLED = {"qwen3_30b_decode": (32, None), "e512_decode": (32, None), "qwen3_30b_prefill": (32, None),
            "e512_prefill": (32, None), "kimi_k2_prefill": (32, 48)}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", list(_SAMPLED))
def test_moe_ffn_full_size_sampled(name):
    """Full-size layers in the bench's launch configuration. The permutation is checked on every pair;
    at decode sizes every live gate/up input row is checked bit-exact; 32 sampled tokens go through
    the oracle (their gate/up input rows bit-exact, down input admissible, outputs teacher-forced row
    by row and non-forced tensor-wide)."""
    from ffn_check import compare_ffn_parallel
    r = _full_run(name)
    wl, ids, inter = r["wl"], r["ids"], r["inter"]
    rc, ro, rs, ri = moe.permute(ids, wl.E)
    assert np.array_equal(inter["offsets"], ro) and np.array_equal(inter["inv"], ri)
    assert np.array_equal(inter["sorted"][:int(ro[-1])], rs)
    assert int(inter["status"][0]) == 0
    if wl.P <= 4096:
        # every live gate/up input row (pair order: row p = t*k + j), bit-exact
        e_row = ids.ravel()[rs]
        rc13, rs13 = nvfp4.quantize(r["x"][rs // wl.k], r["g13"][e_row].astype(np.float64))
        assert np.array_equal(inter["a13_codes"][rs], rc13) and np.array_equal(inter["a13_scales"][rs], rs13)
    ntok, busiest = _SAMPLED[name]
    rng = np.random.default_rng(1)
    cand = np.arange(wl.T)
    if busiest:
        top = np.argsort(-np.bincount(ids.ravel(), minlength=wl.E), kind="stable")[:busiest]
        cand = np.nonzero(np.isin(ids, top).all(axis=1))[0]
        assert len(cand) >= ntok
    toks = np.sort(rng.choice(cand, ntok, replace=False))
    st = compare_ffn_parallel(r["x"], ids, r["wts"], r["dense_expert"], r["g13"], r["g2"], r["out"], inter, toks)
    print(name, st)


def _three_experts(counts, bm=128):
    """The busiest expert, the busiest other one whose last m-block is partial (more than one m-block),
    and one with a single row (else the least busy live one)."""
    order = np.argsort(-counts, kind="stable")
    heavy = int(order[0])
    ragged = [int(e) for e in order[1:] if counts[e] > bm and counts[e] % bm]
    live = [int(e) for e in np.nonzero(counts > 0)[0] if e != heavy]
    single = [e for e in live if counts[e] == 1] or sorted(live, key=lambda e: counts[e])
    return [heavy] + ragged[:1] + [single[0]]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["qwen3_30b_prefill", "e512_prefill", "kimi_k2_prefill"])
def test_moe_ffn_every_row_of_three_experts(name):
    """Every row of the busiest expert, of one with a ragged last m-block and of a single-row expert
    (late-scheduled work items, partial m-blocks, the XCD item order): gate/up input rows bit-exact,
    down input rows equal or admissible under the fp32 error bound, and the down rows (times the
    router weight) within 1e-3 row by row of the oracle's grouped GEMM on the GPU's down input."""
    from ffn_check import gamma_for, oracle_layer
    r = _full_run(name)
    wl, ids, inter = r["wl"], r["ids"], r["inter"]
    counts = np.bincount(ids.ravel(), minlength=wl.E)
    chosen = _three_experts(counts)
    ow13, ow2 = oracle_layer(r["dense_expert"], chosen)
    for e in chosen:
        r0, r1 = int(inter["offsets"][e]), int(inter["offsets"][e + 1])
        n = r1 - r0
        assert n == counts[e]
        sp = inter["sorted"][r0:r1]
        xs = r["x"][sp // wl.k]
        c13, s13 = nvfp4.quantize(xs, np.float64(r["g13"][e]))
        assert np.array_equal(inter["a13_codes"][sp], c13) and np.array_equal(inter["a13_scales"][sp], s13), e
        W13 = moe.dequant_weight(ow13[0][e], ow13[1][e], ow13[2][e], ow13[3][e])
        gu = nvfp4.dequantize(c13, s13, np.float64(r["g13"][e])) @ W13.T
        h = moe.silu(gu[:, :wl.I]) * gu[:, wl.I:]
        c2, s2 = nvfp4.quantize(h, np.float64(r["g2"][e]))
        gc, gsc = inter["a2_codes"][r0:r1], inter["a2_scales"][r0:r1]
        same = (gsc == s2) & (nvfp4.unpack_codes(gc).reshape(n, -1, 32) ==
                              nvfp4.unpack_codes(c2).reshape(n, -1, 32)).all(axis=2)
        flips = int((~same).sum())
        if flips:
            one = np.full((n, 1), e)
            B = moe.h_error_bound(xs, one, ow13, r["g13"], r["g2"], gamma_for(wl.H))
            ok = nvfp4.check_admissible(h, B, np.float64(r["g2"][e]), gc, gsc)
            assert ok[~same].all(), (e, int((~same & ~ok).sum()))
            amb = int(nvfp4.ambiguous_groups(h, B, np.float64(r["g2"][e])).sum())
            assert flips <= max(3, amb // 2), (e, flips, amb)
        y = moe.grouped_gemm(gc, gsc, [r["g2"][e]], [0, n], [ow2[0][e]], [ow2[1][e]], [ow2[2][e]], [ow2[3][e]])
        y = y * r["wts"].ravel()[sp].astype(np.float64)[:, None]
        err = rowwise(inter["down_rows"][r0:r1], y)
        assert err <= 1e-3, (e, err)
        print(name, "expert", e, "rows", n, "h flips", flips, "down rows max row-normwise err", err)


@pytest.mark.parametrize("layout", [0, 1])
def test_grouped_gemm_every_scale_byte(layout):
    """Every finite E4M3 byte 0x00..0x7E on both operands through the GEMM (the hardware FP8 to f16
    conversion of the scales), element by element against the oracle. Activation row r holds codes in
    one 32-K block only, with scale byte r there; weight row n has scale byte (n + 17 b) % 127 in block
    b: every output isolates one pair of scale bytes, and over the outputs every byte meets every
    block. Globals keep all products in fp32's normal range. Run with the decode (4 experts of 32
    rows) and the prefill tactic (1 expert of 128 rows)."""
    K, N = 256, 128
    rows = 128
    rng = np.random.default_rng(91)
    packed, mask, _, _ = synth.random_sparse_weights(92, 1, N, K, 1)
    wscale = np.array([[(n + 17 * b) % 127 for b in range(K // 32)] for n in range(N)], np.uint8)[None]
    codes = np.zeros((rows, K // 2), np.uint8)
    ascale = rng.integers(0, 0x7F, size=(rows, K // 32)).astype(np.uint8)
    for r in range(rows):
        b = r % 8
        codes[r, 16 * b:16 * b + 16] = rng.integers(0, 256, 16)
        ascale[r, b] = r % 127
    for E in (1, 4):
        offsets = np.arange(0, rows + 1, rows // E).astype(np.int32)
        wg = np.full((E, 1), np.float32(2.0 ** -3), np.float32)
        a_global = np.full(E, np.float32(2.0 ** -3), np.float32)
        pk, mk, sc = (np.repeat(t, E, axis=0) for t in (packed, mask, wscale))
        w = moesq.SparseWeights(*(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in (pk, mk, sc, wg)))
        if layout == 1:
            w = moesq.prepare_weights(w)
        out = moesq.grouped_gemm(torch.from_numpy(codes).to(DEV), torch.from_numpy(ascale).to(DEV),
                                 torch.from_numpy(a_global).to(DEV), torch.from_numpy(offsets).to(DEV), w)
        ref = moe.grouped_gemm(codes, ascale, a_global, offsets, pk, mk, sc, wg)
        # bound per element: 32 kept products (exact) summed with at most 4 fp32 roundings + 2 global
        # products, each at most one unit of 2^-24 of the sum of |terms|
        mag = np.zeros_like(ref)
        for e in range(E):
            r0, r1 = offsets[e], offsets[e + 1]
            X = nvfp4.dequantize(codes[r0:r1], ascale[r0:r1], np.float64(a_global[e]))
            W = np.abs(moe.dequant_weight(pk[e], mk[e], sc[e], wg[e]))
            mag[r0:r1] = np.abs(X) @ W.T
        got = out.cpu().numpy().astype(np.float64)
        assert (np.abs(got - ref) <= 8 * 2.0 ** -24 * mag + 1e-37).all(), E
        assert np.isin(np.arange(127), ascale[np.arange(rows), np.arange(rows) % 8]).all()


def _ffn_both_paths(x, ids, wts, w13, w2, g13, g2):
    """moe_ffn on the one-launch path and on the separate launches (same inputs, own workspaces)."""
    T, H = x.shape
    k = ids.shape[1]
    E, I = w13.E, w2.K
    res = []
    for flags in (moesq.FLAG_FUSED, moesq.FLAG_UNFUSED):
        lay = moesq.ffn_layout(T, H, I, k, E, flags)
        ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
        ws.fill_(0xA5)                                   # arbitrary contents, barrier area included
        out = moesq.moe_ffn(x, torch.from_numpy(ids).to(DEV), torch.from_numpy(wts).to(DEV), w13, w2,
                            torch.from_numpy(g13).to(DEV), torch.from_numpy(g2).to(DEV), workspace=ws, flags=flags)
        inter = {kk: v.cpu().numpy() for kk, v in moesq.ffn_intermediates(ws, T, H, I, k, E).items()}
        res.append((lay["fused"], out.cpu().numpy(), inter))
    return res


@pytest.mark.parametrize("case", ["qwen3_30b_decode", "dup_invalid", "skewed"])
def test_moe_ffn_fused_matches_separate_launches(case):
    """The one-launch decode path against the separate launches, bit for bit: output and every
    intermediate (rows of dropped pairs excepted). Duplicate and invalid router ids, and an expert with
    more than one m-block (32 rows), are covered by the small cases."""
    if case == "qwen3_30b_decode":
        wl = synth.WORKLOADS[case]
        E, H, I, T, k = wl.E, wl.H, wl.I, wl.T, wl.k
        w13, w2, dense_expert = _layer(0, E, H, I)
        x = synth.activations(0, T, H, device=DEV)
        ids, wts = synth.routing(0, T, E, k)
    else:
        E, H, I, T, k = (8, 512, 256, 48, 4) if case == "dup_invalid" else (8, 256, 512, 96, 2)
        w13, w2, dense_expert = _layer(31, E, H, I, True)
        x = synth.activations(32, T, H, device=DEV)
        ids, wts = synth.routing(33, T, E, k)
        if case == "dup_invalid":
            ids[3, 1] = ids[3, 0]                        # a token naming one expert twice
            ids[5, 2] = -1                               # a dropped pair
            ids[7, 0] = E + 3                            # invalid ids, counted in status
            ids[9, 3] = -5
        else:
            ids[:70, 0] = 0                              # expert 0: 70+ rows, three m-blocks
            ids[:70, 1] = np.where(ids[:70, 1] == 0, 1, ids[:70, 1])
    clean = np.where((ids < -1) | (ids >= E), -1, ids)     # invalid ids are dropped like -1
    g13, g2 = _globals(x, clean, E, dense_expert, False)
    (f_on, out_f, it_f), (f_off, out_u, it_u) = _ffn_both_paths(x, ids, wts, w13, w2, g13, g2)
    assert f_on == 1 and f_off == 0
    assert np.array_equal(out_f, out_u)
    for key in ("counts", "offsets", "inv", "status"):
        assert np.array_equal(it_f[key], it_u[key]), key
    n = int(it_u["offsets"][-1])
    assert np.array_equal(it_f["sorted"][:n], it_u["sorted"][:n])
    live = it_u["sorted"][:n]
    for key in ("a13_codes", "a13_scales"):
        assert np.array_equal(it_f[key][live], it_u[key][live]), key
    for key in ("a2_codes", "a2_scales", "down_rows"):
        assert np.array_equal(it_f[key][:n], it_u[key][:n]), key
    rc, ro, rs, ri = moe.permute(clean, E)
    assert np.array_equal(it_f["offsets"], ro) and np.array_equal(it_f["inv"], ri)
    assert int(it_f["status"][0]) == int(((ids < -1) | (ids >= E)).sum())


@pytest.mark.parametrize("T", [64, 1024])
def test_moe_ffn_graph_replay_matches_eager(T):
    """A moe_ffn call captured into a HIP graph (no allocation, memset or host synchronization on its
    path) replays to the eager result bit for bit, three times over, with other eager work of the
    program (another FFN call on other inputs, a torch product) and synchronizations between the
    replays. T = 64 runs the decode kernels, T = 1024 the large-batch ones (several routing tiles)."""
    E, H, I, k = 8, 512, 256, 4
    w13, w2, dense_expert = _layer(61, E, H, I)
    x = synth.activations(62, T, H, device=DEV)
    ids, wts = synth.routing(63, T, E, k)
    g13, g2 = _globals(x, ids, E, dense_expert)
    x2 = synth.activations(64, T, H, device=DEV)
    ids2, wts2 = synth.routing(65, T, E, k)
    args = (torch.from_numpy(ids).to(DEV), torch.from_numpy(wts).to(DEV), w13, w2,
            torch.from_numpy(g13).to(DEV), torch.from_numpy(g2).to(DEV))
    args2 = (torch.from_numpy(ids2).to(DEV), torch.from_numpy(wts2).to(DEV), w13, w2,
             torch.from_numpy(g13).to(DEV), torch.from_numpy(g2).to(DEV))
    ref = moesq.moe_ffn(x, *args).cpu()
    ref2 = moesq.moe_ffn(x2, *args2).cpu()
    ws = torch.empty(moesq.ffn_layout(T, H, I, k, E)["total"], dtype=torch.uint8, device=DEV)
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moesq.moe_ffn(x, *args, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moesq.moe_ffn(x, *args, out=out, workspace=ws)
    a = torch.randn(256, 256, device=DEV)
    for i in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), ref), i
        assert torch.equal(moesq.moe_ffn(x2, *args2).cpu(), ref2), i     # eager work between replays
        a = a @ a.T / 256.0
        torch.cuda.synchronize()


@pytest.mark.parametrize("flags", [0, moesq.FLAG_FUSED])
def test_stage_events_time_the_kernels(flags):
    """moesq_set_stage_events with 13 events: the five stage events bracket the stages and every
    stage's kernels record their own start/end pair (hipExtLaunchKernel); each kernel pair lies
    inside its stage interval, and the outputs are those of a call without events."""
    import bench
    E, H, I, T, k = 8, 512, 256, 64, 4
    w13, w2, dense_expert = _layer(41, E, H, I)
    x = synth.activations(42, T, H, device=DEV)
    ids, wts = synth.routing(43, T, E, k)
    g13, g2 = _globals(x, ids, E, dense_expert)
    args = (x, torch.from_numpy(ids).to(DEV), torch.from_numpy(wts).to(DEV), w13, w2,
            torch.from_numpy(g13).to(DEV), torch.from_numpy(g2).to(DEV))
    ref = moesq.moe_ffn(*args, flags=flags).cpu()
    ev = bench.HipEvents()
    evs = ev.create(13)
    try:
        moesq.set_stage_events(evs)
        out = moesq.moe_ffn(*args, flags=flags)
        moesq.set_stage_events(None)
        torch.cuda.synchronize()
        stage = [ev.elapsed_ms(evs[j], evs[j + 1]) for j in range(4)]
        kern = [ev.elapsed_ms(evs[5 + 2 * j], evs[6 + 2 * j]) for j in range(4)]
        fused = moesq.ffn_layout(T, H, I, k, E, flags)["fused"] == 1
        if fused:
            # one kernel: its pair lies inside the whole call; the other pairs are back-to-back event
            # records after it, empty intervals like the stage intervals that follow the kernel (up
            # to a few microseconds of event-record jitter) and far shorter than the kernel
            assert 0.0 < kern[0] <= sum(stage) + 1e-3, (stage, kern)
            assert all(t <= max(stage[1:]) + 5e-3 and t < 0.5 * kern[0] for t in kern[1:]), (stage, kern)
        else:
            for s_ms, k_ms in zip(stage, kern):
                assert 0.0 < k_ms <= s_ms + 1e-3, (stage, kern)
        assert torch.equal(out.cpu(), ref)
    finally:
        moesq.set_stage_events(None)
        ev.destroy(evs)


def test_probe_read_returns_bytes_and_keeps_sink():
    """The read probe reads all of src (1 MiB of ones: every thread's fold is 0, not the constant that
    triggers the store) and leaves the sink alone."""
    src = torch.ones(1 << 20, dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    assert moesq.probe_read(src, sink) == 1 << 20
    torch.cuda.synchronize()
    assert sink.item() == 7


def test_probe_smfmac_counts_and_writes():
    """The MFMA throughput probe issues blocks x 4 waves x iters x 32 instructions and writes its sink."""
    sink = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device=DEV)
    n = moesq.probe_smfmac(4, 16, sink)
    torch.cuda.synchronize()
    assert n == 4 * 4 * 16 * 32
    assert torch.isfinite(sink).all()


def test_fused_barrier_timeout_is_reported():
    """A spin limit of 0 polls makes every bounded barrier wait of the one-launch path give up at once
    (every workgroup still exits); the call with SYNC_CHECK reports MOESQ_ERR_DEVICE. The next call on
    the same workspace, with the default limit, matches the separate launches bit for bit."""
    wl = synth.WORKLOADS["qwen3_30b_decode"]
    E, H, I, T, k = wl.E, wl.H, wl.I, wl.T, wl.k
    w13, w2, dense_expert = _layer(0, E, H, I)
    x = synth.activations(0, T, H, device=DEV)
    ids, wts = synth.routing(0, T, E, k)
    g13, g2 = _globals(x, ids, E, dense_expert, False)
    lay = moesq.ffn_layout(T, H, I, k, E, moesq.FLAG_FUSED)
    assert lay["fused"] == 1
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=DEV)
    args = (x, torch.from_numpy(ids).to(DEV), torch.from_numpy(wts).to(DEV), w13, w2,
            torch.from_numpy(g13).to(DEV), torch.from_numpy(g2).to(DEV))
    moesq.set_fused_spin_limit(0)
    try:
        with pytest.raises(moesq.MoesqError) as ei:
            moesq.moe_ffn(*args, workspace=ws, flags=moesq.FLAG_FUSED | moesq.FLAG_SYNC_CHECK)
        assert ei.value.status == -5, str(ei.value)
    finally:
        moesq.set_fused_spin_limit(-1)
    out = moesq.moe_ffn(*args, workspace=ws, flags=moesq.FLAG_FUSED | moesq.FLAG_SYNC_CHECK)
    ref = moesq.moe_ffn(*args, flags=moesq.FLAG_UNFUSED | moesq.FLAG_SYNC_CHECK)
    assert torch.equal(out, ref)
