"""Host-side checks of the C ABI (no GPU): the library loads, exports every declared symbol, and its
synchronous argument checks return the documented status without launching anything."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

moesq = pytest.importorskip("sparse_quantized_moe_amd")
if not os.path.exists(moesq.library_path):
    pytest.skip("libmoesq.so not built (run python -m sparse_quantized_moe_amd.build)", allow_module_level=True)

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP, DEVICE = 0, -1, -2, -3, -4, -5


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "moesq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moesq_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L = moesq.lib()
    decl = declared_symbols()
    assert len(decl) >= 14
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(decl) == sorted(moesq.EXPORTED_SYMBOLS)
    hdr = open(os.path.join(ROOT, "include", "moesq.h")).read()
    declared = int(re.search(r"#define MOESQ_ABI_VERSION (\d+)", hdr).group(1))
    assert moesq.abi_version() == moesq.ABI_VERSION == declared


def test_status_strings():
    L = moesq.lib()
    for s, want in [(OK, b"ok"), (INVALID, b"invalid argument"), (UNSUPPORTED, b"unsupported shape"),
                    (WORKSPACE, b"workspace too small"), (HIP, b"HIP error"),
                    (DEVICE, b"device-side wait ran out")]:
        assert L.moesq_status_string(s) == want


def test_layout_is_aligned_and_ordered():
    lay = moesq.ffn_layout(256, 2048, 768, 8, 128)
    offs = [lay[n] for n in ("counts", "offsets", "tile_offsets", "status", "sorted", "inv", "a13_codes",
                             "a13_scales", "a2_codes", "a2_scales", "down_rows")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    P = 256 * 8
    assert lay["down_rows"] + P * 2048 * 4 <= lay["total"]
    assert lay["rows_per_mblock"] == 32                     # decode tactic for 16 rows per expert
    assert moesq.ffn_layout(8192, 2048, 768, 8, 128)["rows_per_mblock"] == 128
    assert moesq.lib().moesq_moe_ffn_workspace_size(256, 2048, 768, 8, 128, 0) == lay["total"]


def _weights(E=2, N=64, K=256, G=1, ptr=16):
    return moesq._CWeights(ptr, ptr, ptr, ptr, E, N, K, G)


def test_argument_checks_return_status_without_launching():
    L = moesq.lib()
    P = ctypes.c_void_p(16)
    # quantize: K not a multiple of 32, null pointers, bad dtype
    assert L.moesq_quantize_act(P, 0, 4, 48, 48, None, None, 0, P, P, P, None) == INVALID
    assert L.moesq_quantize_act(None, 0, 4, 64, 64, None, None, 0, P, P, P, None) == INVALID
    assert L.moesq_quantize_act(P, 7, 4, 64, 64, None, None, 0, P, P, P, None) == INVALID
    assert L.moesq_quantize_act(P, 0, 0, 64, 64, None, None, 0, P, P, P, None) == OK        # rows = 0: no-op
    L.moesq_quantize_act(P, 0, 4, 48, 48, None, None, 0, P, P, P, None)
    assert b"K must be a multiple of 32" in L.moesq_last_error()
    # permute: k out of range, too many experts
    assert L.moesq_permute(P, 4, 0, 8, P, P, P, P, P, None, 0, None) == INVALID
    assert L.moesq_permute(P, 4, 2, 2000, P, P, P, P, P, None, 0, None) == UNSUPPORTED
    # more than one 512-token tile needs scratch
    assert L.moesq_permute_workspace_size(512, 8) == 0
    assert L.moesq_permute_workspace_size(513, 8) == 2 * 9 * 4
    assert L.moesq_permute(P, 1000, 2, 8, P, P, P, P, P, None, 0, None) == WORKSPACE
    # grouped GEMM: K % 256, G, workspace
    w = _weights(K=96)
    assert L.moesq_grouped_gemm(P, P, P, P, 4, ctypes.byref(w), P, P, 1 << 20, None) == UNSUPPORTED
    w = _weights(G=3)
    assert L.moesq_grouped_gemm(P, P, P, P, 4, ctypes.byref(w), P, P, 1 << 20, None) == INVALID
    w = _weights()
    assert L.moesq_grouped_gemm(P, P, P, P, 4, ctypes.byref(w), P, P, 4, None) == WORKSPACE
    assert b"workspace" in L.moesq_last_error()
    assert L.moesq_grouped_gemm(P, P, P, P, 4, None, P, P, 1 << 20, None) == INVALID
    # moe_ffn: inconsistent shapes, missing fused gate|up, workspace
    H, I, E = 256, 256, 4
    w13 = _weights(E=E, N=2 * I, K=H, G=2)
    w2 = _weights(E=E, N=H, K=I, G=1)
    w2_bad = _weights(E=E, N=H + 64, K=I, G=1)
    args = lambda a, b, ws: (P, 8, H, P, P, 2, ctypes.byref(a), ctypes.byref(b), P, P, P, P, ws, 0, None)
    assert L.moesq_moe_ffn(*args(w13, w2_bad, 1 << 30)) == INVALID
    assert L.moesq_moe_ffn(*args(_weights(E=E, N=2 * I, K=H, G=1), w2, 1 << 30)) == INVALID
    assert L.moesq_moe_ffn(*args(w13, w2, 16)) == WORKSPACE
    assert L.moesq_moe_ffn(P, 0, H, P, P, 2, ctypes.byref(w13), ctypes.byref(w2), P, P, P, P, 16, 0, None) == OK
    # 32-bit buffer offsets: the down input codes (I > H) past 2 GiB are refused, the gate/up ones fit
    Hs, Is, Ts, ks = 256, 4096, 131072, 8                   # T*k*I/2 = 2^31, T*k*H/2 = 2^27
    w13s = _weights(E=E, N=2 * Is, K=Hs, G=2)
    w2s = _weights(E=E, N=Hs, K=Is, G=1)
    assert L.moesq_moe_ffn(P, Ts, Hs, P, P, ks, ctypes.byref(w13s), ctypes.byref(w2s), P, P, P, P, 1 << 62, 0,
                           None) == UNSUPPORTED
    assert b"2 GiB" in L.moesq_last_error()
    assert L.moesq_moe_ffn(P, Ts - 1, Hs, P, P, ks, ctypes.byref(w13s), ctypes.byref(w2s), P, P, P, P, 16, 0,
                           None) == WORKSPACE                # one token fewer: past the offset check
    # the allocation-free variant: its static scratch bounds the call (checked before any device call)
    assert L.moesq_noalloc_scratch_bytes() == 64 << 20
    w13d = _weights(E=128, N=2 * 768, K=2048, G=2)
    w2d = _weights(E=128, N=2048, K=768, G=1)
    assert L.moesq_moe_ffn_workspace_size(1024, 2048, 768, 8, 128, 0) > 64 << 20
    assert L.moesq_moe_ffn_noalloc(P, 1024, 2048, P, P, 8, ctypes.byref(w13d), ctypes.byref(w2d), P, P, P, 0,
                                   None) == WORKSPACE
    assert b"static scratch" in L.moesq_last_error()
    assert L.moesq_moe_ffn_noalloc(P, 8, 2048, P, P, 8, ctypes.byref(w13d), ctypes.byref(w2_bad), P, P, P, 0,
                                   None) == INVALID          # the checks of moesq_moe_ffn
    assert L.moesq_moe_ffn_noalloc(P, 0, 2048, P, P, 8, ctypes.byref(w13d), ctypes.byref(w2d), P, P, P, 0,
                                   None) == OK               # T = 0: a no-op
    # router: k out of range, too many experts, bad dtype, null outputs; no tokens is a no-op
    assert L.moesq_route_topk(P, 0, 4, 8, 9, 1, P, P, None) == INVALID
    assert L.moesq_route_topk(P, 0, 4, 128, 65, 1, P, P, None) == INVALID
    assert L.moesq_route_topk(P, 0, 4, 1025, 8, 1, P, P, None) == INVALID
    assert L.moesq_route_topk(P, 7, 4, 8, 2, 1, P, P, None) == INVALID
    assert L.moesq_route_topk(P, 0, 4, 8, 2, 1, None, P, None) == INVALID
    assert b"null pointer" in L.moesq_last_error()
    assert L.moesq_route_topk(None, 0, 0, 8, 2, 1, None, None, None) == OK
    # gate/up fold: odd N, K not a multiple of 32, null pointers; no experts is a no-op
    assert L.moesq_fold_gate_up_globals(P, P, 4, 63, 256, None) == INVALID
    assert L.moesq_fold_gate_up_globals(P, P, 4, 64, 48, None) == INVALID
    assert L.moesq_fold_gate_up_globals(None, P, 4, 64, 256, None) == INVALID
    assert L.moesq_fold_gate_up_globals(None, None, 0, 64, 256, None) == OK
    # probes: bad sizes, null or misaligned pointers
    assert L.moesq_probe_read(P, 0, P, None) == INVALID
    assert L.moesq_probe_read(P, 40, P, None) == INVALID
    assert L.moesq_probe_read(None, 64, P, None) == INVALID
    assert L.moesq_probe_read(ctypes.c_void_p(24), 64, P, None) == INVALID
    assert L.moesq_probe_smfmac(0, 4, P, ctypes.byref(ctypes.c_int64()), None) == INVALID
    # compress and codec
    assert L.moesq_compress_weights(P, 4, 40, P, P, P, P, None) == INVALID
    assert L.moesq_validate_weights(P, 4, 40, P, None) == INVALID
    assert L.moesq_unpack_pair_bitmask(P, P, 4, 40, P, P, None) == INVALID
    assert L.moesq_pack_pair_bitmask(P, 4, 40, P, P, P, None) == INVALID


def test_tiled_layout_size_and_checks():
    L = moesq.lib()
    assert L.moesq_tiled_bytes(128, 1536, 2048) == 128 * (1536 // 16) * (2048 // 256) * 1408
    assert L.moesq_tiled_bytes(128, 1536, 2048) == 128 * 1536 * 2048 * 11 // 32     # same bytes as stored
    assert L.moesq_tiled_bytes(1, 24, 256) == 0 and L.moesq_tiled_bytes(1, 16, 96) == 0
    P = ctypes.c_void_p(16)
    w = _weights(E=2, N=64, K=256)
    w.layout = 1
    assert L.moesq_prepare_weights(ctypes.byref(w), P, None) == INVALID        # source must be pair-bitmask
    w.layout = 0
    w.N = 24
    assert L.moesq_prepare_weights(ctypes.byref(w), P, None) == UNSUPPORTED
    bad = _weights()
    bad.layout = 7
    assert L.moesq_grouped_gemm(P, P, P, P, 4, ctypes.byref(bad), P, P, 1 << 20, None) == INVALID
    tiled = _weights()
    tiled.layout = 1
    tiled.mask = None
    tiled.scale = None
    assert L.moesq_grouped_gemm(P, P, P, P, 4, ctypes.byref(tiled), P, P, 4, None) == WORKSPACE  # past the layout checks


def test_binding_refuses_cpu_tensors():
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(moesq.MoesqError):
        moesq.quantize_act(x, torch.ones(1))
