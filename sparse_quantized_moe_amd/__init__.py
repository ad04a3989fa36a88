"""moesq: paired-4:8 sparse NVFP4 (W4A4) MoE expert path for AMD Instinct MI355X (gfx950).

Thin ctypes binding of the in-tree HIP library ``libmoesq.so`` (C ABI in ``include/moesq.h``). It only
marshals arguments: every step runs in the library's kernels on the tensors' device, on torch's
current stream. There is no CPU fallback: a missing library or a CPU tensor raises ``MoesqError``.

Weights use the pair-bitmask storage of the MoESQ model cards ("Sparse storage layout"): per expert
linear ``packed`` u8 [N, K/4], ``mask`` u8 [N, K/16], ``scale`` u8 (E4M3 bits) [N, K/32] and an fp32
global per tensor (two, gate and up, for a fused gate|up linear).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

__all__ = [
    "MoesqError", "SparseWeights", "lib", "library_path", "abi_version", "ABI_VERSION", "quantize_act", "permute",
    "grouped_gemm", "moe_ffn", "ffn_layout", "compress_weights", "compress_moe_layer", "validate_weights",
    "pack_pair_bitmask", "unpack_pair_bitmask", "FLAG_SYNC_CHECK", "FLAG_UNFUSED", "FLAG_FUSED", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libmoesq.so")
#: The C ABI version (MOESQ_ABI_VERSION in include/moesq.h) these bindings are declared for.
ABI_VERSION = 6
FLAG_SYNC_CHECK = 1
FLAG_UNFUSED = 2      # moe_ffn: separate launches even where the one-launch decode path applies
FLAG_FUSED = 4        # moe_ffn: the one-launch decode path wherever it applies

#: Every function the C ABI exports (include/moesq.h).
EXPORTED_SYMBOLS = (
    "moesq_abi_version", "moesq_status_string", "moesq_last_error", "moesq_quantize_act", "moesq_permute",
    "moesq_grouped_gemm_workspace_size", "moesq_grouped_gemm", "moesq_moe_ffn_layout",
    "moesq_moe_ffn_workspace_size", "moesq_moe_ffn", "moesq_compress_weights", "moesq_validate_weights",
    "moesq_unpack_pair_bitmask", "moesq_pack_pair_bitmask", "moesq_set_stage_events", "moesq_tiled_bytes",
    "moesq_prepare_weights", "moesq_unprepare_weights", "moesq_permute_workspace_size", "moesq_probe_smfmac", "moesq_probe_read",
    "moesq_route_topk", "moesq_fold_gate_up_globals", "moesq_set_fused_spin_limit", "moesq_moe_ffn_noalloc",
    "moesq_noalloc_scratch_bytes",
)


class MoesqError(RuntimeError):
    def __init__(self, msg: str, status: int = 0):
        super().__init__(msg)
        self.status = status


class _CWeights(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("global_", ctypes.c_void_p), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("G", ctypes.c_int32), ("layout", ctypes.c_int32)]


LAYOUT_PAIR_BITMASK = 0
LAYOUT_TILED = 1


class _CLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("counts", "offsets", "tile_offsets", "sorted", "inv", "status",
                                                "a13_codes", "a13_scales", "a2_codes", "a2_scales",
                                                "down_rows", "route_scratch", "sync", "total")] + \
        [("rows_per_mblock", ctypes.c_int32), ("fused", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None
_P, _I32, _I64, _SZ, _U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint32


def _declare(L: ctypes.CDLL) -> None:
    sig = {
        "moesq_abi_version": (ctypes.c_int, []),
        "moesq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moesq_last_error": (ctypes.c_char_p, []),
        "moesq_quantize_act": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I32, _I64, _P, _P, _I32, _P, _P, _P, _P]),
        "moesq_permute_workspace_size": (_SZ, [_I64, _I32]),
        "moesq_permute": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        "moesq_grouped_gemm_workspace_size": (_SZ, [_I32]),
        "moesq_grouped_gemm": (ctypes.c_int, [_P, _P, _P, _P, _I64, ctypes.POINTER(_CWeights), _P, _P, _SZ, _P]),
        "moesq_moe_ffn_layout": (ctypes.c_int, [_I64, _I32, _I32, _I32, _I32, _U32, ctypes.POINTER(_CLayout)]),
        "moesq_moe_ffn_workspace_size": (_SZ, [_I64, _I32, _I32, _I32, _I32, _U32]),
        "moesq_moe_ffn": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _I32, ctypes.POINTER(_CWeights),
                                         ctypes.POINTER(_CWeights), _P, _P, _P, _P, _SZ, _U32, _P]),
        "moesq_moe_ffn_noalloc": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _I32, ctypes.POINTER(_CWeights),
                                                 ctypes.POINTER(_CWeights), _P, _P, _P, _U32, _P]),
        "moesq_noalloc_scratch_bytes": (_SZ, []),
        "moesq_compress_weights": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P, _P, _P]),
        "moesq_validate_weights": (ctypes.c_int, [_P, _I64, _I32, _P, _P]),
        "moesq_unpack_pair_bitmask": (ctypes.c_int, [_P, _P, _I64, _I32, _P, _P, _P]),
        "moesq_pack_pair_bitmask": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P, _P]),
        "moesq_set_stage_events": (ctypes.c_int, [_P, _I32]),
        "moesq_set_fused_spin_limit": (ctypes.c_int, [_I64]),
        "moesq_probe_smfmac": (ctypes.c_int, [_I32, _I32, _P, ctypes.POINTER(_I64), _P]),
        "moesq_probe_read": (ctypes.c_int, [_P, _I64, _P, _P]),
        "moesq_route_topk": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I32, _I32, _I32, _P, _P, _P]),
        "moesq_tiled_bytes": (_SZ, [_I32, _I32, _I32]),
        "moesq_fold_gate_up_globals": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P]),
        "moesq_prepare_weights": (ctypes.c_int, [ctypes.POINTER(_CWeights), _P, _P]),
        "moesq_unprepare_weights": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise MoesqError(f"{library_path} is missing: build it with `python -m sparse_quantized_moe_amd.build`")
        L = ctypes.CDLL(library_path)
        _declare(L)
        if L.moesq_abi_version() != ABI_VERSION:
            raise MoesqError(f"{library_path} has C ABI {L.moesq_abi_version()}, these bindings expect "
                             f"{ABI_VERSION}: rebuild it with `python -m sparse_quantized_moe_amd.build`")
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().moesq_abi_version()


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise MoesqError(f"{L.moesq_status_string(status).decode()}: {L.moesq_last_error().decode()}", status)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MoesqError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if dtype is not None and t.dtype != dtype:
        raise MoesqError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoesqError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclasses.dataclass
class SparseWeights:
    """One linear of every expert (device tensors).

    Pair-bitmask layout: ``packed`` u8 [E, N, K/4], ``mask`` u8 [E, N, K/16], ``scale`` u8 [E, N, K/32].
    Tiled layout (``layout=LAYOUT_TILED``, from ``prepare_weights``): ``packed`` holds the kernel
    records, ``mask``/``scale`` are None and ``shape`` gives (E, N, K).
    """
    packed: torch.Tensor
    mask: Optional[torch.Tensor]
    scale: Optional[torch.Tensor]
    global_scale: torch.Tensor  # float32 [E, G]
    layout: int = LAYOUT_PAIR_BITMASK
    shape: Optional[tuple] = None

    @property
    def E(self) -> int:
        return self.shape[0] if self.shape else self.packed.shape[0]

    @property
    def N(self) -> int:
        return self.shape[1] if self.shape else self.packed.shape[1]

    @property
    def K(self) -> int:
        return self.shape[2] if self.shape else self.packed.shape[2] * 4

    @property
    def G(self) -> int:
        return self.global_scale.shape[1]

    def c_struct(self) -> _CWeights:
        E, N, K = self.E, self.N, self.K
        if self.layout == LAYOUT_TILED:
            if self.packed.numel() != lib().moesq_tiled_bytes(E, N, K):
                raise MoesqError("tiled buffer size does not match (E, N, K)")
            return _CWeights(_dev(self.packed, "packed", torch.uint8), None, None,
                             _dev(self.global_scale, "global_scale", torch.float32), E, N, K, self.G, LAYOUT_TILED)
        if tuple(self.mask.shape) != (E, N, K // 16) or tuple(self.scale.shape) != (E, N, K // 32):
            raise MoesqError("mask/scale shapes do not match packed")
        return _CWeights(_dev(self.packed, "packed", torch.uint8), _dev(self.mask, "mask", torch.uint8),
                         _dev(self.scale, "scale", torch.uint8),
                         _dev(self.global_scale, "global_scale", torch.float32), E, N, K, self.G,
                         LAYOUT_PAIR_BITMASK)

    def nbytes(self) -> int:
        ts = [t for t in (self.packed, self.mask, self.scale, self.global_scale) if t is not None]
        return sum(t.numel() * t.element_size() for t in ts)


def prepare_weights(w: SparseWeights) -> SparseWeights:
    """Load-time re-tiling of pair-bitmask weights into the kernels' layout (the same bytes)."""
    E, N, K = w.E, w.N, w.K
    n = lib().moesq_tiled_bytes(E, N, K)
    if n == 0:
        raise MoesqError("the tiled layout needs N % 16 == 0 and K % 256 == 0")
    tiled = torch.empty(n, dtype=torch.uint8, device=w.packed.device)
    cw = w.c_struct()
    _check(lib().moesq_prepare_weights(ctypes.byref(cw), _dev(tiled, "tiled"), _stream()))
    return SparseWeights(tiled, None, None, w.global_scale, LAYOUT_TILED, (E, N, K))


def unprepare_weights(w: SparseWeights) -> SparseWeights:
    """The pair-bitmask tensors back from tiled weights."""
    E, N, K = w.E, w.N, w.K
    dev = w.packed.device
    packed = torch.empty((E, N, K // 4), dtype=torch.uint8, device=dev)
    mask = torch.empty((E, N, K // 16), dtype=torch.uint8, device=dev)
    scale = torch.empty((E, N, K // 32), dtype=torch.uint8, device=dev)
    _check(lib().moesq_unprepare_weights(_dev(w.packed, "tiled", torch.uint8), E, N, K, _dev(packed, "packed"),
                                         _dev(mask, "mask"), _dev(scale, "scale"), _stream()))
    return SparseWeights(packed, mask, scale, w.global_scale)


def fold_gate_up_globals(w13: SparseWeights) -> SparseWeights:
    """In place: fold each expert's up/gate global ratio into its up block scales and set the up
    global to the gate's (pair-bitmask layout, G = 2). Returns ``w13``."""
    if w13.layout != LAYOUT_PAIR_BITMASK or w13.G != 2:
        raise MoesqError("fold_gate_up_globals needs a pair-bitmask gate|up linear with 2 globals per expert")
    E, N, K = w13.E, w13.N, w13.K
    if tuple(w13.scale.shape) != (E, N, K // 32):
        raise MoesqError("scale shape does not match packed")
    _check(lib().moesq_fold_gate_up_globals(_dev(w13.scale, "scale", torch.uint8),
                                            _dev(w13.global_scale, "global_scale", torch.float32), E, N, K, _stream()))
    return w13


__all__ += ["LAYOUT_PAIR_BITMASK", "LAYOUT_TILED", "prepare_weights", "unprepare_weights", "fold_gate_up_globals"]


def quantize_act(x: torch.Tensor, global_scale: torch.Tensor, src_row: Optional[torch.Tensor] = None,
                 expert_offsets: Optional[torch.Tensor] = None, rows: Optional[int] = None):
    """NVFP4 codes [rows, K/2] and E4M3 scales [rows, K/32] of the rows of x (bf16 or fp32 [*, K])."""
    if x.dtype not in (torch.bfloat16, torch.float32) or x.dim() != 2:
        raise MoesqError("x must be a 2-D bf16 or fp32 tensor")
    K = x.shape[1]
    rows = (src_row.shape[0] if src_row is not None else x.shape[0]) if rows is None else rows
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    E = 0 if expert_offsets is None else expert_offsets.shape[0] - 1
    _check(lib().moesq_quantize_act(
        _dev(x, "x"), 1 if x.dtype == torch.float32 else 0, rows, K, x.stride(0),
        None if src_row is None else _dev(src_row, "src_row", torch.int32),
        None if expert_offsets is None else _dev(expert_offsets, "expert_offsets", torch.int32), E,
        _dev(global_scale, "global_scale", torch.float32), _dev(codes, "codes"), _dev(scales, "scales"), _stream()))
    return codes, scales


def permute(topk_ids: torch.Tensor, E: int):
    """(counts [E], offsets [E+1], sorted [T*k], inv [T*k], status [1]) int32 of the stable grouping."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_ = torch.full((T * k,), -1, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    ws_bytes = lib().moesq_permute_workspace_size(T, E)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().moesq_permute(_dev(topk_ids, "topk_ids", torch.int32), T, k, E, _dev(counts, "counts"),
                               _dev(offsets, "offsets"), _dev(sorted_, "sorted"), _dev(inv, "inv"),
                               _dev(status, "status"), _dev(ws, "workspace"), ws_bytes, _stream()))
    return counts, offsets, sorted_, inv, status


def grouped_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, a_global: torch.Tensor,
                 expert_offsets: torch.Tensor, w: SparseWeights, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 [rows, N]: each expert's rows of the NVFP4 activations times its sparse weight."""
    rows = a_codes.shape[0]
    if out is None:
        out = torch.zeros((rows, w.N), dtype=torch.float32, device=a_codes.device)
    ws_bytes = lib().moesq_grouped_gemm_workspace_size(w.E)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=a_codes.device)
    cw = w.c_struct()
    _check(lib().moesq_grouped_gemm(_dev(a_codes, "a_codes", torch.uint8), _dev(a_scales, "a_scales", torch.uint8),
                                    _dev(a_global, "a_global", torch.float32),
                                    _dev(expert_offsets, "expert_offsets", torch.int32), rows, ctypes.byref(cw),
                                    _dev(out, "out", torch.float32), _dev(ws, "workspace"), ws_bytes, _stream()))
    return out


def ffn_layout(T: int, H: int, I: int, k: int, E: int, flags: int = 0) -> dict:
    L = _CLayout()
    _check(lib().moesq_moe_ffn_layout(T, H, I, k, E, flags, ctypes.byref(L)))
    return {n: getattr(L, n) for n, _ in _CLayout._fields_}


def moe_ffn(x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor, w13: SparseWeights,
            w2: SparseWeights, a13_global: torch.Tensor, a2_global: torch.Tensor, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
    """fp32 [T, H] MoE FFN output of bf16 tokens x [T, H] (see moesq_moe_ffn)."""
    T, H = x.shape
    k = topk_ids.shape[1]
    I = w2.K
    ws_bytes = lib().moesq_moe_ffn_workspace_size(T, H, I, k, w13.E, flags)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    c13, c2 = w13.c_struct(), w2.c_struct()
    _check(lib().moesq_moe_ffn(_dev(x, "x", torch.bfloat16), T, H, _dev(topk_ids, "topk_ids", torch.int32),
                               _dev(topk_weights, "topk_weights", torch.float32), k, ctypes.byref(c13),
                               ctypes.byref(c2), _dev(a13_global, "a13_global", torch.float32),
                               _dev(a2_global, "a2_global", torch.float32), _dev(out, "out", torch.float32),
                               _dev(workspace, "workspace"), workspace.numel(), flags, _stream()))
    return out


def moe_ffn_noalloc(x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor, w13: SparseWeights,
                    w2: SparseWeights, a13_global: torch.Tensor, a2_global: torch.Tensor,
                    out: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
    """moesq_moe_ffn_noalloc: the FFN with the library's static device scratch as its workspace (no
    workspace argument; pass ``out`` to keep the call itself free of allocation)."""
    T, H = x.shape
    k = topk_ids.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    c13, c2 = w13.c_struct(), w2.c_struct()
    _check(lib().moesq_moe_ffn_noalloc(_dev(x, "x", torch.bfloat16), T, H, _dev(topk_ids, "topk_ids", torch.int32),
                                       _dev(topk_weights, "topk_weights", torch.float32), k, ctypes.byref(c13),
                                       ctypes.byref(c2), _dev(a13_global, "a13_global", torch.float32),
                                       _dev(a2_global, "a2_global", torch.float32), _dev(out, "out", torch.float32),
                                       flags, _stream()))
    return out


def ffn_intermediates(workspace: torch.Tensor, T: int, H: int, I: int, k: int, E: int) -> dict:
    """Views of the intermediates a moe_ffn call left in its workspace (stream-ordered after the call).
    a13 rows are in pair order (row p = t*k + j); a2 and down rows in sorted order (row inv[p])."""
    L = ffn_layout(T, H, I, k, E)
    P = T * k

    def view(off, n, dtype, shape):
        b = workspace[off: off + n * torch.tensor([], dtype=dtype).element_size()]
        return b.view(dtype).view(shape)
    return {
        "counts": view(L["counts"], E, torch.int32, (E,)),
        "offsets": view(L["offsets"], E + 1, torch.int32, (E + 1,)),
        "sorted": view(L["sorted"], P, torch.int32, (P,)),
        "inv": view(L["inv"], P, torch.int32, (P,)),
        "status": view(L["status"], 1, torch.int32, (1,)),
        "a13_codes": view(L["a13_codes"], P * H // 2, torch.uint8, (P, H // 2)),
        "a13_scales": view(L["a13_scales"], P * H // 32, torch.uint8, (P, H // 32)),
        "a2_codes": view(L["a2_codes"], P * I // 2, torch.uint8, (P, I // 2)),
        "a2_scales": view(L["a2_scales"], P * I // 32, torch.uint8, (P, I // 32)),
        "down_rows": view(L["down_rows"], P * H, torch.float32, (P, H)),
    }


__all__ += ["ffn_intermediates", "moe_ffn_noalloc"]


def compress_weights(w: torch.Tensor, packed: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                     scale: Optional[torch.Tensor] = None, global_out: Optional[torch.Tensor] = None):
    """Dense fp32 [N, K] -> (packed [N,K/4], mask [N,K/16], scale [N,K/32], global [1]) pair-bitmask NVFP4."""
    N, K = w.shape
    dev = w.device
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=dev) if packed is None else packed
    mask = torch.empty((N, K // 16), dtype=torch.uint8, device=dev) if mask is None else mask
    scale = torch.empty((N, K // 32), dtype=torch.uint8, device=dev) if scale is None else scale
    global_out = torch.empty(1, dtype=torch.float32, device=dev) if global_out is None else global_out
    _check(lib().moesq_compress_weights(_dev(w, "w", torch.float32), N, K, _dev(packed, "packed"), _dev(mask, "mask"),
                                        _dev(scale, "scale"), _dev(global_out, "global"), _stream()))
    return packed, mask, scale, global_out


def compress_moe_layer(E: int, H: int, I: int, dense_expert, device="cuda"):
    """Pair-bitmask storage of a whole MoE layer from ``dense_expert(e) -> (gate [I,H], up [I,H], down [H,I])``
    fp32 device tensors: returns (w13 with rows [gate; up] and G = 2, w2 with G = 1)."""
    w13 = SparseWeights(torch.empty((E, 2 * I, H // 4), dtype=torch.uint8, device=device),
                        torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device=device),
                        torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=device),
                        torch.empty((E, 2), dtype=torch.float32, device=device))
    w2 = SparseWeights(torch.empty((E, H, I // 4), dtype=torch.uint8, device=device),
                       torch.empty((E, H, I // 16), dtype=torch.uint8, device=device),
                       torch.empty((E, H, I // 32), dtype=torch.uint8, device=device),
                       torch.empty((E, 1), dtype=torch.float32, device=device))
    for e in range(E):
        g, u, d = dense_expert(e)
        compress_weights(g.contiguous(), w13.packed[e, :I], w13.mask[e, :I], w13.scale[e, :I], w13.global_scale[e, 0:1])
        compress_weights(u.contiguous(), w13.packed[e, I:], w13.mask[e, I:], w13.scale[e, I:], w13.global_scale[e, 1:2])
        compress_weights(d.contiguous(), w2.packed[e], w2.mask[e], w2.scale[e], w2.global_scale[e, 0:1])
    return w13, w2


#: Stages of one moe_ffn call, in the order set_stage_events() brackets them.
FFN_STAGES = ("route", "gemm_gate_up", "gemm_down", "combine")


def set_stage_events(events) -> None:
    """Record HIP events around the stages of later moe_ffn calls on this thread: ``events`` is a
    ctypes array of >= len(FFN_STAGES) + 1 hipEvent_t handles (None disables)."""
    if events is None:
        _check(lib().moesq_set_stage_events(None, 0))
    else:
        _check(lib().moesq_set_stage_events(ctypes.cast(events, ctypes.c_void_p), len(events)))


def set_fused_spin_limit(polls: int) -> None:
    """Polls after which a barrier wait of the one-launch decode path gives up, for later moe_ffn calls
    on this thread (negative: the default; 0: every wait gives up at once); a failure-handling test
    hook (see moesq_set_fused_spin_limit)."""
    _check(lib().moesq_set_fused_spin_limit(polls))


__all__ += ["FFN_STAGES", "set_stage_events", "set_fused_spin_limit", "probe_smfmac", "probe_read", "route_topk"]


def route_topk(logits: torch.Tensor, k: int, renormalize: bool = True, out_ids: Optional[torch.Tensor] = None,
               out_weights: Optional[torch.Tensor] = None):
    """Router softmax top-k (see moesq_route_topk): logits [T, E] bf16 or fp32 on the device ->
    (topk_ids int32 [T, k], topk_weights fp32 [T, k])."""
    T, E = logits.shape
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise MoesqError("route_topk: logits must be bf16 or fp32")
    dtype = 1 if logits.dtype == torch.float32 else 0
    ids = out_ids if out_ids is not None else torch.empty((T, k), dtype=torch.int32, device=logits.device)
    wts = out_weights if out_weights is not None else torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moesq_route_topk(_dev(logits, "logits", logits.dtype), dtype, T, E, k, 1 if renormalize else 0,
                                  _dev(ids, "topk_ids", torch.int32), _dev(wts, "topk_weights", torch.float32),
                                  _stream()))
    return ids, wts


def probe_smfmac(blocks: int, iters: int, sink: torch.Tensor) -> int:
    """Launch the v_smfmac_f32_16x16x64_f16 throughput probe on the current stream (see
    moesq_probe_smfmac); returns the number of instructions issued. sink: >= blocks*256 fp32 on device."""
    if sink.numel() < blocks * 256:
        raise MoesqError("probe_smfmac: sink too small")
    n = ctypes.c_int64()
    _check(lib().moesq_probe_smfmac(blocks, iters, _dev(sink, "sink", torch.float32), ctypes.byref(n),
                                    _stream()))
    return n.value


def probe_read(src: torch.Tensor, sink: torch.Tensor) -> int:
    """Launch the HBM read-stream probe over all of src (contiguous, 16-byte multiple) on the current
    stream (see moesq_probe_read); returns the bytes read. sink: >= 1 int32 on device."""
    nbytes = src.numel() * src.element_size()
    if sink.numel() < 1:
        raise MoesqError("probe_read: sink too small")
    _check(lib().moesq_probe_read(_dev(src, "src"), nbytes, _dev(sink, "sink", torch.int32), _stream()))
    return nbytes


def validate_weights(mask: torch.Tensor, K: int) -> int:
    """Number of chunk masks without exactly two bits set (synchronizes)."""
    rows = mask.numel() // (K // 16)
    bad = torch.empty(1, dtype=torch.int32, device=mask.device)
    _check(lib().moesq_validate_weights(_dev(mask, "mask", torch.uint8), rows, K, _dev(bad, "bad"), _stream()))
    return int(bad.item())


def unpack_pair_bitmask(packed: torch.Tensor, mask: torch.Tensor, K: int):
    """Sparse -> dense packed NVFP4 [rows, K/2]; returns (dense, bad-count tensor)."""
    rows = packed.numel() // (K // 4)
    dense = torch.empty((rows, K // 2), dtype=torch.uint8, device=packed.device)
    bad = torch.empty(1, dtype=torch.int32, device=packed.device)
    _check(lib().moesq_unpack_pair_bitmask(_dev(packed, "packed", torch.uint8), _dev(mask, "mask", torch.uint8), rows, K,
                                           _dev(dense, "dense"), _dev(bad, "bad"), _stream()))
    return dense, bad


def pack_pair_bitmask(dense: torch.Tensor, K: int):
    """Dense packed NVFP4 [rows, K/2] -> (packed [rows, K/4], mask [rows, K/16], bad-count tensor)."""
    rows = dense.numel() // (K // 2)
    packed = torch.empty((rows, K // 4), dtype=torch.uint8, device=dense.device)
    mask = torch.empty((rows, K // 16), dtype=torch.uint8, device=dense.device)
    bad = torch.empty(1, dtype=torch.int32, device=dense.device)
    _check(lib().moesq_pack_pair_bitmask(_dev(dense, "dense", torch.uint8), rows, K, _dev(packed, "packed"),
                                         _dev(mask, "mask"), _dev(bad, "bad"), _stream()))
    return packed, mask, bad
