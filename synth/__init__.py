"""Seeded synthetic inputs for paired-4:8 sparse NVFP4 MoE layers.

This module is shared by the tests, the bench and the smoke check. It holds random draws and the
routing of the synthetic workloads only: no NVFP4 rounding, no pair pruning, no pair-bitmask packing
and no GEMM of the method. Both the CPU oracle and the HIP library receive what is drawn here as inputs.

Workloads (MoE shapes follow the model families on the MoESQ repository README, "Supported models"):

* ``linear``  one expert linear, M=16 tokens, N=256 outputs, K=512.
* ``qwen3_30b_decode``   128 experts, top-8, hidden 2048, moe_intermediate 768, T=256.
* ``qwen3_30b_prefill``  the same layer at T=8192 with Zipf(1.1)-skewed expert popularity.
* ``e512_decode`` / ``e512_prefill``  512 experts, top-10, hidden 4096, moe_intermediate 1024 at T=64 / 4096,
  activation global scale 1/(6*448) for every expert linear.
* ``kimi_k2_prefill``  384 experts, top-8, hidden 7168, moe_intermediate 2048, T=16384, Zipf(1.0)
  routing, 0.1 % activation outliers scaled by 50.

Weights are drawn dense fp32 ~ N(0, 0.02) per (expert, linear); the paired-4:8 prune, the NVFP4
quantization and the packing happen in the code under test (and independently in the oracle).
Every draw uses a seed derived from ``(seed, tag, indices...)`` so any part can be regenerated alone.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

__all__ = [
    "Workload", "WORKLOADS", "derive_seed", "torch_generator", "dense_weight", "expert_dense_weights",
    "activations", "routing", "act_globals_from_x", "down_global_from_dense", "random_act_codes",
    "random_sparse_weights", "VALID_NIBBLES", "ACT_GLOBAL_FIXED",
]

# Tags separating the independent random streams.
_TAG_WEIGHT, _TAG_ACT, _TAG_ROUTE, _TAG_OUTLIER, _TAG_RANDCODE, _TAG_RANDW = 11, 12, 13, 14, 15, 16

# Linear ids inside one expert: gate_proj, up_proj, down_proj.
GATE, UP, DOWN = 0, 1, 2

#: Activation global scale given as a constant (1/(6*448)) by the 512-expert workloads.
ACT_GLOBAL_FIXED = np.float32(1.0) / np.float32(2688.0)

#: The six 4-bit masks with exactly two bits set (a valid pair-bitmask nibble).
VALID_NIBBLES = np.array([0x3, 0x5, 0x6, 0x9, 0xA, 0xC], dtype=np.uint8)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    E: int                 # experts (1 for the single linear)
    k: int                 # top-k
    H: int                 # hidden (K of gate/up, N of down); for ``linear``: K
    I: int                 # moe_intermediate; for ``linear``: N
    T: int                 # tokens
    routing: str           # "softmax", "zipf" or "none"
    zipf_s: float = 0.0
    zipf_beta: float = 0.0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    fixed_act_global: bool = False

    @property
    def P(self) -> int:
        return self.T * self.k


WORKLOADS = {
    "linear": Workload("linear", E=1, k=1, H=512, I=256, T=16, routing="none"),
    "qwen3_30b_decode": Workload("qwen3_30b_decode", E=128, k=8, H=2048, I=768, T=256, routing="softmax"),
    "qwen3_30b_prefill": Workload("qwen3_30b_prefill", E=128, k=8, H=2048, I=768, T=8192, routing="zipf",
                                  zipf_s=1.1, zipf_beta=1.2),
    "e512_decode": Workload("e512_decode", E=512, k=10, H=4096, I=1024, T=64, routing="softmax",
                            fixed_act_global=True),
    "e512_prefill": Workload("e512_prefill", E=512, k=10, H=4096, I=1024, T=4096, routing="softmax",
                             fixed_act_global=True),
    "kimi_k2_prefill": Workload("kimi_k2_prefill", E=384, k=8, H=7168, I=2048, T=16384, routing="zipf",
                                zipf_s=1.0, zipf_beta=1.0, outlier_frac=0.001, outlier_scale=50.0),
}


def derive_seed(seed: int, *tags: int) -> int:
    """A 63-bit seed for the stream named by ``tags`` under ``seed`` (numpy SeedSequence)."""
    st = np.random.SeedSequence([int(seed), *[int(t) for t in tags]]).generate_state(2, np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def torch_generator(device, seed: int, *tags: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(seed, *tags))
    return g


def dense_weight(seed: int, expert: int, which: int, N: int, K: int, device="cpu") -> torch.Tensor:
    """Dense fp32 weight [N, K] ~ N(0, 0.02) of linear ``which`` (GATE/UP/DOWN) of ``expert``.

    The values depend on the device type (torch's CPU and GPU generators differ); a run that compares
    two implementations draws once and hands the same tensor to both.
    """
    g = torch_generator(device, seed, _TAG_WEIGHT, expert, which)
    return torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * 0.02


def expert_dense_weights(seed: int, expert: int, H: int, I: int, device="cpu"):
    """(gate [I,H], up [I,H], down [H,I]) dense fp32 weights of one expert."""
    return (dense_weight(seed, expert, GATE, I, H, device), dense_weight(seed, expert, UP, I, H, device),
            dense_weight(seed, expert, DOWN, H, I, device))


def activations(seed: int, T: int, H: int, device="cpu", outlier_frac: float = 0.0,
                outlier_scale: float = 1.0) -> torch.Tensor:
    """bf16 activations [T, H] ~ N(0, 1) (drawn in fp32, rounded to bf16 by torch's nearest-even cast).

    With ``outlier_frac`` > 0, round(frac*T*H) positions drawn without replacement are multiplied by
    ``outlier_scale`` in fp32 before the bf16 cast.
    """
    g = torch_generator(device, seed, _TAG_ACT)
    x = torch.randn((T, H), generator=g, device=device, dtype=torch.float32)
    n_out = int(round(outlier_frac * T * H))
    if n_out > 0:
        go = torch_generator(device, seed, _TAG_OUTLIER)
        pos = torch.randperm(T * H, generator=go, device=device)[:n_out]
        x.view(-1)[pos] *= outlier_scale
    return x.to(torch.bfloat16)


def routing(seed: int, T: int, E: int, k: int, kind: str = "softmax", zipf_s: float = 0.0,
            zipf_beta: float = 0.0):
    """Router output of a synthetic layer: (topk_ids int32 [T,k], topk_weights fp32 [T,k]).

    logits ~ N(0,1) [T,E] (fp64). For ``zipf``: logits += beta * (-s * ln rank_e), where the expert
    ranks are a seeded permutation of 1..E. Softmax in fp64, top-k (ties to the lower expert id),
    weights renormalised over the k picks and cast to fp32.
    """
    rng = np.random.Generator(np.random.PCG64(derive_seed(seed, _TAG_ROUTE)))
    logits = rng.standard_normal((T, E))
    if kind == "zipf":
        ranks = rng.permutation(E) + 1
        logits = logits + zipf_beta * (-zipf_s * np.log(ranks.astype(np.float64)))[None, :]
    elif kind != "softmax":
        raise ValueError(kind)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    pk = np.take_along_axis(p, order, axis=1)
    w = pk / pk.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def act_globals_from_x(x: torch.Tensor, topk_ids: np.ndarray, E: int) -> np.ndarray:
    """Per-expert input global scale of gate/up: fp32(amax of |x| over tokens routed to e) / 2688.

    A calibration of the static ``input_global_scale`` on the synthetic batch; experts that get no
    token take 1/2688.
    """
    amax_tok = x.float().abs().amax(dim=1).cpu().numpy().astype(np.float32)  # [T]
    out = np.full(E, ACT_GLOBAL_FIXED, dtype=np.float32)
    T, k = topk_ids.shape
    for e in np.unique(topk_ids[topk_ids >= 0]):
        rows = np.nonzero((topk_ids == e).any(axis=1))[0]
        out[e] = np.float32(amax_tok[rows].max()) / np.float32(2688.0)
    return out


def down_global_from_dense(x_rows: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
                           max_rows: int = 512) -> np.float32:
    """Input global scale of down_proj for one expert, calibrated on the *unquantized, unpruned* layer.

    fp32(amax |silu(x Wg^T) * (x Wu^T)|) / 2688 over at most ``max_rows`` routed rows (1/2688 if none).
    Plain torch fp32 arithmetic; it only picks a scalar input and is not the arithmetic under test.
    """
    if x_rows.shape[0] == 0:
        return ACT_GLOBAL_FIXED
    xr = x_rows[:max_rows].float()
    g = xr @ w_gate.float().t()
    u = xr @ w_up.float().t()
    h = torch.nn.functional.silu(g) * u
    amax = np.float32(h.abs().max().item())
    if amax == 0:
        return ACT_GLOBAL_FIXED
    return np.float32(amax) / np.float32(2688.0)


def random_act_codes(seed: int, rows: int, K: int):
    """Uniformly random NVFP4 activation bytes: codes u8 [rows, K/2] (any byte), scales u8 [rows, K/32]
    drawn from the finite non-negative E4M3 bytes 0x00..0x7E."""
    rng = np.random.Generator(np.random.PCG64(derive_seed(seed, _TAG_RANDCODE, rows, K)))
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales


def random_sparse_weights(seed: int, E: int, N: int, K: int, G: int = 1):
    """Uniformly random pair-bitmask weights: packed u8 [E,N,K/4] (any byte), mask u8 [E,N,K/16]
    (each nibble one of the six two-bit masks), scale u8 [E,N,K/32] in 0x00..0x7E, and fp32
    global scales [E,G] in [2^-12, 2^-8)."""
    rng = np.random.Generator(np.random.PCG64(derive_seed(seed, _TAG_RANDW, E, N, K)))
    packed = rng.integers(0, 256, size=(E, N, K // 4), dtype=np.uint8)
    nib = VALID_NIBBLES[rng.integers(0, 6, size=(E, N, K // 8))]
    mask = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    scale = rng.integers(0, 0x7F, size=(E, N, K // 32), dtype=np.uint8)
    gw = (2.0 ** rng.uniform(-12, -8, size=(E, G))).astype(np.float32)
    return packed, mask, scale, gw
