"""Plain FP64 CPU oracle of the paired-4:8 sparse NVFP4 (W4A4) MoE expert path.

TEST INFRASTRUCTURE ONLY. Nothing in the product (the ``sparse_quantized_moe_amd`` package, its HIP
library or its C ABI) may import, call or link this package; only ``tests/``, the smoke check and the
bench's CPU-baseline leg do. It shares no code, table or constant generator with the HIP library.

What it states, each function citing the passage it follows:

* ``nvfp4``      E2M1 / E4M3FN codecs and the per-32 NVFP4 quantizer (model cards, "Compression details").
* ``pairbitmask`` the pair-bitmask storage codec (model cards, "Sparse storage layout").
* ``compress``   synthetic weight compression: paired-4:8 magnitude prune, NVFP4, pack.
* ``moe``        the router (softmax top-k), the token->expert permutation, the grouped GEMM, the
                 load-time gate/up global fold and the MoE FFN with top-k combine.

Every value is computed in float64 from exact inputs; see each docstring for why that reaches the exact
decision where an integer (a code or a scale byte) is decided by a real-valued comparison.

Parity status: the codecs, the quantizer, the codec of the storage format, the prune, the permutation,
the grouped GEMM, the router and the gate/up fold are pinned by tests against textbook tables, a
library cast, exact-rational brute force, rank counts, closed forms, hand-derived fixtures and the
pages' storage figures. ``moe.moe_ffn`` is pinned against an exact evaluation written independently
of it (exact rationals, silu to 60 digits, nearest-value search over the format tables) on a small
layer whose down-input globals put quantization decisions next to rounding boundaries, and by
metamorphic relations (top-1 equals the single-expert FFN, token shuffles permute the rows, top-k is
the weighted sum of top-1 runs); ``moe.h_error_bound``, ``nvfp4.check_admissible`` and
``nvfp4.ambiguous_groups`` by fp32 accumulations in several orders, constructed boundary cases and
brute force. The pages print no worked FFN example.
"""
from . import nvfp4, pairbitmask, compress, moe  # noqa: F401
