"""The allocation-free FFN entry point (moesq_moe_ffn_noalloc, workspace in the library's static device
scratch) against moesq_moe_ffn with a caller workspace, through the C ABI: bit-identical outputs on two
calls in a row, the second on a smaller batch (the scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

moesq = pytest.importorskip("sparse_quantized_moe_amd")
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    _need_gpu()
    E, H, I, k = 128, 2048, 768, 8
    dense = {e: synth.expert_dense_weights(0, e, H, I, device=DEV) for e in range(E)}
    w13, w2 = moesq.compress_moe_layer(E, H, I, lambda e: dense[e], device=DEV)
    w13, w2 = moesq.prepare_weights(w13), moesq.prepare_weights(w2)
    for T, seed in ((256, 0), (40, 1)):                  # the second call: a smaller batch
        x = synth.activations(seed, T, H, device=DEV)
        ids, wts = synth.routing(seed, T, E, k)
        ids[3, 2] = -1                                   # a dropped pair
        g13 = torch.from_numpy(synth.act_globals_from_x(x, ids, E)).to(DEV)
        g2 = torch.full((E,), float(synth.ACT_GLOBAL_FIXED) * 64, dtype=torch.float32, device=DEV)
        ids_t, wts_t = torch.from_numpy(ids).to(DEV), torch.from_numpy(wts).to(DEV)
        out = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
        moesq.moe_ffn_noalloc(x, ids_t, wts_t, w13, w2, g13, g2, out=out, flags=moesq.FLAG_SYNC_CHECK)
        ref = moesq.moe_ffn(x, ids_t, wts_t, w13, w2, g13, g2, flags=moesq.FLAG_SYNC_CHECK | moesq.FLAG_UNFUSED)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), T
        assert torch.isfinite(out).all() and out.abs().max() > 0
