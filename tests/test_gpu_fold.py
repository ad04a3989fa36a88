"""GPU gate/up global fold (moesq_fold_gate_up_globals) against the oracle's fold_gate_up_globals:
scale bytes and globals bit-exact, and the MoE FFN over the folded layer against the oracle FFN over
the oracle-folded layer."""
import numpy as np
import pytest
import torch

import sparse_quantized_moe_amd as moesq
import synth
from oracle import moe

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _random_w13(seed, E, N, K):
    rng = np.random.default_rng(seed)
    scale = rng.integers(0, 0x7F, size=(E, N, K // 32), dtype=np.uint8)
    scale[:, N // 2:][rng.random((E, N // 2, K // 32)) < 0.02] = 0xFF          # a few bytes that are not scales
    scale[:, N // 2:][rng.random((E, N // 2, K // 32)) < 0.02] = 0x7F
    gg = (10.0 ** rng.uniform(-4, 1, E)).astype(np.float32)
    kind = np.arange(E) % 4
    ratio = np.where(kind == 0, 10.0 ** rng.uniform(-3, 3, E),                  # saturation / underflow
                     np.where(kind == 1, 1.0, np.where(kind == 2, 2.0 ** rng.integers(-6, 6, E), 3.0)))
    gw = np.stack([gg, (gg * ratio).astype(np.float32)], axis=1)
    w = moesq.SparseWeights(torch.zeros((E, N, K // 4), dtype=torch.uint8, device=DEV),
                            torch.zeros((E, N, K // 16), dtype=torch.uint8, device=DEV),
                            torch.from_numpy(scale).to(DEV), torch.from_numpy(gw).to(DEV))
    return w, scale, gw


@pytest.mark.parametrize("E,N,K", [(3, 128, 256),        # 16-byte path, one slab per expert
                                   (7, 3072, 2048),      # 16-byte path, several slabs per expert
                                   (2, 6, 32),           # byte path (3 bytes per expert)
                                   (5, 80, 96)])         # byte path (120 bytes per expert)
def test_fold_matches_oracle_bit_exact(E, N, K):
    w, scale, gw = _random_w13(E * N + K, E, N, K)
    moesq.fold_gate_up_globals(w)
    got_s = w.scale.cpu().numpy()
    got_g = w.global_scale.cpu().numpy()
    for e in range(E):
        want_s, want_g = moe.fold_gate_up_globals(scale[e], gw[e])
        assert np.array_equal(got_s[e], want_s), e
        assert np.array_equal(got_g[e].view(np.uint32), want_g.view(np.uint32)), e
    # a second fold finds equal globals: nothing changes
    moesq.fold_gate_up_globals(w)
    assert np.array_equal(w.scale.cpu().numpy(), got_s)
    assert np.array_equal(w.global_scale.cpu().numpy(), got_g)


def test_fold_no_experts():
    w, _, _ = _random_w13(1, 1, 64, 256)
    assert moesq.lib().moesq_fold_gate_up_globals(None, None, 0, 64, 256, None) == 0
    before = w.scale.cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(w.scale.cpu().numpy(), before)


@pytest.mark.parametrize("T", [64, 512])                 # decode and prefill tactics
def test_ffn_over_folded_layer(T):
    from ffn_check import compare_ffn, oracle_layer
    E, H, I, k = 8, 512, 256, 4

    def dense_expert(e):
        return synth.expert_dense_weights(31, e, H, I, device=DEV)
    w13, w2 = moesq.compress_moe_layer(E, H, I, dense_expert, device=DEV)
    # spread the up globals away from the gate's so that the fold re-rounds most scales
    w13.global_scale[:, 1] *= torch.tensor([1.0, 1.37, 0.61, 2.9, 0.23, 1.0001, 5.5, 0.9], device=DEV)
    ow13, ow2 = oracle_layer(dense_expert, range(E))
    gw_before = w13.global_scale.cpu().numpy()
    for e in range(E):
        ow13[3][e] = gw_before[e].copy()
        ow13[2][e], ow13[3][e] = moe.fold_gate_up_globals(ow13[2][e], ow13[3][e])
    up_before = w13.scale[:, I:].cpu().numpy()
    moesq.fold_gate_up_globals(w13)
    for e in range(E):
        assert np.array_equal(w13.scale[e].cpu().numpy(), ow13[2][e])
    changed = (w13.scale[:, I:].cpu().numpy() != up_before).mean()
    assert changed > 0.5, changed                       # the fold is not a no-op on this layer
    w13t, w2t = moesq.prepare_weights(w13), moesq.prepare_weights(w2)
    x = synth.activations(32, T, H, device=DEV)
    ids, wts = synth.routing(33, T, E, k)
    g13 = synth.act_globals_from_x(x, ids, E)
    g2 = np.full(E, synth.ACT_GLOBAL_FIXED, np.float32)
    ws = torch.empty(moesq.lib().moesq_moe_ffn_workspace_size(T, H, I, k, E, 0), dtype=torch.uint8, device=DEV)
    out = moesq.moe_ffn(x, torch.from_numpy(ids).to(DEV), torch.from_numpy(wts).to(DEV), w13t, w2t,
                        torch.from_numpy(g13).to(DEV), torch.from_numpy(g2).to(DEV), workspace=ws)
    inter = {kk: v.cpu().numpy() for kk, v in moesq.ffn_intermediates(ws, T, H, I, k, E).items()}
    st = compare_ffn(x.float().cpu().numpy(), ids, wts, ow13, ow2, g13, g2, out.cpu().numpy(), inter)
    print("ffn over folded layer", T, st)
