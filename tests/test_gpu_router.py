"""GPU router (moesq_route_topk) against the oracle's route_topk: expert ids bit-exact, weights within
a bound derived from fp32 rounding."""
import numpy as np
import pytest
import torch

import sparse_quantized_moe_amd as moesq
from oracle import moe

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _check(logits_t, k, renormalize=True):
    ids, wts = moesq.route_topk(logits_t, k, renormalize)
    torch.cuda.synchronize()
    l = logits_t.float().cpu().numpy().astype(np.float64)        # the exact input values
    rid, rw = moe.route_topk(l, k, renormalize)
    assert np.array_equal(ids.cpu().numpy(), rid)
    # fp32 weights: exp of (logit - max) (one rounded difference, up to spread * 2^-24 in the
    # exponent), a sum of up to E positive terms, one division
    spread = (l.max(axis=1) - l.min(axis=1))[:, None]
    E = l.shape[1]
    terms = k if renormalize else E
    tol = (2 * spread + np.ceil(np.log2(terms)) + terms / 64 + 16) * 2.0 ** -24
    err = np.abs(wts.cpu().numpy() - rw) / rw
    assert (err <= tol).all(), float((err / tol).max())
    return ids, wts


@pytest.mark.parametrize("T,E,k,dtype", [(257, 128, 8, torch.float32), (64, 512, 10, torch.bfloat16),
                                         (1000, 384, 8, torch.bfloat16), (5, 1024, 64, torch.float32),
                                         (3, 1, 1, torch.float32), (130, 65, 7, torch.bfloat16)])
def test_route_topk_random(T, E, k, dtype):
    g = torch.Generator().manual_seed(T * 7 + E)
    logits = torch.randn((T, E), generator=g).to(dtype).to(DEV)
    _check(logits, k)


def test_route_topk_ties_pick_the_lower_id():
    g = torch.Generator().manual_seed(3)
    logits = torch.randint(-2, 3, (300, 100), generator=g).float().to(DEV)   # many equal logits
    ids, _ = _check(logits, 7)
    eq = torch.zeros((4, 70), device=DEV)                                      # all equal: ids 0..k-1
    ids_eq, w_eq = moesq.route_topk(eq, 5)
    assert ids_eq.cpu().tolist() == [[0, 1, 2, 3, 4]] * 4
    assert torch.allclose(w_eq.cpu(), torch.full((4, 5), 0.2), rtol=0, atol=1e-7)


def test_route_topk_without_renormalization_is_softmax():
    g = torch.Generator().manual_seed(4)
    logits = (3 * torch.randn((33, 33), generator=g)).to(DEV)
    ids, w = _check(logits, 33, renormalize=False)
    assert torch.allclose(w.sum(dim=1).cpu(), torch.ones(33), rtol=0, atol=1e-5)
    _check(logits, 4, renormalize=False)


def test_route_topk_feeds_the_permutation():
    """Router output straight into moesq_permute: the stable grouping the FFN runs on."""
    g = torch.Generator().manual_seed(5)
    logits = torch.randn((256, 128), generator=g).to(torch.bfloat16).to(DEV)
    ids, _ = moesq.route_topk(logits, 8)
    counts, offsets, sorted_p, inv, status = moesq.permute(ids, 128)
    rc, ro, rs, ri = moe.permute(ids.cpu().numpy(), 128)
    assert np.array_equal(offsets.cpu().numpy(), ro) and np.array_equal(inv.cpu().numpy(), ri)


def test_route_topk_no_tokens():
    ids, w = moesq.route_topk(torch.empty((0, 16), device=DEV), 2)
    assert ids.shape == (0, 2) and w.shape == (0, 2)
