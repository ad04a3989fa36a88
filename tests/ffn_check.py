"""Comparison of the HIP MoE FFN with the oracle, shared by the GPU tests, the smoke check and the bench.

Bit-exact: the permutation and the gate/up input codes/scales (exact inputs, exact decisions).
The down input (quantized h) may differ from the oracle only where the oracle's own decision lies
within the HIP path's fp32 error bound of a rounding boundary (both neighbours are correct results);
every such group must be one of the oracle's admissible encodings, and the number of such flips is
capped by the number of groups whose admissible set holds more than one encoding. Two output gates:

* teacher-forced: the oracle's output recomputed from the admissible encoding the GPU picked, compared
  row by row (max |y - yref| / max |yref| <= 1e-3 on every row);
* non-forced: the oracle's own output, compared tensor-normwise (max |y - yref| / max |yref| <= 1e-3
  over all compared rows), with the rows above 1e-3 row-normwise counted and each required to hold a
  flipped group.

Rows whose oracle output is exactly zero (every pair of the token dropped) must be exactly zero.
"""
from __future__ import annotations

import numpy as np

from oracle import compress, moe, nvfp4

TOL = 1e-3


def oracle_layer(dense_expert, experts):
    """Oracle's own compression of the dense weights of the given experts: (w13, w2) dicts-of-arrays."""
    w13 = [dict(), dict(), dict(), dict()]
    w2 = [dict(), dict(), dict(), dict()]
    for e in experts:
        g, u, d = (t.float().cpu().numpy() for t in dense_expert(e))
        cg, cu, cd = compress.compress(g), compress.compress(u), compress.compress(d)
        for i in range(3):
            w13[i][e] = np.concatenate([cg[i], cu[i]])
            w2[i][e] = cd[i]
        w13[3][e] = np.array([cg[3], cu[3]], np.float32)
        w2[3][e] = np.array([cd[3]], np.float32)
    return w13, w2


def gamma_for(K: int) -> float:
    # The sparse MFMA adds its products to the fp32 accumulator in groups of 8 kept products (16 dense
    # K), one rounding per group (measured on gfx950 with an accumulator of 1 and equal tiny products):
    # K/16 roundings along K, each at most one unit of the running sum, plus a margin for the
    # epilogue's global-scale products.
    return K / 16.0 + 16.0


def gather_gpu(gpu, tok, k):
    """The GPU intermediates of the pairs of tokens ``tok`` (in (token, j) order): gate/up input rows
    (pair order on the GPU) and down input rows (sorted order on the GPU, row inv[p])."""
    p = (np.asarray(tok)[:, None] * k + np.arange(k)[None, :]).ravel()
    rows = gpu["inv"][p]
    live = rows >= 0
    r = np.where(live, rows, 0)
    out = {"live": live, "a13_codes": gpu["a13_codes"][p], "a13_scales": gpu["a13_scales"][p],
           "a2_codes": gpu["a2_codes"][r], "a2_scales": gpu["a2_scales"][r]}
    return out


def compare_tokens(xs, ids_s, wts_s, ow13, ow2, g13, g2, y, gs):
    """Oracle against the GPU on one set of tokens: xs [n, H], their ids / weights [n, k], the GPU's
    output rows y [n, H] and its intermediates gs = gather_gpu(...) for these tokens. Checks everything
    that is decided per token (bit-exact gate/up input, admissible down input, teacher-forced rows,
    exact zero rows) and returns the figures the tensor-wide gates need."""
    xs = np.asarray(xs, np.float64)
    n, H = xs.shape
    k = ids_s.shape[1]
    out_ref, inter = moe.moe_ffn(xs, ids_s, wts_s, ow13, ow2, g13, g2, want=True)
    I = inter["h"].shape[1]
    p_sub = inter["sorted_pairs"]              # pair ids t * k + j of these tokens, oracle sorted order
    assert gs["live"][p_sub].all()
    assert np.array_equal(gs["a13_codes"][p_sub], inter["a13_codes"]), "gate/up input codes differ"
    assert np.array_equal(gs["a13_scales"][p_sub], inter["a13_scales"]), "gate/up input scales differ"
    a2c_gpu = gs["a2_codes"][p_sub]
    a2s_gpu = gs["a2_scales"][p_sub]
    same = (a2s_gpu == inter["a2_scales"]) & (
        nvfp4.unpack_codes(a2c_gpu).reshape(-1, I // 32, 32) ==
        nvfp4.unpack_codes(inter["a2_codes"]).reshape(-1, I // 32, 32)).all(axis=2)
    n_diff = int((~same).sum())
    out_own = out_ref
    n_amb = 0
    if n_diff:
        bound = moe.h_error_bound(xs, ids_s, ow13, g13, g2, gamma_for(H))
        ge = np.asarray(g2, np.float64)[ids_s.ravel()[p_sub]]
        ok = nvfp4.check_admissible(inter["h"], bound, ge, a2c_gpu, a2s_gpu)
        bad = (~same) & (~ok)
        assert not bad.any(), f"{int(bad.sum())} down-input groups are not an admissible encoding"
        n_amb = int(nvfp4.ambiguous_groups(inter["h"], bound, ge).sum())
        adopted_c = inter["a2_codes"].copy()
        adopted_s = inter["a2_scales"].copy()
        rows_d, grp_d = np.nonzero(~same)
        cu = nvfp4.unpack_codes(adopted_c)
        cg = nvfp4.unpack_codes(a2c_gpu)
        for r, gi in zip(rows_d, grp_d):
            cu[r, 32 * gi:32 * gi + 32] = cg[r, 32 * gi:32 * gi + 32]
            adopted_s[r, gi] = a2s_gpu[r, gi]
        adopted_c = (cu[:, 0::2] | (cu[:, 1::2] << 4)).astype(np.uint8)
        out_ref = moe.down_combine(adopted_c, adopted_s, g2, inter["offsets"], p_sub, wts_s, ow2, n, H)
    y = np.asarray(y, np.float64)
    den = np.abs(out_ref).max(axis=1)
    zero = den == 0
    assert (y[zero] == 0).all(), "rows with every pair dropped must be exactly zero"
    err = np.abs(y - out_ref).max(axis=1) / np.maximum(den, 1e-300)
    worst = float(err[~zero].max()) if (~zero).any() else 0.0
    assert worst <= TOL, f"row-normwise error {worst:.3e} > {TOL}"
    # non-forced: against the oracle's own encoding of h
    dev = np.abs(y - out_own)
    row_own = dev.max(axis=1) / np.maximum(np.abs(out_own).max(axis=1), 1e-300)
    hot = np.nonzero((row_own > TOL) & ~zero)[0]
    if len(hot):
        tok_flipped = set((p_sub[np.nonzero((~same).any(axis=1))[0]] // k).tolist())
        assert set(hot.tolist()) <= tok_flipped, "a row above 1e-3 (non-forced) without a flipped h group"
    return {"rows": int(n), "max_row_rel_err": worst, "nonforced_max_dev": float(dev.max()),
            "nonforced_max_ref": float(np.abs(out_own).max()), "nonforced_rows_above_tol": int(len(hot)),
            "admissible_flips": n_diff, "ambiguous_groups": n_amb, "groups": int(same.size)}


def finish(stats):
    """The tensor-wide gates over the per-token figures of compare_tokens (one dict or a list)."""
    if isinstance(stats, dict):
        stats = [stats]
    tot = {"rows": sum(s["rows"] for s in stats), "max_row_rel_err": max(s["max_row_rel_err"] for s in stats),
           "nonforced_rows_above_tol": sum(s["nonforced_rows_above_tol"] for s in stats),
           "admissible_flips": sum(s["admissible_flips"] for s in stats),
           "ambiguous_groups": sum(s["ambiguous_groups"] for s in stats), "groups": sum(s["groups"] for s in stats)}
    ref = max(s["nonforced_max_ref"] for s in stats)
    tot["nonforced_tensor_err"] = max(s["nonforced_max_dev"] for s in stats) / max(ref, 1e-300)
    assert tot["nonforced_tensor_err"] <= TOL, f"non-forced tensor-normwise error {tot['nonforced_tensor_err']:.3e} > {TOL}"
    # an unbiased fp32 error far inside its worst-case bound flips a small share of the groups that lie
    # within the bound of a boundary; a systematic shift of h would flip most of them
    assert tot["admissible_flips"] <= max(3, tot["ambiguous_groups"] // 2), \
        f"{tot['admissible_flips']} flipped groups of {tot['ambiguous_groups']} ambiguous ones"
    return tot


def compare_ffn(x, ids, wts, ow13, ow2, g13, g2, gpu_out, gpu, tokens=None, E=None):
    """Check the GPU FFN against the oracle on ``tokens`` (all if None). ``gpu`` holds numpy copies of
    the GPU intermediates (sorted, offsets, inv, a13_codes, a13_scales, a2_codes, a2_scales).
    Returns a stats dict; raises AssertionError on any mismatch."""
    x = np.asarray(x, np.float64)
    k = ids.shape[1]
    tok = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    st = compare_tokens(x[tok], ids[tok], wts[tok], ow13, ow2, g13, g2, np.asarray(gpu_out)[tok],
                        gather_gpu(gpu, tok, k))
    return finish(st)


def _compress_job(args):
    e, which, w = args
    return e, which, compress.compress(w)


def _compare_job(args):
    return compare_tokens(*args)


def compare_ffn_parallel(x, ids, wts, dense_expert, g13, g2, gpu_out, gpu, tokens, workers=16, chunk=2):
    """compare_ffn over many tokens with the oracle spread over worker processes (the oracle itself
    unchanged): the touched experts are compressed in parallel, then the tokens are checked in chunks
    of ``chunk``, each with only its experts' weights. dense_expert(e) -> (gate, up, down) tensors."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    x = np.asarray(x, np.float64)
    k = ids.shape[1]
    tok = np.asarray(tokens)
    experts = sorted(set(ids[tok].ravel().tolist()) - {-1})
    ctx = multiprocessing.get_context("spawn")
    w13 = [dict(), dict(), dict(), dict()]
    w2 = [dict(), dict(), dict(), dict()]
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        comp = {}
        for b0 in range(0, len(experts), workers):      # a bounded number of dense tensors in flight
            jobs = []
            for e in experts[b0:b0 + workers]:
                dense = [t.float().cpu().numpy() for t in dense_expert(e)]
                jobs += [(e, which, dense[which]) for which in range(3)]
            for e, which, c in ex.map(_compress_job, jobs):
                comp[(e, which)] = c
        for e in experts:
            cg, cu, cd = comp[(e, 0)], comp[(e, 1)], comp[(e, 2)]
            for i in range(3):
                w13[i][e] = np.concatenate([cg[i], cu[i]])
                w2[i][e] = cd[i]
            w13[3][e] = np.array([cg[3], cu[3]], np.float32)
            w2[3][e] = np.array([cd[3]], np.float32)
        y = np.asarray(gpu_out)
        args = []
        for c0 in range(0, len(tok), chunk):
            tc = tok[c0:c0 + chunk]
            ex_c = sorted(set(ids[tc].ravel().tolist()) - {-1})
            sub13 = [{e: w13[i][e] for e in ex_c} for i in range(4)]
            sub2 = [{e: w2[i][e] for e in ex_c} for i in range(4)]
            args.append((x[tc], ids[tc], wts[tc], sub13, sub2, g13, g2, y[tc], gather_gpu(gpu, tc, k)))
        stats = list(ex.map(_compare_job, args))
    return finish(stats)
