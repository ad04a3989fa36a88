#!/usr/bin/env python3
"""Throughput of the paired-4:8 sparse NVFP4 MoE FFN on one MI355X.

Headline: effective dense TFLOP/s (6*P*H*I per second of the whole moesq_moe_ffn call, P = live
(token, expert) pairs) of the largest single-GPU layer: 384 experts, top-8, hidden 7168,
moe_intermediate 2048, T=16384 tokens with Zipf(1.0)-skewed routing and 0.1 % activation outliers (one
GPU's full share of a Kimi-K2-shaped layer). Beside it: the weight-stream GB/s (stored sparse bytes of
the touched experts per second of the call) of the decode layers (128 experts at T=256, 512 experts at
T=64) and the effective dense TFLOP/s of the other prefill layers.

One step = one moesq_moe_ffn call (permute, quantize, gate/up GEMM + SiLU*up + quantize, down GEMM,
top-k combine) over one batch already resident in HBM. The 128-expert layer's weights (207.6 MB) fit
in the 256 MB last-level cache, so its decode steps rotate over several weight copies.

Output: one JSON line. ``roofline`` is the headline layer's dominant kernel (the gate/up GEMM; kept-half
multiply-adds against the dense f16 MFMA peak), timed with HIP events its own dispatch records;
every sub-object carries the rooflines of its GEMMs the same way. ``cpu_baseline`` times the CPU
oracle on a bounded token sample of the headline layer.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
DEFAULT_FLAGS = 0              # moe_ffn flags of the timed calls (0: the library's default path)
F16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 MFMA (the sparse MFMA doubles the dense-equivalent rate)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            if self.hip.hipEventCreate(ctypes.byref(arr, i * ctypes.sizeof(ctypes.c_void_p))) != 0:
                raise RuntimeError("hipEventCreate failed")
        return arr

    def record(self, e) -> None:
        import torch
        if self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, arr):
        for h in arr:
            self.hip.hipEventDestroy(h)


def build_layer(wl, seed, dev):
    import torch
    import sparse_quantized_moe_amd as moesq
    import synth

    def dense_expert(e):
        return synth.expert_dense_weights(seed, e, wl.H, wl.I, device=dev)
    t0 = time.time()
    w13, w2 = moesq.compress_moe_layer(wl.E, wl.H, wl.I, dense_expert, device=dev)
    # load-time re-tiling into the kernels' layout (the same bytes)
    w13, w2 = moesq.prepare_weights(w13), moesq.prepare_weights(w2)
    torch.cuda.synchronize()
    log(f"layer {wl.name}: compressed {wl.E} experts in {time.time() - t0:.1f}s "
        f"({(w13.nbytes() + w2.nbytes()) / 1e6:.1f} MB sparse storage)")
    return w13, w2, dense_expert


def batch(wl, seed, dev, dense_expert):
    import torch
    import synth
    x = synth.activations(seed, wl.T, wl.H, device=dev, outlier_frac=wl.outlier_frac, outlier_scale=wl.outlier_scale)
    ids, wts = synth.routing(seed, wl.T, wl.E, wl.k, wl.routing, wl.zipf_s, wl.zipf_beta)
    if wl.fixed_act_global:
        g13 = np.full(wl.E, synth.ACT_GLOBAL_FIXED, np.float32)
        g2 = g13.copy()
    else:
        g13 = synth.act_globals_from_x(x, ids, wl.E)
        g2 = np.full(wl.E, synth.ACT_GLOBAL_FIXED, np.float32)
        for e in np.unique(ids):
            rows = np.nonzero((ids == e).any(axis=1))[0]
            g, u, _ = dense_expert(int(e))
            g2[e] = synth.down_global_from_dense(x[torch.from_numpy(rows).to(dev)], g, u)
    return x, ids, wts, g13, g2


def touched_bytes(ids, E, H, I):
    """Stored sparse bytes of the experts with >= 1 row: 3*H*I*11/32 per expert + fp32 globals (3)."""
    n = len(np.unique(ids[ids >= 0]))
    per = (2 * I * H + H * I) * 11 // 32 + 4 * 3
    return n, n * per


def run_steps(moesq, torch, ev, x, ids_t, wts_t, layers, g13_t, g2_t, out, ws, warmup, steps, staged=False, flags=0):
    """Untimed warmup, then exactly ``steps`` timed calls bracketed by synchronizations.

    Returns (wall seconds, stage times [steps][2 * stages] in ms or None, GPU ms per step). Without
    ``staged`` the calls run back to back with HIP events only around the whole region; with it every
    call records events between its stages (on the library's stream), which adds a little time: the
    first ``stages`` columns are those intervals (launch gaps included), the next ``stages`` the
    stages' kernels alone, from the events their own dispatches record (on the one-launch path the
    single kernel is the first of these and the others are empty)."""
    nl = len(layers)
    ns = len(moesq.FFN_STAGES)
    for i in range(warmup):
        w13, w2 = layers[i % nl]
        moesq.moe_ffn(x, ids_t, wts_t, w13, w2, g13_t, g2_t, out=out, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    evs = [ev.create(3 * ns + 1) for _ in range(steps)] if staged else []
    region = ev.create(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(region[0])
    for i in range(steps):
        w13, w2 = layers[i % nl]
        if staged:
            moesq.set_stage_events(evs[i])
        moesq.moe_ffn(x, ids_t, wts_t, w13, w2, g13_t, g2_t, out=out, workspace=ws, flags=flags)
    ev.record(region[1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev.elapsed_ms(region[0], region[1]) / steps
    stages = None
    if staged:
        moesq.set_stage_events(None)
        stages = np.array([[ev.elapsed_ms(e[j], e[j + 1]) for j in range(ns)] +
                           [ev.elapsed_ms(e[ns + 1 + 2 * j], e[ns + 2 + 2 * j]) for j in range(ns)] for e in evs])
    for e in evs + [region]:
        ev.destroy(e)
    return wall, stages, gpu_ms


def graph_step_s(moesq, torch, x, ids_t, wts_t, layers, g13_t, g2_t, out, ws, reps):
    """Seconds per FFN call when one call per weight copy is captured into a HIP graph and the graph is
    replayed ``reps`` times back to back (host launch cost and most of the launch gaps go away)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for w13, w2 in layers:
            moesq.moe_ffn(x, ids_t, wts_t, w13, w2, g13_t, g2_t, out=out, workspace=ws, flags=DEFAULT_FLAGS)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for w13, w2 in layers:
            moesq.moe_ffn(x, ids_t, wts_t, w13, w2, g13_t, g2_t, out=out, workspace=ws, flags=DEFAULT_FLAGS)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / (reps * len(layers))
    del g
    return dt


def measured_peaks(moesq, torch, ev):
    """What this GPU sustains, beside the published peaks: a plain 1 GiB device copy (read + write
    bytes per second), the library's read-stream probe over the same 1 GiB (the ceiling of kernels
    that read much and write little, as the decode GEMMs do) and its probe of
    v_smfmac_f32_16x16x64_f16 (kept-half FLOP/s: 16384 per instruction), all timed with HIP events
    on the current stream."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    e = ev.create(2)
    for _ in range(2):
        dst.copy_(src)
    ev.record(e[0])
    for _ in range(5):
        dst.copy_(src)
    ev.record(e[1])
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 5 / (ev.elapsed_ms(e[0], e[1]) * 1e-3) / 1e9
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        moesq.probe_read(src, word)
    ev.record(e[0])
    for _ in range(5):
        moesq.probe_read(src, word)
    ev.record(e[1])
    torch.cuda.synchronize()
    read_gbs = n * 5 / (ev.elapsed_ms(e[0], e[1]) * 1e-3) / 1e9
    del src, dst
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    moesq.probe_smfmac(blocks, 64, sink)
    ev.record(e[0])
    insts = moesq.probe_smfmac(blocks, 1024, sink)
    ev.record(e[1])
    torch.cuda.synchronize()
    tf = insts * 16384 / (ev.elapsed_ms(e[0], e[1]) * 1e-3) / 1e12
    ev.destroy(e)
    return {"copy_GBps": round(copy_gbs, 1), "read_GBps": round(read_gbs, 1), "smfmac_f16_kept_TFLOPs": round(tf, 1)}


def router_figures(moesq, torch, ev, reps=50):
    """The router kernel that feeds the permutation (softmax top-k over bf16 logits), timed with HIP
    events over back-to-back calls at the decode and the largest prefill shape; bytes = logits in +
    ids and weights out."""
    res = {}
    for name, T, E, k in (("decode_T256_E128_k8", 256, 128, 8), ("prefill_T16384_E384_k8", 16384, 384, 8)):
        g = torch.Generator(device="cuda").manual_seed(T + E)
        logits = torch.randn((T, E), generator=g, device="cuda").to(torch.bfloat16)
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        for _ in range(3):
            moesq.route_topk(logits, k, out_ids=ids, out_weights=w)
        # the calls queue up behind a long matmul, so the GPU runs them back to back whatever the
        # host's launch rate (each call's time then includes the gap between dependent launches)
        a = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
        e = ev.create(2)
        torch.cuda.synchronize()
        _ = a @ a
        ev.record(e[0])
        for _ in range(reps):
            moesq.route_topk(logits, k, out_ids=ids, out_weights=w)
        ev.record(e[1])
        torch.cuda.synchronize()
        us = ev.elapsed_ms(e[0], e[1]) / reps * 1e3
        ev.destroy(e)
        del a
        nbytes = T * E * 2 + T * k * 8
        res[name] = {"us_per_call": round(us, 2), "tokens_per_s": round(T / (us * 1e-6), 0),
                     "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes": nbytes}
    return res


def fold_figures(moesq, torch, ev, reps=20):
    """The load-time gate/up global fold (in place on the up block scales), timed with HIP events over
    back-to-back calls at the decode layer and the largest layer; each call gets globals of its own,
    and the calls rotate over enough copies of the scales (>= 768 MB of up scales) that they are
    not served from the 256 MB last-level cache, as a fold at load time is not.
    bytes = the up scales read and written + the globals."""
    res = {}
    for name, E, H, I in (("E128_H2048_I768", 128, 2048, 768), ("E384_H7168_I2048", 384, 7168, 2048)):
        N, K = 2 * I, H
        up_bytes = E * I * (K // 32)
        copies = min(64, max(2, -(-768 * 2 ** 20 // up_bytes)))
        g = torch.Generator(device="cuda").manual_seed(E + H)
        scales = [torch.randint(0, 0x7F, (E, N, K // 32), generator=g, device="cuda", dtype=torch.uint8)
                  for _ in range(copies)]
        gw = torch.rand((reps + 3, E, 2), generator=g, device="cuda") + 0.5
        P = moesq.lib().moesq_fold_gate_up_globals
        stream = torch.cuda.current_stream().cuda_stream

        def call(i):
            st = P(scales[i % copies].data_ptr(), gw[i].data_ptr(), E, N, K, stream)
            if st != 0:
                raise RuntimeError(f"fold_gate_up_globals: status {st}")
        for i in range(3):
            call(reps + i)
        a = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
        e = ev.create(2)
        torch.cuda.synchronize()
        _ = a @ a
        ev.record(e[0])
        for i in range(reps):
            call(i)
        ev.record(e[1])
        torch.cuda.synchronize()
        us = ev.elapsed_ms(e[0], e[1]) / reps * 1e3
        ev.destroy(e)
        del a
        del scales
        nbytes = 2 * up_bytes + E * 2 * 4 * 2
        res[name] = {"us_per_call": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes": nbytes,
                     "copies_rotated": copies}
    return res


def side_passes(wl, P, route_ms, combine_ms):
    """The two HBM-bound passes around the GEMMs, from their kernels' own start/end events: routing
    (router ids in; x in, bf16; activation codes and scales out; sorted and inv out) and the top-k
    combine (the P fp32 down rows and inv in, the fp32 output out)."""
    rb = P * 4 + wl.T * wl.H * 2 + P * (wl.H // 2 + wl.H // 32) + 2 * P * 4
    cb = P * wl.H * 4 + P * 4 + wl.T * wl.H * 4
    return {"route": {"us": round(route_ms * 1e3, 2), "bytes": rb, "GBps": round(rb / (route_ms * 1e-3) / 1e9, 1)},
            "combine": {"us": round(combine_ms * 1e3, 2), "bytes": cb, "GBps": round(cb / (combine_ms * 1e-3) / 1e9, 1)}}


def cpu_baseline(wl, seed, x, ids, wts, g13, g2, dense_expert, max_experts, metric):
    """The oracle (unchanged) on a bounded sample of the workload: tokens drawn at random (seeded) as
    long as the experts they name stay within ``max_experts``; the oracle's compression of those
    experts runs first, untimed. metric "tflops": effective dense TFLOP/s (6 P H I per second over the
    sample's pairs); "gbps": stored bytes of the sample's experts per second."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    from oracle import compress, moe
    import threadpoolctl

    rng = np.random.default_rng(seed)
    toks, experts = [], set()
    for t in rng.permutation(wl.T):
        e_t = set(ids[t].tolist()) - {-1}
        if toks and len(experts | e_t) > max_experts:
            break
        toks.append(int(t))
        experts |= e_t
    toks = np.sort(np.array(toks))
    experts = sorted(experts)
    t0 = time.time()
    comp = {}
    with ProcessPoolExecutor(max_workers=min(16, os.cpu_count() or 1),
                             mp_context=multiprocessing.get_context("spawn")) as ex:
        for b0 in range(0, len(experts), 16):
            jobs = [(e, i) for e in experts[b0:b0 + 16] for i in range(3)]
            dense = {e: [t.cpu().numpy() for t in dense_expert(e)] for e in experts[b0:b0 + 16]}
            for (e, i), r in zip(jobs, ex.map(compress.compress, [dense[e][i] for e, i in jobs])):
                comp[(e, i)] = r
    log(f"cpu baseline: oracle compression of {len(experts)} experts (not timed) {time.time() - t0:.1f}s")
    w13 = [dict(), dict(), dict(), dict()]
    w2 = [dict(), dict(), dict(), dict()]
    for e in experts:
        cg, cu, cd = comp[(e, 0)], comp[(e, 1)], comp[(e, 2)]
        for i in range(3):
            w13[i][e] = np.concatenate([cg[i], cu[i]])
            w2[i][e] = cd[i]
        w13[3][e] = np.array([cg[3], cu[3]], np.float32)
        w2[3][e] = np.array([cd[3]], np.float32)
    xs = x.float().cpu().numpy()[toks]
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    moe.moe_ffn(xs, ids[toks], wts[toks], w13, w2, g13, g2)
    dt = time.perf_counter() - t0
    P = int((ids[toks] >= 0).sum())
    n, nbytes = touched_bytes(ids[toks], wl.E, wl.H, wl.I)
    if metric == "tflops":
        value, unit = 6.0 * P * wl.H * wl.I / dt / 1e12, "effective dense TFLOP/s"
    else:
        value, unit = nbytes / dt / 1e9, "GB/s"
    return {"value": round(value, 6), "unit": unit, "cores": int(threads), "kind": "oracle",
            "sample": f"{len(toks)} of {wl.T} tokens of {wl.name} ({P} pairs, {n} experts), {dt:.2f}s fp64 NumPy"}


def prefill_figure(moesq, torch, ev, wl, seed, dev, warmup, steps, peaks, layer=None):
    """One prefill layer: effective dense TFLOP/s of the whole call (6 P H I per second, P live
    pairs), each stage's kernel time, and the rooflines of the two GEMM kernels (kept-half
    multiply-adds, 2 P N K / 2 flops, against the dense f16 MFMA peak), from the kernels' own
    start/end events."""
    w13, w2, dense = layer if layer else build_layer(wl, seed, dev)
    x, ids, wts, g13, g2 = batch(wl, seed, dev, dense)
    ws = torch.empty(moesq.lib().moesq_moe_ffn_workspace_size(wl.T, wl.H, wl.I, wl.k, wl.E, 0), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)
    a = (moesq, torch, ev, x, torch.from_numpy(ids).to(dev), torch.from_numpy(wts).to(dev), [(w13, w2)],
         torch.from_numpy(g13).to(dev), torch.from_numpy(g2).to(dev), out, ws, warmup, steps)
    wall, _, gpu_ms = run_steps(*a)
    _, st, _ = run_steps(*a, staged=True)
    ns = len(moesq.FFN_STAGES)
    m = st.mean(axis=0)
    P = int((ids >= 0).sum())
    t = wall / steps
    eff = 6.0 * P * wl.H * wl.I / t / 1e12
    gu_ms, dn_ms = float(m[ns + 1]), float(m[ns + 2])
    gu_flops = 2.0 * P * (2 * wl.I) * wl.H / 2
    dn_flops = 2.0 * P * wl.H * wl.I / 2
    src = ("gemm.hip", "gemm_common.h", "moesq_device.h")

    def roof(kname, flops, ms, tname):
        ach = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": kname, "achieved": round(ach, 2), "peak": F16_DENSE_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / F16_DENSE_PEAK_TFLOPS, 4), "traffic": _traffic(tname, src),
                "algorithmic_flops_per_launch": flops, "avg_launch_ms": round(ms, 4),
                "measured_peak": peaks["smfmac_f16_kept_TFLOPs"],
                "frac_of_measured": round(ach / peaks["smfmac_f16_kept_TFLOPs"], 4)}
    res = {"workload": wl.name, "experts": wl.E, "top_k": wl.k, "hidden": wl.H, "moe_intermediate": wl.I,
           "tokens": wl.T, "pairs": P, "value": round(eff, 2), "unit": "effective dense TFLOP/s",
           "ms_per_step": round(t * 1e3, 4), "gpu_ms_per_step": round(gpu_ms, 4), "steps": steps,
           "stage_ms": {n: round(float(v), 4) for n, v in zip(moesq.FFN_STAGES, m)},
           "kernel_ms": {n: round(float(v), 4) for n, v in zip(moesq.FFN_STAGES, m[ns:])},
           "side_passes": side_passes(wl, P, float(m[ns]), float(m[ns + 3])),
           "roofline": roof("k_gemm_prefill<gate_up>", gu_flops, gu_ms, f"traffic_gemm_gate_up_{wl.name}.json"),
           "roofline_down": roof("k_gemm_prefill<down>", dn_flops, dn_ms, f"traffic_gemm_down_{wl.name}.json")}
    log(f"{wl.name}: {t * 1e3:.3f} ms/step, {eff:.1f} effective dense TFLOP/s; kernels (ms) "
        + ", ".join(f"{n}={v:.3f}" for n, v in zip(moesq.FFN_STAGES, m[ns:]))
        + f"; gate/up {res['roofline']['frac']:.3f}, down {res['roofline_down']['frac']:.3f} of the f16 peak")
    return res, (x, ids, wts, g13, g2, dense)


def decode_figure(moesq, torch, ev, wl, seed, dev, warmup, steps, copies, peaks):
    """One decode layer: weight-stream GB/s of the whole call (stored bytes of the touched experts per
    second), rotating ``copies`` weight copies so the stream does not come from the 256 MB last-level
    cache (when the layer is smaller than that), with the roofline of the gate/up kernel (its
    algorithmic bytes: touched W13 stored bytes + activation codes in + down-input codes out)."""
    w13, w2, dense = build_layer(wl, seed, dev)
    layers = [(w13, w2)]
    for _ in range(copies - 1):
        layers.append(tuple(moesq.SparseWeights(w.packed.clone(), None, None, w.global_scale.clone(), w.layout, w.shape)
                            for w in (w13, w2)))
    x, ids, wts, g13, g2 = batch(wl, seed, dev, dense)
    ids_t, wts_t = torch.from_numpy(ids).to(dev), torch.from_numpy(wts).to(dev)
    g13_t, g2_t = torch.from_numpy(g13).to(dev), torch.from_numpy(g2).to(dev)
    ws = torch.empty(moesq.lib().moesq_moe_ffn_workspace_size(wl.T, wl.H, wl.I, wl.k, wl.E, 0), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)
    a = (moesq, torch, ev, x, ids_t, wts_t, layers, g13_t, g2_t, out, ws, warmup, steps)
    wall, _, gpu_ms = run_steps(*a, flags=DEFAULT_FLAGS)
    _, stages, st_gpu = run_steps(*a, staged=True, flags=DEFAULT_FLAGS)
    ns = len(moesq.FFN_STAGES)
    m = stages.mean(axis=0)
    n_touched, wbytes = touched_bytes(ids, wl.E, wl.H, wl.I)
    t = wall / steps
    value = wbytes / t / 1e9
    P = int((ids >= 0).sum())
    fused = bool(moesq.ffn_layout(wl.T, wl.H, wl.I, wl.k, wl.E, DEFAULT_FLAGS)["fused"])
    alt = None
    if fused or moesq.ffn_layout(wl.T, wl.H, wl.I, wl.k, wl.E, moesq.FLAG_FUSED)["fused"]:
        alt_flags = moesq.FLAG_UNFUSED if fused else moesq.FLAG_FUSED
        wall_a, _, _ = run_steps(*a, flags=alt_flags)
        alt = {"path": "separate launches" if fused else "one fused launch",
               "us_per_step": round(wall_a / steps * 1e6, 2), "GBps": round(wbytes / (wall_a / steps) / 1e9, 2)}
    wall_w, _, _ = run_steps(moesq, torch, ev, x, ids_t, wts_t, layers[:1], g13_t, g2_t, out, ws, warmup, steps,
                             flags=DEFAULT_FLAGS)
    t_graph = graph_step_s(moesq, torch, x, ids_t, wts_t, layers, g13_t, g2_t, out, ws, max(1, steps // len(layers)))
    warm = wbytes / (wall_w / steps) / 1e9
    kbytes = n_touched * (2 * wl.I * wl.H * 11 // 32 + 8) + P * (wl.H // 2 + wl.H // 32) + P * (wl.I // 2 + wl.I // 32)
    k_ms = float(m[ns + 1])
    achieved = kbytes / (k_ms * 1e-3) / 1e9
    dbytes = n_touched * (wl.H * wl.I * 11 // 32 + 4) + P * (wl.I // 2 + wl.I // 32) + P * wl.H * 4
    d_ms = float(m[ns + 2])
    src = ("gemm.hip", "gemm_common.h", "moesq_device.h")
    # the library's decode kernels: the whole K staged once for gate/up up to K = 2048 and for the
    # other linears up to K = 1024, else 512-K chunks
    gu_kernel = "k_gemm_decode_stream<gate_up>" if wl.H <= 2048 else "k_gemm_decode<gate_up>"
    dn_kernel = "k_gemm_decode_nloop<down>" if wl.I <= 1024 else "k_gemm_decode<down>"
    res = {"workload": wl.name, "experts": wl.E, "top_k": wl.k, "hidden": wl.H, "moe_intermediate": wl.I,
           "tokens": wl.T, "value": round(value, 2), "unit": "weight-stream GB/s", "us_per_step": round(t * 1e6, 2),
           "gpu_us_per_step": round(gpu_ms * 1e3, 2), "experts_touched": n_touched, "stored_bytes_streamed": wbytes,
           "weight_copies_rotated": copies, "warm_cache_GBps": round(warm, 2), "fused_launch": fused,
           "graph_replay": {"us_per_step": round(t_graph * 1e6, 2), "GBps": round(wbytes / t_graph / 1e9, 2),
                            "note": "one call per weight copy captured in one HIP graph, replayed back to back"},
           "stage_us": {n: round(float(v) * 1e3, 2) for n, v in zip(moesq.FFN_STAGES, m)},
           "kernel_us": {n: round(float(v) * 1e3, 2) for n, v in zip(moesq.FFN_STAGES, m[ns:])},
           "other_path": alt,
           "side_passes": side_passes(wl, P, float(m[ns]), float(m[ns + 3])),
           "roofline": {"bound": "hbm", "kernel": gu_kernel, "achieved": round(achieved, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": _traffic(f"traffic_gemm_gate_up_{wl.name}.json", src),
                        "algorithmic_bytes_per_launch": kbytes, "avg_launch_us": round(k_ms * 1e3, 2),
                        "measured_peak": peaks["read_GBps"], "measured_peak_kind": "read stream (library probe)",
                        "frac_of_measured": round(achieved / peaks["read_GBps"], 4)},
           "roofline_down": {"bound": "hbm", "kernel": dn_kernel,
                             "achieved": round(dbytes / (d_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(dbytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "traffic": _traffic(f"traffic_gemm_down_{wl.name}.json", src),
                             "algorithmic_bytes_per_launch": dbytes, "avg_launch_us": round(d_ms * 1e3, 2)}}
    log(f"{wl.name}: {t * 1e6:.1f} us/step ({t_graph * 1e6:.1f} as graph replay), {value:.1f} GB/s (warm {warm:.1f}); kernels (us) "
        + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in zip(moesq.FFN_STAGES, m[ns:]))
        + f"; gate/up {res['roofline']['frac']:.3f} of 8 TB/s")
    del layers
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="kimi_k2_prefill",
                    help="the headline layer (the largest single-GPU configuration)")
    ap.add_argument("--decode-workloads", default="qwen3_30b_decode,e512_decode",
                    help="decode layers reported beside the headline ('' for none)")
    ap.add_argument("--prefill-workloads", default="qwen3_30b_prefill,e512_prefill",
                    help="other prefill layers reported beside the headline ('' for none)")
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated at decode (cache-cold stream)")
    ap.add_argument("--cpu-experts", type=int, default=32,
                    help="experts the oracle baseline's token sample may name (about 15-20 s of fp64 NumPy at 384 "
                         "experts, hidden 7168; the per-expert dequantization dominates)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the router, fold and measured-peak figures")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run 3 plain device copies of MIB MiB (a known-size kernel for scaling HBM "
                         "byte counters under rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs the expert path on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_quantized_moe_amd as moesq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ev = HipEvents()
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {n} bytes")
        del src, dst
    if args.no_extras:
        peaks = {"copy_GBps": None, "read_GBps": None, "smfmac_f16_kept_TFLOPs": None}
    else:
        peaks = measured_peaks(moesq, torch, ev)
        log(f"measured: device copy {peaks['copy_GBps']} GB/s, read stream {peaks['read_GBps']} GB/s, "
            f"smfmac f16 {peaks['smfmac_f16_kept_TFLOPs']} TFLOP/s (kept half)")
    if peaks["smfmac_f16_kept_TFLOPs"] is None:
        peaks = {"copy_GBps": 1.0, "read_GBps": 1.0, "smfmac_f16_kept_TFLOPs": 1.0}
    wl = synth.WORKLOADS[args.workload]
    decode_head = wl.T * wl.k <= 48 * wl.E
    if decode_head:
        head = decode_figure(moesq, torch, ev, wl, args.seed, dev, args.warmup, args.steps, args.copies, peaks)
        layer = build_layer(wl, args.seed, dev) if not args.no_cpu_baseline else None
        hx = batch(wl, args.seed, dev, layer[2]) if layer else None
    else:
        layer = build_layer(wl, args.seed, dev)
        head, hx = prefill_figure(moesq, torch, ev, wl, args.seed, dev, args.warmup, args.steps, peaks, layer)
        hx = hx[:5]
    result = {
        "metric": "MoE FFN effective dense TFLOP/s (prefill) + weight-stream GB/s (decode), 1 GPU",
        "value": head["value"], "unit": "GB/s" if decode_head else "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3 if decode_head else head["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 w4a4 (f16 sparse MFMA, fp32 accumulate)", "data": "synthetic (seeded; random-init weights)",
        "config": {k: v for k, v in head.items() if k not in ("value", "unit", "roofline")},
        "roofline": head["roofline"],
        "measured_peaks": None if args.no_extras else peaks,
    }
    if not args.no_cpu_baseline:
        w = layer[2]
        x, ids, wts, g13, g2 = hx
        result["cpu_baseline"] = cpu_baseline(wl, args.seed, x, ids, wts, g13, g2, w, args.cpu_experts,
                                              "gbps" if decode_head else "tflops")
    else:
        result["cpu_baseline"] = None
    del layer, hx
    torch.cuda.empty_cache()
    result["decode"] = {}
    for name in [n for n in args.decode_workloads.split(",") if n]:
        result["decode"][name] = decode_figure(moesq, torch, ev, synth.WORKLOADS[name], args.seed, dev, args.warmup,
                                               max(args.steps, 20), args.copies, peaks)
        torch.cuda.empty_cache()
    result["prefill"] = {}
    for name in [n for n in args.prefill_workloads.split(",") if n]:
        result["prefill"][name] = prefill_figure(moesq, torch, ev, synth.WORKLOADS[name], args.seed, dev, args.warmup,
                                                 args.steps, peaks)[0]
        torch.cuda.empty_cache()
    if not args.no_extras:
        result["router"] = router_figures(moesq, torch, ev)
        result["fold_gate_up"] = fold_figures(moesq, torch, ev)
    print(json.dumps(result), flush=True)


def _traffic(name, sources):
    """HBM bytes per launch from a committed counter summary in profiles/, or None when there is none
    or the kernel code has changed since the counters were taken."""
    tfile = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(tfile):
        return None
    t = json.load(open(tfile))
    return t.get("bytes_per_launch") if t.get("kernel_source_sha") == _kernel_sha(sources) else None


def _kernel_sha(files) -> str:
    """Hash of the kernel sources' code: comments and whitespace runs are dropped first, so an edit
    of the comments alone keeps a traffic figure taken on the same code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        text = open(os.path.join(ROOT, "sparse_quantized_moe_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
