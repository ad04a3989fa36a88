#!/usr/bin/env python3
"""Throughput of the paired-4:8 sparse NVFP4 MoE FFN on one MI355X.

Metric: weight-stream GB/s at decode (stored sparse bytes of the experts a batch touches, per second
of the whole moesq_moe_ffn call) on the 128-expert, top-8, hidden-2048, moe_intermediate-768 layer at
T=256 tokens, and effective dense TFLOP/s (6*P*H*I per second, P = T*k) of the same layer at
prefill, T=8192 with Zipf(1.1)-skewed routing.

One step = one moesq_moe_ffn call (permute, quantize, gate/up GEMM + SiLU*up + quantize, down GEMM,
top-k combine) over one batch already resident in HBM. The layer's weights (207.6 MB) fit in the
256 MB Infinity Cache, so decode steps rotate over several copies of the weights (a cold-cache
stream, the reported value) and the warm single-copy figure is reported beside it.

Output: one JSON line (rank 0). ``roofline`` is for the dominant kernel (at decode the one-launch
FFN kernel, else the gate/up GEMM), timed with HIP events recorded by the library on its own stream;
``cpu_baseline`` times the CPU oracle on a bounded sample of the same decode workload.
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


def other_workloads(moesq, torch, ev, seed, dev, names=("e512_decode", "e512_prefill", "kimi_k2_prefill")):
    """The other layer shapes, each timed on its own batch like the headline ones (no weight-copy
    rotation: their touched weights are far larger than the 256 MB last-level cache): decode rows give
    the weight-stream GB/s on the stored bytes of the touched experts, prefill rows the effective dense
    TFLOP/s; both with each stage's kernel time."""
    import synth
    res = {}
    for name in names:
        wl = synth.WORKLOADS[name]
        w13, w2, dense = build_layer(wl, seed, dev)
        x, ids, wts, g13, g2 = batch(wl, seed, dev, dense)
        ws = torch.empty(moesq.lib().moesq_moe_ffn_workspace_size(wl.T, wl.H, wl.I, wl.k, wl.E, 0),
                         dtype=torch.uint8, device=dev)
        out = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)
        decode = wl.T * wl.k <= 48 * wl.E
        steps = 20 if decode else 5
        a = (moesq, torch, ev, x, torch.from_numpy(ids).to(dev), torch.from_numpy(wts).to(dev), [(w13, w2)],
             torch.from_numpy(g13).to(dev), torch.from_numpy(g2).to(dev), out, ws, 2, steps)
        wall, _, _ = run_steps(*a)
        _, st, _ = run_steps(*a, staged=True)
        t = wall / steps
        ns = len(moesq.FFN_STAGES)
        r = {"tokens": wl.T, "experts": wl.E, "top_k": wl.k, "hidden": wl.H, "moe_intermediate": wl.I,
             "us_per_step": round(t * 1e6, 2),
             "kernel_us": {n: round(float(v) * 1e3, 2) for n, v in zip(moesq.FFN_STAGES, st.mean(axis=0)[ns:])}}
        if decode:
            n, wb = touched_bytes(ids, wl.E, wl.H, wl.I)
            r.update({"metric": "weight-stream GB/s", "value": round(wb / t / 1e9, 2), "experts_touched": n,
                      "stored_bytes_streamed": wb})
        else:
            P = int((ids >= 0).sum())
            r.update({"metric": "effective dense TFLOP/s", "value": round(6.0 * P * wl.H * wl.I / t / 1e12, 2)})
        log(f"{name}: {r['value']} {r['metric']}, {r['us_per_step']} us/step")
        res[name] = r
        del w13, w2, ws, out, x
        torch.cuda.empty_cache()
    return res


def side_passes(wl, P, route_ms, combine_ms):
    """The two HBM-bound passes around the GEMMs, from their kernels' own start/end events: routing
    (router ids in; x in, bf16; activation codes and scales out; sorted and inv out) and the top-k
    combine (the P fp32 down rows and inv in, the fp32 output out)."""
    rb = P * 4 + wl.T * wl.H * 2 + P * (wl.H // 2 + wl.H // 32) + 2 * P * 4
    cb = P * wl.H * 4 + P * 4 + wl.T * wl.H * 4
    return {"route": {"us": round(route_ms * 1e3, 2), "bytes": rb, "GBps": round(rb / (route_ms * 1e-3) / 1e9, 1)},
            "combine": {"us": round(combine_ms * 1e3, 2), "bytes": cb, "GBps": round(cb / (combine_ms * 1e-3) / 1e9, 1)}}


def cpu_baseline(wl, seed, x, ids, wts, g13, g2, dense_expert, ntok):
    """The oracle (unchanged) on a bounded sample of the decode batch: ntok tokens and their experts."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    from oracle import compress, moe
    import threadpoolctl

    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(wl.T, ntok, replace=False))
    experts = sorted(set(ids[toks].ravel().tolist()) - {-1})
    dense = {e: [t.cpu().numpy() for t in dense_expert(e)] for e in experts}
    t0 = time.time()
    jobs = [(e, i) for e in experts for i in range(3)]
    with ProcessPoolExecutor(max_workers=min(16, os.cpu_count() or 1),
                             mp_context=multiprocessing.get_context("spawn")) as ex:
        res = list(ex.map(compress.compress, [dense[e][i] for e, i in jobs]))
    log(f"cpu baseline: oracle compression of {len(experts)} experts (not timed) {time.time() - t0:.1f}s")
    by = {(e, i): r for (e, i), r in zip(jobs, res)}
    w13 = [dict(), dict(), dict(), dict()]
    w2 = [dict(), dict(), dict(), dict()]
    for e in experts:
        cg, cu, cd = by[(e, 0)], by[(e, 1)], by[(e, 2)]
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
    n, nbytes = touched_bytes(ids[toks], wl.E, wl.H, wl.I)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{ntok} of {wl.T} tokens of {wl.name} ({n} experts, {nbytes / 1e6:.1f} MB stored), "
                      f"{dt:.2f}s fp64 NumPy"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_30b_decode")
    ap.add_argument("--prefill-workload", default="qwen3_30b_prefill", help="'' to skip the prefill figure")
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated at decode (cache-cold stream)")
    ap.add_argument("--cpu-tokens", type=int, default=64,
                    help="tokens of the decode batch the oracle baseline runs on (about 6-7 s of CPU work: nearly "
                         "every expert is touched, and the per-expert dequantization dominates)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the 512-expert and 384-expert layers (timed after the headline ones)")
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
    peaks = measured_peaks(moesq, torch, ev)
    log(f"measured: device copy {peaks['copy_GBps']} GB/s, read stream {peaks['read_GBps']} GB/s, smfmac f16 {peaks['smfmac_f16_kept_TFLOPs']} TFLOP/s (kept half)")
    wl = synth.WORKLOADS[args.workload]
    w13, w2, dense_expert = build_layer(wl, args.seed, dev)
    layers = [(w13, w2)]
    for _ in range(args.copies - 1):
        layers.append(tuple(moesq.SparseWeights(w.packed.clone(), None, None, w.global_scale.clone(), w.layout, w.shape)
                            for w in (w13, w2)))
    x, ids, wts, g13, g2 = batch(wl, args.seed, dev, dense_expert)
    ids_t, wts_t = torch.from_numpy(ids).to(dev), torch.from_numpy(wts).to(dev)
    g13_t, g2_t = torch.from_numpy(g13).to(dev), torch.from_numpy(g2).to(dev)
    ws = torch.empty(moesq.lib().moesq_moe_ffn_workspace_size(wl.T, wl.H, wl.I, wl.k, wl.E, 0), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.float32, device=dev)

    wall, _, gpu_ms = run_steps(moesq, torch, ev, x, ids_t, wts_t, layers, g13_t, g2_t, out, ws,
                                args.warmup, args.steps, flags=DEFAULT_FLAGS)
    ms = wall / args.steps * 1e3
    n_touched, wbytes = touched_bytes(ids, wl.E, wl.H, wl.I)
    value = wbytes / (wall / args.steps) / 1e9
    log(f"decode: {ms * 1e3:.1f} us/step wall, {gpu_ms * 1e3:.1f} us/step GPU events, {value:.1f} GB/s")
    fused = bool(moesq.ffn_layout(wl.T, wl.H, wl.I, wl.k, wl.E, DEFAULT_FLAGS)["fused"])
    # stage breakdown (events between the stages of every call), same rotation of weight copies; the
    # one-launch path records all its stages around its single kernel
    _, stages, st_gpu = run_steps(moesq, torch, ev, x, ids_t, wts_t, layers, g13_t, g2_t, out, ws,
                                  args.warmup, args.steps, staged=True, flags=DEFAULT_FLAGS)
    st_mean = stages.mean(axis=0)
    log("decode stage us (mean): " + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in zip(moesq.FFN_STAGES, st_mean))
        + f"; {st_gpu * 1e3:.1f} us/step with stage events" + (" (one fused launch: all in the first)" if fused else "")
        + "; kernels alone " + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in zip(moesq.FFN_STAGES, st_mean[len(moesq.FFN_STAGES):])))
    # the other path on the same batch, for comparison (separate launches vs the one-launch kernel)
    alt = None
    alt_flags = moesq.FLAG_UNFUSED if fused else moesq.FLAG_FUSED
    if fused or moesq.ffn_layout(wl.T, wl.H, wl.I, wl.k, wl.E, moesq.FLAG_FUSED)["fused"]:
        wall_a, _, _ = run_steps(moesq, torch, ev, x, ids_t, wts_t, layers, g13_t, g2_t, out, ws,
                                 args.warmup, args.steps, flags=alt_flags)
        _, st_a, _ = run_steps(moesq, torch, ev, x, ids_t, wts_t, layers, g13_t, g2_t, out, ws,
                               args.warmup, args.steps, staged=True, flags=alt_flags)
        alt = {"path": "separate launches" if fused else "one fused launch",
               "us_per_step": round(wall_a / args.steps * 1e6, 2),
               "GBps": round(wbytes / (wall_a / args.steps) / 1e9, 2),
               "stage_us": {n: round(float(v) * 1e3, 2) for n, v in zip(moesq.FFN_STAGES, st_a.mean(axis=0))}}
        log(f"decode, {alt['path']}: {alt['us_per_step']} us/step; stages {alt['stage_us']}")
    # warm (single copy) figure
    wall_w, _, _ = run_steps(moesq, torch, ev, x, ids_t, wts_t, layers[:1], g13_t, g2_t, out, ws,
                             args.warmup, args.steps, flags=DEFAULT_FLAGS)
    warm = wbytes / (wall_w / args.steps) / 1e9
    P = int((ids >= 0).sum())
    if fused:
        # dominant (only) kernel: the fused FFN; algorithmic bytes = stored weight bytes of the touched
        # experts + the tokens in (bf16) + router ids and weights + the output (fp32)
        kname = "k_ffn_fused (route, gate/up, down, combine in one launch)"
        kbytes = wbytes + wl.T * wl.H * 2 + P * 8 + wl.T * wl.H * 4
        k_ms = float(st_mean[len(moesq.FFN_STAGES)])       # the one kernel, its own start/end events
        tname, tsrc = "traffic_ffn_fused_qwen3_30b_decode.json", ("ffn_fused.hip", "gemm_common.h", "moesq_device.h")
    else:
        # dominant kernel: gate/up GEMM; algorithmic bytes = W13 stored bytes of touched experts + its
        # activation input (codes + scales) + its output (down-input codes + scales)
        kname = "k_gemm_decode_stream<gate_up>"
        kbytes = n_touched * (2 * wl.I * wl.H * 11 // 32 + 8) + P * (wl.H // 2 + wl.H // 32) + P * (wl.I // 2 + wl.I // 32)
        k_ms = float(st_mean[len(moesq.FFN_STAGES) + 1])   # the gate/up kernel, its own start/end events
        tname, tsrc = "traffic_gemm_gate_up_qwen3_30b_decode.json", ("gemm.hip", "gemm_common.h", "moesq_device.h")
    achieved = kbytes / (k_ms * 1e-3) / 1e9
    traffic = _traffic(tname, tsrc)
    result = {
        "metric": "MoE FFN effective dense TFLOP/s (prefill) + weight-stream GB/s (decode), 1 GPU",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 w4a4 (f16 sparse MFMA, fp32 accumulate)", "data": "synthetic (seeded; random-init weights)",
        "config": {"workload": wl.name, "experts": wl.E, "top_k": wl.k, "hidden": wl.H, "moe_intermediate": wl.I,
                   "tokens": wl.T, "experts_touched": n_touched, "stored_bytes_streamed": wbytes,
                   "weight_copies_rotated": args.copies, "warm_cache_GBps": round(warm, 2),
                   "gpu_us_per_step": round(gpu_ms * 1e3, 2), "fused_launch": fused,
                   "stage_us": {n: round(float(v) * 1e3, 2) for n, v in zip(moesq.FFN_STAGES, st_mean)},
                   "kernel_us": {n: round(float(v) * 1e3, 2) for n, v in zip(moesq.FFN_STAGES, st_mean[len(moesq.FFN_STAGES):])},
                   "other_path": alt},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": kbytes,
                     "avg_launch_us": round(k_ms * 1e3, 2),
                     "measured_peak": peaks["read_GBps"], "measured_peak_kind": "read stream (library probe)",
                     "frac_of_measured": round(achieved / peaks["read_GBps"], 4)},
        "measured_peaks": peaks,
        "side_passes": None if fused else side_passes(wl, P, float(st_mean[len(moesq.FFN_STAGES)]),
                                                      float(st_mean[len(moesq.FFN_STAGES) + 3])),
        "router": router_figures(moesq, torch, ev),
        "fold_gate_up": fold_figures(moesq, torch, ev),
    }
    del layers[1:]
    torch.cuda.empty_cache()

    if args.prefill_workload:
        pw = synth.WORKLOADS[args.prefill_workload]
        if (pw.E, pw.H, pw.I) != (wl.E, wl.H, wl.I):
            w13, w2, dense_expert = build_layer(pw, args.seed, dev)
        px, pids, pwts, pg13, pg2 = batch(pw, args.seed, dev, dense_expert)
        pws = torch.empty(moesq.lib().moesq_moe_ffn_workspace_size(pw.T, pw.H, pw.I, pw.k, pw.E, 0),
                          dtype=torch.uint8, device=dev)
        pout = torch.empty((pw.T, pw.H), dtype=torch.float32, device=dev)
        psteps = max(3, min(args.steps, 20))
        pargs = (moesq, torch, ev, px, torch.from_numpy(pids).to(dev), torch.from_numpy(pwts).to(dev), [(w13, w2)],
                 torch.from_numpy(pg13).to(dev), torch.from_numpy(pg2).to(dev), pout, pws, min(args.warmup, 3), psteps)
        pwall, _, _ = run_steps(*pargs)
        _, pst, _ = run_steps(*pargs, staged=True)
        PP = int((pids >= 0).sum())
        eff = 6.0 * PP * pw.H * pw.I / (pwall / psteps) / 1e12
        pst_mean = pst.mean(axis=0)
        g_ms = float(pst_mean[len(moesq.FFN_STAGES) + 1])  # the gate/up kernel, its own start/end events
        alg_flops = 2.0 * PP * (2 * pw.I) * pw.H / 2          # multiply-adds on the kept half of W13
        ach = alg_flops / (g_ms * 1e-3) / 1e12
        log("prefill stage ms (mean): " + ", ".join(f"{n}={v:.3f}ms" for n, v in zip(moesq.FFN_STAGES, pst_mean))
            + "; kernels alone " + ", ".join(f"{n}={v:.3f}ms" for n, v in zip(moesq.FFN_STAGES, pst_mean[len(moesq.FFN_STAGES):])))
        log(f"prefill: {pwall / psteps * 1e3:.3f} ms/step, {eff:.1f} effective dense TFLOP/s")
        result["prefill"] = {
            "workload": pw.name, "tokens": pw.T, "value": round(eff, 2), "unit": "effective dense TFLOP/s",
            "ms_per_step": round(pwall / psteps * 1e3, 4), "steps": psteps,
            "stage_ms": {n: round(float(v), 4) for n, v in zip(moesq.FFN_STAGES, pst_mean)},
            "kernel_ms": {n: round(float(v), 4) for n, v in zip(moesq.FFN_STAGES, pst_mean[len(moesq.FFN_STAGES):])},
            "side_passes": side_passes(pw, PP, float(pst_mean[len(moesq.FFN_STAGES)]),
                                       float(pst_mean[len(moesq.FFN_STAGES) + 3])),
            "roofline": {"bound": "mfma", "kernel": "k_gemm_prefill<gate_up>",
                         "achieved": round(ach, 2), "peak": F16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach / F16_DENSE_PEAK_TFLOPS, 4),
                         "traffic": _traffic(f"traffic_gemm_gate_up_{pw.name}.json", ("gemm.hip", "gemm_common.h", "moesq_device.h")),
                         "algorithmic_flops_per_launch": alg_flops, "avg_launch_ms": round(g_ms, 4),
                         "measured_peak": peaks["smfmac_f16_kept_TFLOPs"],
                         "frac_of_measured": round(ach / peaks["smfmac_f16_kept_TFLOPs"], 4)},
        }

    if not args.no_other_workloads:
        del layers, w13, w2
        torch.cuda.empty_cache()
        result["other_workloads"] = other_workloads(moesq, torch, ev, args.seed, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.seed, x, ids, wts, g13, g2, dense_expert, args.cpu_tokens)
    else:
        result["cpu_baseline"] = None
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
