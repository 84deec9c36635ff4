#!/usr/bin/env python3
"""Throughput benchmark of the sparse direct convolution forward pass on one MI355X.

A step is one sparseconv_forward over one batch: the 112x112 layer, batch 8, C = M = 128,
3x3, stride 1, pad 1, whose output channels have Beta(0.5, b) densities with mean
sparsity 95% (the middle of the 90-99% range the method targets).  Packing happens once,
before timing, as in deployment (weights stay resident), and so does the choice of kernel for
the batch size where the grid leaves SIMDs idle (sparseconv_tune times the handle's kernels and
pins the fastest); the forward launches one kernel (on this layer the staged weights-in-code
kernel).

Timing: W warm-up steps, then exactly K steps between two HIP events on the launch stream,
with a device synchronisation on both sides, one library call per step; no event is recorded
inside a window shorter than 200 steps (an event between two forwards holds the stream for
~1.5-3 us: with one every 2 steps, a 20-step window ran 1.5 us per step slower), and the SEM
comes from 5 further windows of K steps timed after it.  The same K steps launched from HIP
graphs (up to 24 forwards captured once and replayed, and a graph of the remaining steps) are
timed too and reported beside them (--launch graph makes those the value).  Both run after
the bench's other measurements of the same layer (references, dense baselines, roof probes,
1000 warm forwards), so the GPU's clock has left its idle state: from idle it rises over the
first ~30 ms of sustained work, and a window of a few dozen steps right after start-up would
time that ramp.
Input/output buffer sets rotate so the working set exceeds the 256 MB Infinity Cache and every
step reads its input from HBM ("cold").

Printed: one JSON line with effective TFLOP/s (2*nnz*N*E*F per second) as ``value``, the
roofline of the kernel (bound from the arithmetic intensity against the ridge of 8 TB/s and
the 157.3 TFLOP/s fp32 vector FMA peak, which plain v_fmac_f32 reaches: the FMA probe timed
here measures it), the HBM fraction, the plan the forward launched, the roof probes (FMA rate
by wavefronts per SIMD, LDS read bandwidth), every other workload layer timed the same way
(``per_config``; with ``graph_us``, the same forwards replayed from one HIP graph, which leaves
out the host's launch cost of about 5 us per call that bounds the smallest layers), the dense
direct baseline and torch's conv2d (MIOpen) on the same GPU, and the CPU oracle on this host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stored_traffic(tag: str, mapping: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when it is
    missing, for another workload, or taken on different kernel sources."""
    from sparse_weight_direct_amd.rocprof_summary import kernel_digest
    kernel = {0: "sparse_direct_fwd", 1: "escoin_sconv", 2: "sc_baked"}.get(mapping, "?")
    path = os.path.join(PROFILE_DIR, f"{kernel}_{tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^(\w+):\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel_digest") != kernel_digest(kernel) or kv.get("workload") != tag:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layer", default=None, help="layer name from workloads.LAYERS")
    ap.add_argument("--rotate-mb", type=int, default=768, help="total size of the rotated buffer sets")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline (and the parity check)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense direct baseline")
    ap.add_argument("--no-miopen", action="store_true", help="skip torch conv2d (MIOpen) as context")
    ap.add_argument("--no-configs", action="store_true", help="skip timing the other workload layers")
    ap.add_argument("--lds-tile", action="store_true", help="use the LDS-tile kernel (SC_PACK_LDS_TILE)")
    ap.add_argument("--chain", default=None,
                    help="also time a layer stack from workloads.CHAINS, eager launches vs one graph replay")
    ap.add_argument("--fp16-word", action="store_true",
                    help="pack the weights as 32-bit words with an fp16 value (SC_PACK_FP16_WORD)")
    ap.add_argument("--escoin", action="store_true",
                    help="time the second mapping (SC_PACK_ESCOIN_MAP: pad_in + one output channel per workgroup)")
    ap.add_argument("--cpu-seconds", type=float, default=4.0, help="target CPU time of one timed oracle run")
    ap.add_argument("--no-probes", action="store_true", help="skip the FMA and LDS roof probes")
    ap.add_argument("--no-tune", action="store_true",
                    help="launch the kernels the cost estimate picks instead of tuning each layer first")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="how the timed steps are launched: one library call per step (default) or from HIP "
                         "graphs of up to 24 forwards each; the other form is reported beside it")
    ap.add_argument("--copy-mb", type=int, default=1024,
                    help="size of the device-to-device copy timed as the achievable-HBM reference (0: skip)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: the forward pass needs no collective and "
                                   "multi-GPU sharding is described, not implemented; use --gpus 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_weight_direct_amd as sc
    import workloads
    from sparse_weight_direct_amd import roofline

    flags = ((sc.SC_PACK_FP16_WORD if args.fp16_word else 0) | (sc.SC_PACK_ESCOIN_MAP if args.escoin else 0)
             | (sc.SC_PACK_LDS_TILE if args.lds_tile else 0))
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def run(fn, steps, warmup, nsets):
        """ms per step over exactly ``steps`` launches between two HIP events (after ``warmup``
        untimed ones and a synchronisation) and its SEM.  An event recorded between launches
        holds the stream for ~1.5-3 us, so the timed window gets inner events (groups for the
        SEM) only every 100 steps or more; a shorter window takes its SEM from 5 further
        windows of the same length, timed after it."""
        for i in range(warmup):
            fn(i % nsets)
        torch.cuda.synchronize()
        groups = max(1, min(10, steps // 100))
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
        bounds = [round(g * steps / groups) for g in range(groups + 1)]
        evs[0].record(stream)
        for g in range(groups):
            for i in range(bounds[g], bounds[g + 1]):
                fn(i % nsets)
            evs[g + 1].record(stream)
        torch.cuda.synchronize()
        total = evs[0].elapsed_time(evs[-1])
        per = [evs[g].elapsed_time(evs[g + 1]) / (bounds[g + 1] - bounds[g]) for g in range(groups)]
        if groups == 1:
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(steps):
                    fn(i % nsets)
                e1.record(stream)
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) / steps)
        sem = float(np.std(per, ddof=1) / math.sqrt(len(per)))
        return total / steps, sem

    def run_graph(fwd, steps, warmup, nsets, per_graph=24):
        """ms per step and its SEM when the steps are launched from HIP graphs: ``warmup`` forwards
        launched one by one, then per_graph forwards over the rotated buffer sets (forward j on set
        j % nsets) captured once and replayed, plus a graph of the remaining steps, so exactly
        ``steps`` forwards run in the timed region."""
        for i in range(warmup):
            fwd(i % nsets)
        torch.cuda.synchronize()
        per_graph = max(1, min(per_graph, steps))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())

        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for j in range(n):
                    fwd(j % nsets, None)
            return g

        full, rest = capture(per_graph), (capture(steps % per_graph) if steps % per_graph else None)
        torch.cuda.synchronize()
        # no untimed replay: a graph's first launch measured no slower than its later ones
        # an inner event (for the SEM) after every `every` replays: at least 100 forwards apart
        nrep, every = steps // per_graph, -(-100 // per_graph)
        marks = [r for r in range(every, nrep + 1, every)]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(marks) + 2)]
        evs[0].record(stream)
        for r in range(1, nrep + 1):
            full.replay()
            if r in marks:
                evs[marks.index(r) + 1].record(stream)
        if rest is not None:
            rest.replay()
        evs[-1].record(stream)
        torch.cuda.synchronize()
        total = evs[0].elapsed_time(evs[-1])
        per = [evs[i].elapsed_time(evs[i + 1]) / (every * per_graph) for i in range(len(marks))]
        sem = float(np.std(per, ddof=1) / math.sqrt(len(per))) if len(per) > 1 else 0.0
        del full, rest
        return total / steps, sem

    def setup(name):
        """Pack a layer and allocate rotated buffer sets (inputs resident in HBM)."""
        d = workloads.make(name)
        L = d["layer"]
        h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"], flags=flags)
        ws_bytes = h.workspace_size(L.N)
        ws = torch.empty(max(ws_bytes, 4) // 4, dtype=torch.float32, device=dev) if ws_bytes else None
        set_bytes = 4 * (L.N * L.C * L.H * L.W + L.N * L.M * L.E * L.F)
        nsets = max(1, math.ceil(args.rotate_mb * (1 << 20) / set_bytes))
        x0 = torch.from_numpy(d["x"]).to(dev)
        xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
        ys = [torch.empty((L.N, L.M, L.E, L.F), dtype=torch.float32, device=dev) for _ in range(nsets)]
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        if not args.no_tune and ws is None and h.launch_info(L.N)["waves"] < 4 * cus:
            # deployment setup, once per layer and batch size: where the grid leaves SIMDs without
            # a wavefront the forward's choice rests on a coarse estimate, so time the handle's
            # kernels for this batch and pin the fastest (sparseconv_tune; it times one warm
            # buffer set, which misleads on the large layers, where the base kernel is launched)
            h.tune(xs[0], ys[0], reps=5, stream=stream)
        return d, L, h, ws, xs, ys, nsets, set_bytes

    def graph_us(hh, xxs, yys, nn, wws, k=20, reps=3):
        """GPU time per forward with no host launch cost between forwards: k forwards over
        rotated (cold) buffer sets captured in one HIP graph, replayed reps times."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(k):
                hh.forward(xxs[i % nn], yys[i % nn], workspace=wws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / (k * reps)

    def describe(L, info, ms):
        nnz = info["nnz"]
        flops = roofline.effective_flops(nnz, L.N, L.E, L.F)
        alg = roofline.algorithmic_bytes(L.N, L.C, L.H, L.W, L.M, L.E, L.F, nnz, info["entry_bytes"])
        ai = flops / alg
        ridge = roofline.FP32_VECTOR_PEAK_TFLOPS * 1e12 / (roofline.HBM_PEAK_GBS * 1e9)
        tflops = flops / (ms * 1e-3) / 1e12
        gbs = alg / (ms * 1e-3) / 1e9
        bound = "alu" if ai > ridge else "hbm"
        frac = tflops / roofline.FP32_VECTOR_PEAK_TFLOPS if bound == "alu" else gbs / roofline.HBM_PEAK_GBS
        return dict(flops=flops, alg=alg, ai=ai, tflops=tflops, gbs=gbs, bound=bound, frac=frac)

    layer = args.layer or workloads.BENCH_LAYER
    d, L, h, ws, xs, ys, nsets, set_bytes = setup(layer)
    N, C, H, W, M, R, S, st, pad, E, F = L.N, L.C, L.H, L.W, L.M, L.R, L.S, L.stride, L.pad, L.E, L.F
    info = h.info()
    nnz = info["nnz"]
    launch = h.launch_info(N)
    log(f"[bench] layer {layer}: N={N} C={C} {H}x{W} M={M} {R}x{S} s{st} p{pad} -> {E}x{F}, nnz={nnz}, "
        f"launch {launch}, {nsets} rotated sets ({nsets * set_bytes / 2**20:.0f} MiB)")

    extra = {}
    # The bench's other measurements of this layer (references, baselines, roof probes) run
    # first and the headline's own warm-up and timed steps right after them: from idle the GPU
    # raises its clock over the first ~30 ms of sustained work (this layer measured 30-33 us per
    # forward in its first 500 launches from idle, 25.8 us after 1000), so a short timed window
    # right after start-up would measure the clock's ramp rather than the kernel.
    t_aux = time.perf_counter()

    if not args.no_dense:
        wd = torch.from_numpy(d["w_masked"]).to(dev)
        yd = torch.empty((N, M, E, F), dtype=torch.float32, device=dev)
        def dense_step(i):
            sc.sparseconv_dense_forward(wd, xs[i], yd, N, C, H, W, M, R, S, st, pad, stream)
        kind = "sparseconv_dense_forward (dense fp32 weights on the device, every tap, vector FMA)"
        dsteps = max(10, args.steps // 10)
        dms, dsem = run(dense_step, dsteps, 2, nsets)
        extra["dense_direct"] = {"kind": kind, "ms_per_step": round(dms, 5), "sem_ms": round(dsem, 5),
                                 "tflops_dense_work": round(roofline.dense_flops(N, C, M, E, F, R, S) / (dms * 1e-3)
                                                            / 1e12, 3)}
        log(f"[bench] dense direct {dms * 1e3:.1f} us/step")
    if not args.no_miopen:
        wd = torch.from_numpy(d["w_masked"]).to(dev)

        def miopen_step(i):
            torch.nn.functional.conv2d(xs[i], wd, stride=st, padding=pad)

        mms, msem = run(miopen_step, max(10, args.steps // 10), 3, nsets)
        extra["torch_conv2d_miopen"] = {"ms_per_step": round(mms, 5), "sem_ms": round(msem, 5),
                                        "tflops_dense_work": round(roofline.dense_flops(N, C, M, E, F, R, S)
                                                                   / (mms * 1e-3) / 1e12, 3)}
        log(f"[bench] torch conv2d (MIOpen, dense fp32) {mms * 1e3:.1f} us/step")

    if args.chain:
        from sparse_weight_direct_amd.chain import LayerChain
        layers = workloads.make_chain(args.chain)
        chain = LayerChain([sc.Handle(values=cd["w"], mask=cd["mask"], **cd["geom"]) for cd in layers],
                           N=layers[0]["x"].shape[0], device=dev)
        chain.x.copy_(torch.from_numpy(layers[0]["x"]))
        eager_ms, _ = run(lambda i: chain.run(), args.steps, args.warmup, 1)
        chain.capture()
        graph_ms, _ = run(lambda i: chain.replay(), args.steps, args.warmup, 1)
        # the same stack 20 times per graph launch: its time on the GPU, without the host's cost
        # of launching a graph (which bounds one small stack per launch)
        rep = 20
        chain.capture(repeat=rep)
        gpu_ms, _ = run(lambda i: chain.replay(), max(10, args.steps // rep), 2, 1)
        gpu_ms /= rep
        cflops = sum(roofline.effective_flops(int(cd["mask"].sum()), cd["x"].shape[0] if j == 0 else chain.N,
                                              chain.handles[j].E, chain.handles[j].F)
                     for j, cd in enumerate(layers))
        extra["chain"] = {"name": args.chain, "layers": len(layers), "eager_us": round(eager_ms * 1e3, 2),
                          "graph_us": round(graph_ms * 1e3, 2),
                          "graph_tflops": round(cflops / (graph_ms * 1e-3) / 1e12, 3),
                          "gpu_us_20_stacks_per_graph": round(gpu_ms * 1e3, 2)}
        log(f"[bench] chain {args.chain}: eager {eager_ms * 1e3:.1f} us, graph {graph_ms * 1e3:.1f} us per stack, "
            f"{gpu_ms * 1e3:.1f} us per stack with 20 stacks per graph launch")

    if args.copy_mb > 0:
        nb = args.copy_mb << 20
        src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        cms, _ = run(lambda i: dst.copy_(src), 10, 2, 1)
        extra["copy_reference"] = {"bytes_per_copy": nb, "ms": round(cms, 5),
                                   "gbs_read_plus_write": round(2 * nb / (cms * 1e-3) / 1e9, 1)}
        log(f"[bench] copy of {args.copy_mb} MiB: {2 * nb / (cms * 1e-3) / 1e9:.0f} GB/s (read+write)")
        del src, dst
        # the same traffic as one forward of the headline layer, in the same form: a device copy
        # of one input buffer set (read) into an output-sized buffer (written), rotated over the
        # same sets, launched back to back -- what plain streaming reaches at this size
        if xs[0].numel() == ys[0].numel():
            zs = [torch.empty_like(y) for y in ys]  # the forward's outputs stay for the parity check
            ms_copy, _ = run(lambda i: zs[i].view(-1).copy_(xs[i].view(-1)), args.steps, args.warmup, nsets)
            del zs
            same_bytes = xs[0].numel() * 4 + ys[0].numel() * 4
            extra["copy_same_size"] = {
                "bytes_read_plus_written": same_bytes, "us": round(ms_copy * 1e3, 2),
                "gbs": round(same_bytes / (ms_copy * 1e-3) / 1e9, 1),
                "frac_of_8tbs": round(same_bytes / (ms_copy * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 4)}
            log(f"[bench] copy of one input set into an output buffer ({same_bytes / 2**20:.0f} MiB moved): "
                f"{ms_copy * 1e3:.2f} us, {extra['copy_same_size']['gbs']:.0f} GB/s")

    if not args.no_probes:
        # roofs of the instruction mixes the kernels are made of (csrc/probes.hip): the fp32 FMA
        # rate of plain v_fmac_f32 (literal weight, as in the weights-in-code kernels; VGPR
        # weight) by wavefronts per SIMD, and the LDS read bandwidth
        from sparse_weight_direct_amd import probes
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        fma = {f"literal_{w}_waves_per_simd": round(probes.fma_rate(cus, w, True), 2) for w in (1, 2, 4)}
        fma["vgpr_4_waves_per_simd"] = round(probes.fma_rate(cus, 4, False), 2)
        best = max(fma.values())
        extra["roof_probes"] = {
            "fma_tflops": fma, "fma_peak_tflops": roofline.FP32_VECTOR_PEAK_TFLOPS,
            "fma_frac_of_peak": round(best / roofline.FP32_VECTOR_PEAK_TFLOPS, 3),
            "lds_read_tbs": {"b32": round(probes.lds_read_rate(cus, 1), 2), "b128": round(probes.lds_read_rate(cus, 4), 2)},
            # a pure read stream over the headline layer's input buffer sets (one per launch,
            # rotated as the forward reads them): the HBM read rate at this size
            "hbm_read_gbs_input_sets": round(max(probes.read_rate(xs, cus * k) for k in (4, 8, 16)), 1),
            "headline_kernel_lds_bytes_per_workgroup": launch["lds_bytes"],
            "headline_kernel_stages_input_in_lds": bool(launch["stage"])}
        log(f"[bench] roof probes: FMA {fma} TFLOP/s, LDS {extra['roof_probes']['lds_read_tbs']} TB/s, "
            f"HBM read {extra['roof_probes']['hbm_read_gbs_input_sets']} GB/s")

    # warm variant, measured last before the headline: 1000 back-to-back forwards on one buffer
    # set, whose input and output stay in the Infinity Cache when they fit (context only; value
    # is the rotated, cold form)
    wms, wsem = run(lambda i: h.forward(xs[0], ys[0], stream=stream, workspace=ws), 1000, 3, 1)
    extra["warm_one_set"] = {"ms_per_step": round(wms, 5), "sem_ms": round(wsem, 5), "steps": 1000,
                             "tflops": round(describe(L, info, wms)["tflops"], 3),
                             "set_mb": round(set_bytes / 2**20, 1)}
    log(f"[bench] warm (one buffer set): {wms * 1e3:.2f} us/step")
    aux_ms = (time.perf_counter() - t_aux) * 1e3
    log(f"[bench] sparse: warmup {args.warmup}, timed {args.steps} (after {aux_ms:.0f} ms of the bench's other "
        f"measurements of this layer)")

    def fwd(i, st=stream):
        h.forward(xs[i], ys[i], stream=st, workspace=ws)

    ms_eager, sem_eager = run(fwd, args.steps, args.warmup, nsets)
    ms_graph, sem_graph = run_graph(fwd, args.steps, args.warmup, nsets)
    ms, sem = (ms_graph, sem_graph) if args.launch == "graph" else (ms_eager, sem_eager)
    m = describe(L, info, ms)
    log(f"[bench] sparse {ms * 1e3:.2f} us/step (SEM {sem * 1e3:.2f}, launched {args.launch}; eager "
        f"{ms_eager * 1e3:.2f}, from graphs {ms_graph * 1e3:.2f}), {m['tflops']:.2f} TFLOP/s, "
        f"{m['gbs']:.0f} GB/s algorithmic, AI {m['ai']:.1f}")
    if "dense_direct" in extra:
        extra["dense_direct"]["speedup_sparse_over_dense"] = round(extra["dense_direct"]["ms_per_step"] / ms, 3)
        log(f"[bench] sparse over dense direct: {extra['dense_direct']['speedup_sparse_over_dense']:.2f}x")
    if "torch_conv2d_miopen" in extra:
        extra["torch_conv2d_miopen"]["speedup_sparse_over_miopen"] = round(
            extra["torch_conv2d_miopen"]["ms_per_step"] / ms, 3)
    if "copy_same_size" in extra:
        extra["copy_same_size"]["forward_over_copy"] = round(ms / (extra["copy_same_size"]["us"] * 1e-3), 3)
        log(f"[bench] the forward takes {extra['copy_same_size']['forward_over_copy']:.2f}x the same-size copy")

    # every workload layer, timed the same way (cold, rotated sets), with the launched plan
    if not args.no_configs and not args.layer:
        per = {}
        for name in workloads.LAYERS:
            if name == layer:
                continue
            dd, LL, hh, wws, xxs, yys, nn, _ = setup(name)
            steps = 400  # enough launches that the first ones after the synchronisation do not weigh
            cms_, csem = run(lambda i: hh.forward(xxs[i], yys[i], stream=stream, workspace=wws), steps, 20, nn)
            mm = describe(LL, hh.info(), cms_)
            li = hh.launch_info(LL.N)
            gus = graph_us(hh, xxs, yys, nn, wws)
            per[name] = {"us": round(cms_ * 1e3, 2), "sem_us": round(csem * 1e3, 2), "graph_us": round(gus, 2),
                         "tflops": round(mm["tflops"], 3),
                         "frac_of_8tbs": round(mm["gbs"] / roofline.HBM_PEAK_GBS, 4), "ai": round(mm["ai"], 2),
                         "bound": mm["bound"], "roofline_frac": round(mm["frac"], 4), "nnz": hh.info()["nnz"],
                         "launch": {k: li[k] for k in ("mapping", "variant", "stage", "groups", "splits",
                                                       "units_per_wg", "depth", "grid", "waves", "vgprs",
                                                       "lds_bytes", "tile_pixels", "chunk_channels", "quad")}}
            log(f"[bench] config {name}: {cms_ * 1e3:.1f} us ({gus:.1f} us replayed from a graph), {mm['tflops']:.2f} TFLOP/s, "
                f"{mm['gbs'] / roofline.HBM_PEAK_GBS:.3f} of 8 TB/s, launch {per[name]['launch']}")
            del dd, hh, xxs, yys
            torch.cuda.empty_cache()
        per[layer] = {"us": round(ms * 1e3, 2), "sem_us": round(sem * 1e3, 2),
                      "graph_us": round(graph_us(h, xs, ys, nsets, ws), 2), "tflops": round(m["tflops"], 3),
                      "frac_of_8tbs": round(m["gbs"] / roofline.HBM_PEAK_GBS, 4), "ai": round(m["ai"], 2),
                      "bound": m["bound"], "roofline_frac": round(m["frac"], 4), "nnz": nnz,
                      "launch": {k: launch[k] for k in ("mapping", "variant", "stage", "groups", "splits",
                                                        "units_per_wg", "depth", "grid", "waves", "vgprs",
                                                        "lds_bytes", "tile_pixels", "chunk_channels", "quad")}}
        extra["per_config"] = per

    # CPU oracle: one untimed run over the whole batch (whose result also checks every output
    # of the first timed buffer set), then three timed runs over a bounded sample of images
    # (median), and a single-thread run over a few output planes
    cpu = None
    parity = None
    if not args.no_cpu:
        import oracle

        rowptr, colidx, value = oracle.csr_from_dense(d["w"], d["mask"])
        if args.fp16_word:
            colidx, value = oracle.csr_from_words(oracle.words_from_csr(colidx, value, C, R, S), R, S)
        threads = oracle.max_threads()
        t = time.perf_counter()
        y64, mag = oracle.conv_csr(d["x"], rowptr, colidx, value, M, R, S, st, pad)
        t_full = time.perf_counter() - t
        got = ys[0].cpu().numpy()
        ok = oracle.within_tolerance(got, y64, mag, 1e-5)
        parity = {"checked": int(ok.size), "outside_tolerance": int((~ok).sum()), "all_within": bool(ok.all())}
        log(f"[bench] CPU oracle: full batch {t_full:.3f} s on {threads} threads; parity on timed buffers {parity}")
        # a timed run repeats the whole batch until about cpu_seconds have passed
        reps = max(1, int(math.ceil(args.cpu_seconds / max(t_full, 1e-4))))
        times = []
        for _ in range(3):
            t = time.perf_counter()
            for _ in range(reps):
                oracle.conv_csr(d["x"], rowptr, colidx, value, M, R, S, st, pad)
            times.append(time.perf_counter() - t)
        tmed = statistics.median(times)
        n_img = N * reps
        planes = np.arange(min(64, M))
        t = time.perf_counter()
        oracle.conv_csr_planes(d["x"][:1], rowptr, colidx, value, M, R, S, st, pad, planes, nthreads=1)
        t1 = time.perf_counter() - t
        nnz_planes = int(sum(rowptr[p + 1] - rowptr[p] for p in planes))
        cpu = {"value": round(roofline.effective_flops(nnz, n_img, E, F) / tmed / 1e12, 6), "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle",
               "sample": f"list-form oracle (fp64 accumulate), median of 3 timed runs, each the whole batch "
                         f"({N} images, all {M} output channels) {reps} times over ({tmed:.2f} s each), after one "
                         f"untimed run over the batch ({t_full:.3f} s)",
               "single_thread_tflops": round(2.0 * nnz_planes * E * F / t1 / 1e12, 6),
               "single_thread_sample": f"{len(planes)} output planes of one image, 1 thread, {t1:.2f} s"}

    traffic = stored_traffic(layer + ("_fp16word" if args.fp16_word else "") + ("_escoin" if args.escoin else ""),
                             launch["mapping"])
    sp = round(100 * L.sparsity)
    mask_text = {"beta_rows": f"per-channel density Beta(0.5,b) mean sparsity {sp}%",
                 "exact": f"uniform unstructured {sp}% sparsity (exact count)",
                 "bernoulli": f"i.i.d. Bernoulli mask, {sp}% sparsity"}.get(L.mask_kind, f"{sp}% sparsity")
    mask_text += {"u11": ", inputs U[-1,1]", "relu_n01": ", inputs ReLU(N(0,1))"}.get(L.x_dist, "")
    mask_text += {"u11": ", weights U[-1,1]", "n0.05": ", weights N(0,0.05)", "n0.02": ", weights N(0,0.02)"}.get(
        L.w_dist, "")
    peak = roofline.FP32_VECTOR_PEAK_TFLOPS if m["bound"] == "alu" else roofline.HBM_PEAK_GBS
    achieved = m["tflops"] if m["bound"] == "alu" else m["gbs"]
    out = {
        "metric": "sparse conv effective TFLOP/s (2*nnz*N*E*F/s) and % of HBM roofline",
        "value": round(m["tflops"], 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "launch": {"timed_with": args.launch,
                   "after_other_measurements_ms": round(aux_ms, 1),
                   "graph": "HIP graphs of 24 forwards each over the rotated buffer sets (one step = one forward)",
                   "ms_per_step_graph": round(ms_graph, 6), "sem_ms_graph": round(sem_graph, 6),
                   "ms_per_step_eager": round(ms_eager, 6), "sem_ms_eager": round(sem_eager, 6)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{layer}: N={N} C={C} H=W={H} M={M} {R}x{S} stride {st} pad {pad}, "
                               f"{mask_text}, realized nnz={nnz} ({100 * (1 - nnz / (M * C * R * S)):.2f}% sparse)"
                               + (", weights as 32-bit words with fp16 values" if args.fp16_word else "")
                               + (", Escoin mapping (pad_in + one output channel per workgroup)" if args.escoin else "")
                               + (", LDS-tile kernel" if args.lds_tile else ""),
                   "N": N, "C": C, "H": H, "W": W, "M": M, "R": R, "S": S, "stride": st, "pad": pad, "nnz": nnz},
        "roofline": {"bound": m["bound"], "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s" if m["bound"] == "alu" else "GB/s", "frac": round(m["frac"], 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "sem_ms": round(sem, 6),
        "hbm": {"achieved_gbs": round(m["gbs"], 1), "peak_gbs": roofline.HBM_PEAK_GBS,
                "frac": round(m["gbs"] / roofline.HBM_PEAK_GBS, 4), "algorithmic_bytes": int(m["alg"])},
        "arithmetic_intensity": round(m["ai"], 2),
        "ridge_flop_per_byte": round(roofline.FP32_VECTOR_PEAK_TFLOPS / roofline.HBM_PEAK_GBS * 1e3, 2),
        "parity_on_timed_buffers": parity,
        "plan": launch,
        "rotated_sets": nsets,
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
