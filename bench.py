#!/usr/bin/env python3
"""Throughput benchmark of the sparse direct convolution forward pass on one MI355X.

A step is one sparseconv_forward over one batch: the 112x112 layer, batch 8, C = M = 128,
3x3, stride 1, pad 1, whose output channels have Beta(0.5, b) densities with mean
sparsity 95% (the middle of the 90-99% range the method targets).  Packing happens once,
before timing, as in deployment (weights stay resident).

Timing: W warm-up steps, then exactly K steps between two HIP events on the launch stream,
with a device synchronisation on both sides.  Input/output buffer sets rotate so the
working set exceeds the 256 MB Infinity Cache and every step reads its input from HBM.

Printed: one JSON line with effective TFLOP/s (2*nnz*N*E*F per second), the roofline of the
kernel (algorithmic bytes per launch over its average duration against 8 TB/s), the dense
direct baseline on the same GPU, and the CPU oracle timed on this host as a baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stored_traffic(layer: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when it is
    missing, for another workload, or taken on different kernel sources.  ``layer`` is the
    workload tag (the layer name, with "_fp16word" for the packed-word form)."""
    from sparse_weight_direct_amd.rocprof_summary import kernel_digest
    path = os.path.join(PROFILE_DIR, f"sparse_direct_fwd_{layer}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^(\w+):\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel_digest") != kernel_digest() or kv.get("workload") != layer:
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
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense direct baseline")
    ap.add_argument("--miopen", action="store_true", help="also time torch conv2d (MIOpen) as context")
    ap.add_argument("--chain", default=None,
                    help="also time a layer stack from workloads.CHAINS, eager launches vs one graph replay")
    ap.add_argument("--fp16-word", action="store_true",
                    help="pack the weights as 32-bit words with an fp16 value (SC_PACK_FP16_WORD)")
    ap.add_argument("--escoin", action="store_true",
                    help="time the second mapping (SC_PACK_ESCOIN_MAP: pad_in + one output channel per workgroup)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
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

    layer = args.layer or workloads.BENCH_LAYER
    d = workloads.make(layer)
    L = d["layer"]
    N, C, H, W, M, R, S, st, pad, E, F = L.N, L.C, L.H, L.W, L.M, L.R, L.S, L.stride, L.pad, L.E, L.F
    log(f"[bench] layer {layer}: N={N} C={C} {H}x{W} M={M} {R}x{S} s{st} p{pad} -> {E}x{F}")
    dev = torch.device("cuda:0")
    h = sc.Handle(M, C, R, S, H, W, st, pad, values=d["w"], mask=d["mask"],
                  flags=(sc.SC_PACK_FP16_WORD if args.fp16_word else 0) | (sc.SC_PACK_ESCOIN_MAP if args.escoin else 0))
    info = h.info()
    nnz = info["nnz"]
    tag = layer + ("_fp16word" if args.fp16_word else "") + ("_escoin" if args.escoin else "")
    ws_bytes = h.workspace_size(N)
    ws = torch.empty(max(ws_bytes, 4) // 4, dtype=torch.float32, device=dev) if ws_bytes else None
    flops = roofline.effective_flops(nnz, N, E, F)
    alg_bytes = roofline.algorithmic_bytes(N, C, H, W, M, E, F, nnz, info["entry_bytes"])
    set_bytes = 4 * (N * C * H * W + N * M * E * F)
    nsets = max(1, math.ceil(args.rotate_mb * (1 << 20) / set_bytes))
    x0 = torch.from_numpy(d["x"]).to(dev)
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    ys = [torch.empty((N, M, E, F), dtype=torch.float32, device=dev) for _ in range(nsets)]
    stream = torch.cuda.current_stream()
    log(f"[bench] nnz={nnz} plan={info} sets={nsets} ({nsets * set_bytes / 2**20:.0f} MiB rotated)")

    def run(fn, steps, warmup):
        for i in range(warmup):
            fn(i % nsets)
        torch.cuda.synchronize()
        groups = 10 if steps >= 10 else 1
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
        mean = total / steps
        sem = float(np.std(per, ddof=1) / math.sqrt(len(per))) if len(per) > 1 else 0.0
        return mean, sem

    def sparse_step(i):
        h.forward(xs[i], ys[i], stream=stream, workspace=ws)

    log(f"[bench] sparse: warmup {args.warmup}, timed {args.steps}")
    ms, sem = run(sparse_step, args.steps, args.warmup)
    tflops = flops / (ms * 1e-3) / 1e12
    achieved_gbs = alg_bytes / (ms * 1e-3) / 1e9
    ai = flops / alg_bytes
    flop_roof = min(roofline.HBM_PEAK_GBS * 1e9 * ai, roofline.FP32_VECTOR_PEAK_TFLOPS * 1e12) / 1e12
    log(f"[bench] sparse {ms * 1e3:.2f} us/step (SEM {sem * 1e3:.2f}), {tflops:.2f} TFLOP/s, {achieved_gbs:.0f} GB/s")

    def oracle_csr():
        """The oracle's CSR of the layer; for the packed-word form, the non-zeros decoded
        from the oracle's own words (fp16-rounded weights)."""
        import oracle
        rowptr, colidx, value = oracle.csr_from_dense(d["w"], d["mask"])
        if args.fp16_word:
            colidx, value = oracle.csr_from_words(oracle.words_from_csr(colidx, value, C, R, S), R, S)
        return rowptr, colidx, value

    # correctness of the timed buffers: sampled planes against the oracle
    parity = None
    try:
        import oracle
        rowptr, colidx, value = oracle_csr()
        rng = np.random.default_rng(0)
        planes = sorted(set(int(p) for p in rng.choice(N * M, min(8, N * M), replace=False)))
        y64, mag = oracle.conv_csr_planes(d["x"], rowptr, colidx, value, M, R, S, st, pad, planes)
        got = ys[0].cpu().numpy().reshape(N * M, E, F)[planes]
        parity = bool(oracle.within_tolerance(got, y64, mag, 1e-5).all())
    except Exception as e:  # report, never hide
        parity = f"error: {e}"
    log(f"[bench] parity on timed buffers: {parity}")

    extra = {}
    # warm variant: back-to-back forwards on one buffer set, whose input and output stay in
    # the Infinity Cache when they fit (context only; value above is the rotated, cold form)
    wsteps = max(10, args.steps // 2)
    wms, wsem = run(lambda i: h.forward(xs[0], ys[0], stream=stream, workspace=ws), wsteps, 3)
    extra["warm_one_set"] = {"ms_per_step": round(wms, 5), "sem_ms": round(wsem, 5),
                             "tflops": round(flops / (wms * 1e-3) / 1e12, 3), "set_mb": round(set_bytes / 2**20, 1)}
    log(f"[bench] warm (one buffer set, {set_bytes / 2**20:.0f} MiB): {wms * 1e3:.2f} us/step")
    if not args.no_dense:
        hd = sc.Handle(M, C, R, S, H, W, st, pad, values=d["w_masked"], flags=sc.SC_PACK_ALL_TAPS)

        def dense_step(i):
            hd.forward(xs[i], ys[i], stream=stream)

        dsteps = max(10, args.steps // 10)
        log(f"[bench] dense direct baseline: warmup 2, timed {dsteps}")
        dms, dsem = run(dense_step, dsteps, 2)
        extra["dense_direct"] = {"ms_per_step": round(dms, 5), "sem_ms": round(dsem, 5),
                                 "tflops_dense_work": round(roofline.dense_flops(N, C, M, E, F, R, S) / (dms * 1e-3) / 1e12, 3),
                                 "speedup_sparse_over_dense": round(dms / ms, 3)}
        log(f"[bench] dense {dms * 1e3:.1f} us/step -> sparse speedup {dms / ms:.2f}x")
    if args.miopen:
        wd = torch.from_numpy(d["w_masked"]).to(dev)

        def miopen_step(i):
            torch.nn.functional.conv2d(xs[i], wd, stride=st, padding=pad)

        mms, _ = run(miopen_step, max(10, args.steps // 10), 3)
        extra["torch_conv2d_miopen_ms"] = round(mms, 5)

    if args.chain:
        from sparse_weight_direct_amd.chain import LayerChain
        layers = workloads.make_chain(args.chain)
        chain = LayerChain([sc.Handle(values=cd["w"], mask=cd["mask"], **cd["geom"]) for cd in layers],
                           N=layers[0]["x"].shape[0], device=dev)
        chain.x.copy_(torch.from_numpy(layers[0]["x"]))
        eager_ms, _ = run(lambda i: chain.run(), args.steps, args.warmup)
        chain.capture()
        graph_ms, _ = run(lambda i: chain.replay(), args.steps, args.warmup)
        cflops = sum(roofline.effective_flops(int(cd["mask"].sum()), cd["x"].shape[0] if j == 0 else chain.N,
                                              chain.handles[j].E, chain.handles[j].F)
                     for j, cd in enumerate(layers))
        extra["chain"] = {"name": args.chain, "layers": len(layers), "eager_us": round(eager_ms * 1e3, 2),
                          "graph_us": round(graph_ms * 1e3, 2),
                          "graph_tflops": round(cflops / (graph_ms * 1e-3) / 1e12, 3)}
        log(f"[bench] chain {args.chain}: eager {eager_ms * 1e3:.1f} us, graph {graph_ms * 1e3:.1f} us per stack")

    if args.copy_mb > 0:
        nb = args.copy_mb << 20
        src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)

        def copy_step(i):
            dst.copy_(src)

        cms, _ = run(copy_step, 10, 2)
        extra["copy_reference"] = {"bytes_per_copy": nb, "ms": round(cms, 5),
                                   "gbs_read_plus_write": round(2 * nb / (cms * 1e-3) / 1e9, 1)}
        log(f"[bench] copy of {args.copy_mb} MiB: {cms * 1e3:.1f} us -> {2 * nb / (cms * 1e-3) / 1e9:.0f} GB/s (read+write)")
        del src, dst

    cpu = None
    if not args.no_cpu:
        import oracle
        rowptr, colidx, value = oracle_csr()
        threads = oracle.max_threads()
        t = time.perf_counter()
        oracle.conv_csr(d["x"][:1], rowptr, colidx, value, M, R, S, st, pad)
        t1 = time.perf_counter() - t
        n_img = max(1, min(N, int(args.cpu_seconds / max(t1, 1e-3))))
        log(f"[bench] CPU oracle: 1 image {t1:.3f} s; timing {n_img} image(s) per run on {threads} threads")
        # a batch that finishes quickly is repeated until about cpu_seconds have passed
        reps = 0
        t = time.perf_counter()
        while True:
            oracle.conv_csr(d["x"][:n_img], rowptr, colidx, value, M, R, S, st, pad)
            reps += 1
            tc = time.perf_counter() - t
            if tc >= args.cpu_seconds or reps >= 10000:
                break
        cpu = {"value": roofline.effective_flops(nnz, n_img, E, F) * reps / tc / 1e12, "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle",
               "sample": f"list-form oracle (fp64 accumulate), {reps} run(s) over {n_img} of {N} images, "
                         f"all {M} output channels, {tc:.1f} s"}

    traffic = stored_traffic(tag)
    sp = round(100 * L.sparsity)
    mask_text = {"beta_rows": f"per-channel density Beta(0.5,b) mean sparsity {sp}%",
                 "exact": f"uniform unstructured {sp}% sparsity (exact count)",
                 "bernoulli": f"i.i.d. Bernoulli mask, {sp}% sparsity"}.get(L.mask_kind, f"{sp}% sparsity")
    mask_text += {"u11": ", inputs U[-1,1]", "relu_n01": ", inputs ReLU(N(0,1))"}.get(L.x_dist, "")
    mask_text += {"u11": ", weights U[-1,1]", "n0.05": ", weights N(0,0.05)", "n0.02": ", weights N(0,0.02)"}.get(
        L.w_dist, "")
    out = {
        "metric": "sparse conv effective TFLOP/s (2*nnz*N*E*F/s) and % of HBM roofline",
        "value": round(tflops, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{layer}: N={N} C={C} H=W={H} M={M} {R}x{S} stride {st} pad {pad}, "
                               f"{mask_text}, "
                               f"realized nnz={nnz} ({100 * (1 - nnz / (M * C * R * S)):.2f}% sparse)"
                               + (", weights as 32-bit words with fp16 values" if args.fp16_word else "")
                               + (", Escoin mapping (pad_in + one output channel per workgroup)" if args.escoin else ""),
                   "N": N, "C": C, "H": H, "W": W, "M": M, "R": R, "S": S, "stride": st, "pad": pad, "nnz": nnz},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": roofline.HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved_gbs / roofline.HBM_PEAK_GBS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "sem_ms": round(sem, 6),
        "arithmetic_intensity": round(ai, 2),
        "flop_roofline_frac": round(tflops / flop_roof, 4),
        "parity_on_timed_buffers": parity,
        "plan": {k: info[k] for k in ("tile_pixels", "rows_per_wave", "row_groups", "chunk_channels", "lds_bytes",
                                      "max_wave_nnz", "entry_bytes", "mapping")},
        "rotated_sets": nsets,
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
