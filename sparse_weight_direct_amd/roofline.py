"""Roofline arithmetic for sparse and dense direct convolution.

Cost model of Tuteja et al., "Theoretical and Empirical Analysis of Sparse Convolution",
Sec. 4: AI = FLOPs / bytes (Eq. (4)); dense FLOPs 2*N*Hout*Wout*OC*K^2*IC (Eq. (5));
dense traffic = (N*H*W*IC + K^2*IC*OC + Hout*Wout*N*OC) * P (Eq. (6)); sparse traffic
= (N*H*W*IC + N*Hout*Wout*OC)*P + (1-S)*K^2*IC*OC*(P + P_idx) (Eq. (7)); sparse FLOPs
= dense FLOPs * (1-S) (Eq. (8)).  Ridge point = peak FLOP/s / bandwidth (Sec. 4).

For this library's measurements the byte count is the algorithmic traffic of the packed
path: the input read once, the output written once, and the canonical packed filter
bank ({u32 offset, fp32 value} per non-zero plus M+1 row pointers) read once.
"""
from __future__ import annotations

# MI355X published peaks.  The fp32 vector peak is 256 CUs x 4 SIMDs x 32 FMA lanes x 2 FLOP x
# 2.4 GHz: a wave64 v_fmac_f32 every 2 cycles per SIMD.  Plain (not packed) v_fmac_f32 reaches
# it: the FMA probe (csrc/probes.hip) measures about 2.4-2.8 cycles per wave64 FMA and SIMD
# with two or more wavefronts per SIMD, so it is the roof of the fp32 FMA kernels here.
HBM_PEAK_GBS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 157.3


def ai_table1(sparsity: float, N=32, IC=32, OC=64, H=256, W=256, K=3, P=4.0, P_idx=0.0,
              packed_entry_bytes=4.0) -> float:
    """Arithmetic intensity per Eq. (7)/(8) with 'same' output size (Hout = H).

    The non-zero entry size (P + P_idx) is the packed 4-byte word of Sec. 5.3."""
    flops = 2.0 * N * H * W * OC * K * K * IC * (1.0 - sparsity)
    mem = (N * H * W * IC + N * H * W * OC) * P + (1.0 - sparsity) * K * K * IC * OC * packed_entry_bytes
    return flops / mem


def ai_dense(N=32, IC=32, OC=64, H=256, W=256, K=3, P=4.0) -> float:
    """Dense arithmetic intensity per Eq. (5)/(6) with Hout = H."""
    flops = 2.0 * N * H * W * OC * K * K * IC
    mem = (N * H * W * IC + K * K * IC * OC + H * W * N * OC) * P
    return flops / mem


def ridge(peak_tflops: float, bw_tbs: float) -> float:
    return peak_tflops / bw_tbs


# Devices of Sec. 4 (FP32 peak TFLOP/s, bandwidth TB/s) and MI355X.  The A100 line of
# Table 2 is reproduced with 1.5 TB/s; the ridge-point paragraph quotes 2 TB/s.
DEVICES = {
    "A100": (19.5, 2.0),
    "A100 (Table 2)": (19.5, 1.5),
    "Jetson AGX Orin 64GB": (5.32, 0.2048),
    "Jetson Orin Nano 8GB": (5.0, 0.068),
    "Jetson Nano (Tegra X1)": (0.236, 0.0256),
    "MI355X (fp32)": (FP32_VECTOR_PEAK_TFLOPS, HBM_PEAK_GBS / 1000.0),
}


def winograd_speedup(OC, IC, peak_tflops, bw_tbs, sparsity=0.9, N=32, H=256, W=None, K=3, reduction=2.0,
                     P=4.0, entry_bytes=4.0) -> float:
    """Roofline time of dense Winograd over roofline time of sparse direct convolution
    (Sec. 4.2): each time is max(T_comp, T_comm).  Winograd does the dense FLOPs of Eq. (5)
    divided by ``reduction`` and moves the dense bytes of Eq. (6); the sparse kernel does the
    FLOPs of Eq. (8) and moves the bytes of Eq. (7) with ``entry_bytes`` per non-zero.
    'Same' output size (Hout = H).  Tables 2 and 3 are reproduced with reduction 2.0."""
    W = H if W is None else W
    peak, bw = peak_tflops * 1e12, bw_tbs * 1e12
    flops = 2.0 * N * H * W * OC * K * K * IC
    dense_bytes = (N * H * W * IC + K * K * IC * OC + N * H * W * OC) * P
    sparse_bytes = (N * H * W * IC + N * H * W * OC) * P + (1.0 - sparsity) * K * K * IC * OC * entry_bytes
    t_wino = max(flops / reduction / peak, dense_bytes / bw)
    t_sparse = max(flops * (1.0 - sparsity) / peak, sparse_bytes / bw)
    return t_wino / t_sparse


def attainable_tflops(ai: float, peak_tflops: float, bw_tbs: float) -> float:
    """Roofline: min(peak, bandwidth * arithmetic intensity)."""
    return min(peak_tflops, bw_tbs * ai)


def _fmt_table(rows, header):
    w = [max(len(str(x)) for x in col) for col in zip(header, *rows)]
    line = lambda r: "| " + " | ".join(str(x).rjust(n) for x, n in zip(r, w)) + " |"
    return "\n".join([line(header), "|" + "|".join("-" * (n + 2) for n in w) + "|"] + [line(r) for r in rows])


def report(bench_json_paths=()) -> str:
    """Text roofline: ridge points, Table 1 intensities with the attainable rate on each
    device, Tables 2 and 3 recomputed (and for MI355X), and measured points from bench.py
    JSON lines (arithmetic intensity on algorithmic bytes, achieved and roof TFLOP/s)."""
    import json
    out = ["Ridge points (FP32 peak / bandwidth, FLOP/byte):"]
    out.append(_fmt_table([(n, p, bw, round(ridge(p, bw), 2)) for n, (p, bw) in DEVICES.items()],
                          ("device", "TFLOP/s", "TB/s", "ridge")))
    sp = [0.90, 0.91, 0.92, 0.93, 0.94, 0.95, 0.96, 0.97, 0.98]
    devs = ["A100", "Jetson Nano (Tegra X1)", "MI355X (fp32)"]
    rows = []
    for s in sp:
        ai = ai_table1(s)
        rows.append((s, round(ai, 2)) + tuple(round(attainable_tflops(ai, *DEVICES[d]), 3) for d in devs))
    out.append("\nTable 1 layer (N=32, IC=32, OC=64, 256x256, 3x3): AI and attainable TFLOP/s")
    out.append(_fmt_table(rows, ("sparsity", "AI") + tuple(devs)))
    for name, dev, N, H, ocs, ics in [("Table 2", "A100 (Table 2)", 32, 256, (32, 64, 128, 256, 512), (1, 16, 32, 64, 128)),
                                      ("Table 3", "Jetson Nano (Tegra X1)", 8, 128, (16, 24, 32, 40, 48), (1, 8, 16, 24, 32)),
                                      ("Table 2 shape on MI355X", "MI355X (fp32)", 32, 256,
                                       (32, 64, 128, 256, 512), (1, 16, 32, 64, 128))]:
        p, bw = DEVICES[dev]
        rows = [(oc,) + tuple(f"{winograd_speedup(oc, ic, p, bw, N=N, H=H):.1f}x" for ic in ics) for oc in ocs]
        out.append(f"\n{name} ({dev}): speedup over Winograd, rows OC, columns IC")
        out.append(_fmt_table(rows, ("OC \\ IC",) + ics))
    pts = []
    for path in bench_json_paths:
        for line in open(path):
            line = line.strip()
            if not line.startswith("{"):
                continue
            d = json.loads(line)
            if "arithmetic_intensity" not in d:
                continue
            ai = d["arithmetic_intensity"]
            roof = attainable_tflops(ai, *DEVICES["MI355X (fp32)"])
            pts.append((d["config"]["workload"].split(":")[0], ai, d["value"], round(roof, 1),
                        f"{100 * d['value'] / roof:.1f}%"))
    if pts:
        out.append("\nMeasured on MI355X (bench.py), AI on algorithmic bytes:")
        out.append(_fmt_table(pts, ("workload", "AI", "TFLOP/s", "roof TFLOP/s", "of roof")))
    return "\n".join(out)


if __name__ == "__main__":
    import sys
    print(report(sys.argv[1:]))


def effective_flops(nnz: int, N: int, E: int, F: int) -> float:
    """2 * nnz * N * E * F: every stored non-zero times every output position (Eq. (8)
    written with the realized non-zero count; taps that fall in padding are counted)."""
    return 2.0 * nnz * N * E * F


def algorithmic_bytes(N, C, H, W, M, E, F, nnz, entry_bytes=8) -> int:
    """Input once + output once + packed filter bank once: (2*nnz + M + 1) * 4 bytes for
    {offset, fp32 value} entries, (nnz + M + 1) * 4 for 32-bit packed words (entry_bytes 4)."""
    return 4 * N * C * H * W + 4 * N * M * E * F + entry_bytes * nnz + 4 * (M + 1)


def dense_flops(N, C, M, E, F, R, S) -> float:
    return 2.0 * N * M * E * F * C * R * S
