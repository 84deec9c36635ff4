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

# MI355X published peaks.
HBM_PEAK_GBS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 157.3      # counts packed FP32 FMA
FP32_VECTOR_NONPACKED_TFLOPS = 78.6  # 256 CUs x 4 SIMD x 16 lanes x 2 FLOP x 2.4 GHz


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
