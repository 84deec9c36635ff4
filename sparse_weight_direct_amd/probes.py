"""Roof probes (csrc/probes.hip, built into libscprobe.so): the fp32 FMA rate of the vector
ALUs and the LDS read bandwidth, measured on the device the way the benchmark times its copy
reference.  Only the benchmark uses them."""
from __future__ import annotations

import ctypes
import os

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libscprobe.so")


def _lib():
    lib = ctypes.CDLL(_LIB)
    for f in (lib.scprobe_fma, lib.scprobe_lds, lib.scprobe_read):
        f.restype = ctypes.c_int
    lib.scprobe_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.scprobe_fma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.scprobe_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


def _time(launch, reps: int) -> float:
    """Milliseconds per launch (one untimed launch first)."""
    import torch
    launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        launch()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def fma_rate(cus: int, waves_per_simd: int, literal: bool = True, iters: int = 64) -> float:
    """fp32 FMA TFLOP/s of wavefronts issuing independent v_fmac_f32 (literal or VGPR weight),
    waves_per_simd wavefronts on each of the 4 SIMDs of every CU."""
    import torch
    lib = _lib()
    blocks = cus * waves_per_simd
    out = torch.empty(blocks * 256, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.scprobe_fma(out.data_ptr(), 0 if literal else 1, blocks, iters, s)
        if rc != 0:
            raise RuntimeError(f"scprobe_fma failed ({rc})")

    ms = _time(launch, 5)
    flops = 2.0 * 64 * 512 * iters * blocks * 4  # 64 lanes, 512 FMAs per iteration, 4 waves per block
    return flops / (ms * 1e-3) / 1e12


def lds_read_rate(cus: int, words: int = 4, blocks_per_cu: int = 4, iters: int = 64) -> float:
    """LDS read bandwidth in TB/s (ds_read_b32 for words=1, ds_read_b128 for words=4)."""
    import torch
    lib = _lib()
    blocks = cus * blocks_per_cu
    out = torch.empty(blocks * 256, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.scprobe_lds(out.data_ptr(), words, blocks, iters, s)
        if rc != 0:
            raise RuntimeError(f"scprobe_lds failed ({rc})")

    ms = _time(launch, 5)
    nbytes = 64.0 * iters * blocks * 256 * 4 * words  # 64 reads per iteration per lane
    return nbytes / (ms * 1e-3) / 1e12


def read_rate(bufs, blocks: int, reps: int = 20) -> float:
    """HBM read rate in GB/s of a pure read stream over the device tensors ``bufs`` (one per
    launch, rotated: each launch reads one whole buffer), blocks workgroups of 256 threads."""
    import torch
    lib = _lib()
    out = torch.empty(blocks * 256, device=bufs[0].device)
    s = torch.cuda.current_stream().cuda_stream
    n4 = bufs[0].numel() * bufs[0].element_size() // 16
    k = [0]

    def launch():
        b = bufs[k[0] % len(bufs)]
        k[0] += 1
        rc = lib.scprobe_read(b.data_ptr(), n4, out.data_ptr(), blocks, s)
        if rc != 0:
            raise RuntimeError(f"scprobe_read failed ({rc})")

    ms = _time(launch, reps)
    return n4 * 16 / (ms * 1e-3) / 1e9
