"""CPU oracle for sparse direct convolution -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The GPU library never does, and this package never imports the GPU
library: the two share no code (only the seeded generators in ``workloads.py`` feed both).

The arithmetic lives in ``oracle.c`` (plain C, double accumulation); this file only
compiles it with gcc, loads it with ctypes and marshals numpy arrays.  Rounding the double
result to fp32 happens here, once, with numpy's round-to-nearest-even cast.

Every function is pinned by the CPU tests in ``tests/test_oracle_pins.py`` against
brute force, torch's float64 conv2d, closed forms and the size/offset invariants printed in
the pages (Tuteja et al., Sec. 3-4; "Escoin", CSR and weight-stretching sections).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP over output planes)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    lib.oracle_out_size.restype = _i64
    lib.oracle_out_size.argtypes = [_i64, _i64, _i64, _i64]
    lib.oracle_count_kept.restype = _i64
    lib.oracle_count_kept.argtypes = [_p, _p, _i64]
    lib.oracle_csr_from_dense.restype = None
    lib.oracle_csr_from_dense.argtypes = [_i32, _i32, _p, _p, _p, _p, _p]
    lib.oracle_stretch.restype = None
    lib.oracle_stretch.argtypes = [_i32] * 5 + [_i64, _p, _p]
    lib.oracle_conv_def.restype = None
    lib.oracle_conv_def.argtypes = [_i32] * 9 + [_p] * 5
    lib.oracle_conv_csr.restype = None
    lib.oracle_conv_csr.argtypes = [_i32] * 9 + [_p] * 6 + [_i32]
    lib.oracle_conv_csr_planes.restype = None
    lib.oracle_conv_csr_planes.argtypes = [_i32] * 9 + [_p] * 4 + [_i64, _p, _p, _p, _i32]
    lib.oracle_fp16_bits.restype = ctypes.c_uint16
    lib.oracle_fp16_bits.argtypes = [ctypes.c_float]
    lib.oracle_fp16_value.restype = ctypes.c_double
    lib.oracle_fp16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_pack_word.restype = ctypes.c_uint32
    lib.oracle_pack_word.argtypes = [ctypes.c_float, _i32, _i32, _i32]
    lib.oracle_unpack_word.restype = None
    lib.oracle_unpack_word.argtypes = [ctypes.c_uint32, _p, _p, _p, _p]
    lib.oracle_words_from_csr.restype = None
    lib.oracle_words_from_csr.argtypes = [_i32, _i32, _i64, _p, _p, _p]
    lib.oracle_csr_from_words.restype = None
    lib.oracle_csr_from_words.argtypes = [_i32, _i32, _i64, _p, _p, _p]
    lib.oracle_max_threads.restype = _i32
    lib.oracle_max_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(_LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def out_size(n_in: int, pad: int, k: int, stride: int) -> int:
    """Output extent along one axis (Tuteja et al., Sec. 3 Eq. (2)); 0 if empty."""
    return int(_load().oracle_out_size(n_in, pad, k, stride))


def csr_from_dense(w: np.ndarray, mask: np.ndarray | None = None):
    """CSR (rowptr, colidx, value) of the M x CRS filter matrix ("Escoin", CSR format).

    With a mask, exactly its non-zero bits are the stored entries; without, every w != 0.0f.
    """
    w = _c(w, np.float32)
    M = w.shape[0]
    crs = int(np.prod(w.shape[1:])) if w.ndim > 1 else 1
    mask = None if mask is None else _c(mask, np.uint8)
    if mask is not None and mask.size != w.size:
        raise ValueError("mask size differs from weight size")
    lib = _load()
    nnz = int(lib.oracle_count_kept(_ptr(w), _ptr(mask), w.size))
    rowptr = np.zeros(M + 1, np.int32)
    colidx = np.zeros(nnz, np.int32)
    value = np.zeros(nnz, np.float32)
    lib.oracle_csr_from_dense(M, crs, _ptr(w), _ptr(mask), _ptr(rowptr), _ptr(colidx), _ptr(value))
    return rowptr, colidx, value


def stretch(colidx: np.ndarray, C: int, R: int, S: int, H: int, W: int) -> np.ndarray:
    """Input offsets f(c,r,s) = (c*H + r)*W + s of each column ("Escoin", weight stretching)."""
    colidx = _c(colidx, np.int32)
    off = np.zeros(colidx.size, np.uint32)
    _load().oracle_stretch(C, R, S, H, W, colidx.size, _ptr(colidx), _ptr(off))
    return off


def conv_def(x: np.ndarray, w: np.ndarray, mask: np.ndarray | None, stride: int, pad: int):
    """7-loop definitional convolution skipping non-stored weights; returns (y64, mag)."""
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    mask = None if mask is None else _c(mask, np.uint8)
    N, C, H, W = x.shape
    M, C2, R, S = w.shape
    if C2 != C:
        raise ValueError("channel mismatch")
    E, F = out_size(H, pad, R, stride), out_size(W, pad, S, stride)
    y = np.zeros((N, M, E, F), np.float64)
    mag = np.zeros((N, M, E, F), np.float64)
    _load().oracle_conv_def(N, C, H, W, M, R, S, stride, pad, _ptr(x), _ptr(w), _ptr(mask),
                            _ptr(y), _ptr(mag))
    return y, mag


def conv_csr(x: np.ndarray, rowptr, colidx, value, M: int, R: int, S: int, stride: int,
             pad: int, nthreads: int = 0):
    """List-form convolution over a CSR filter matrix; returns (y64, mag)."""
    x = _c(x, np.float32)
    rowptr, colidx, value = _c(rowptr, np.int32), _c(colidx, np.int32), _c(value, np.float32)
    N, C, H, W = x.shape
    E, F = out_size(H, pad, R, stride), out_size(W, pad, S, stride)
    y = np.zeros((N, M, E, F), np.float64)
    mag = np.zeros((N, M, E, F), np.float64)
    _load().oracle_conv_csr(N, C, H, W, M, R, S, stride, pad, _ptr(x), _ptr(rowptr),
                            _ptr(colidx), _ptr(value), _ptr(y), _ptr(mag), nthreads)
    return y, mag


def conv_csr_planes(x: np.ndarray, rowptr, colidx, value, M: int, R: int, S: int, stride: int,
                    pad: int, planes, nthreads: int = 0):
    """List-form convolution of selected (n, m) planes (ids n*M + m); returns (y64, mag)
    of shape (len(planes), E, F)."""
    x = _c(x, np.float32)
    rowptr, colidx, value = _c(rowptr, np.int32), _c(colidx, np.int32), _c(value, np.float32)
    planes = _c(planes, np.int64)
    N, C, H, W = x.shape
    E, F = out_size(H, pad, R, stride), out_size(W, pad, S, stride)
    y = np.zeros((planes.size, E, F), np.float64)
    mag = np.zeros((planes.size, E, F), np.float64)
    _load().oracle_conv_csr_planes(N, C, H, W, M, R, S, stride, pad, _ptr(x), _ptr(rowptr),
                                   _ptr(colidx), _ptr(value), planes.size, _ptr(planes),
                                   _ptr(y), _ptr(mag), nthreads)
    return y, mag


def to_fp32(y64: np.ndarray) -> np.ndarray:
    """Round the double result once to fp32 (round to nearest even)."""
    return y64.astype(np.float32)


def reference(x: np.ndarray, w: np.ndarray, mask: np.ndarray | None, stride: int, pad: int,
              nthreads: int = 0):
    """Full oracle result for a dense(+mask) layer.

    Returns a dict: ``y`` (fp32, rounded once), ``y64``, ``mag`` (sum |w*x|), and the
    canonical packed form ``rowptr``, ``offsets`` (u32 stretched offsets), ``values``.
    """
    M, C, R, S = w.shape
    H, W = x.shape[2], x.shape[3]
    rowptr, colidx, value = csr_from_dense(w, mask)
    y64, mag = conv_csr(x, rowptr, colidx, value, M, R, S, stride, pad, nthreads)
    return {"y": to_fp32(y64), "y64": y64, "mag": mag, "rowptr": rowptr, "colidx": colidx,
            "offsets": stretch(colidx, C, R, S, H, W), "values": value}


def fp16_bits(v: float) -> int:
    """IEEE binary16 bits of an fp32 value, round to nearest even (the packed word's weight)."""
    return int(_load().oracle_fp16_bits(float(np.float32(v))))


def fp16_value(h: int) -> float:
    """Value of binary16 bits, exactly."""
    return float(_load().oracle_fp16_value(int(h)))


def pack_word(v: float, ic: int, px: int, py: int) -> int:
    """[T] Sec. 5.3 / Fig. 4 packed word: fp16 weight << 16 | ic << 8 | px << 4 | py."""
    if not (0 <= ic < 256 and 0 <= px < 16 and 0 <= py < 16):
        raise ValueError("packed word fields out of range (ic < 256, px, py < 16)")
    return int(_load().oracle_pack_word(float(np.float32(v)), ic, px, py))


def unpack_word(wd: int):
    """(value as double, ic, px, py) of a packed word."""
    v = ctypes.c_double()
    ic, px, py = _i32(), _i32(), _i32()
    _load().oracle_unpack_word(int(wd), ctypes.byref(v), ctypes.byref(ic), ctypes.byref(px), ctypes.byref(py))
    return v.value, ic.value, px.value, py.value


def words_from_csr(colidx, value, C: int, R: int, S: int) -> np.ndarray:
    """Packed words of the CSR non-zeros in CSR order.  The word holds C <= 256 input
    channels and R, S <= 16 ([T] Fig. 4 field widths)."""
    if C > 256 or R > 16 or S > 16:
        raise ValueError("the packed word holds C <= 256 and R, S <= 16")
    colidx, value = _c(colidx, np.int32), _c(value, np.float32)
    words = np.zeros(colidx.size, np.uint32)
    _load().oracle_words_from_csr(R, S, colidx.size, _ptr(colidx), _ptr(value), _ptr(words))
    return words


def csr_from_words(words, R: int, S: int):
    """(colidx, value) the packed words describe; values are the fp16 weights in fp32."""
    words = _c(words, np.uint32)
    colidx = np.zeros(words.size, np.int32)
    value = np.zeros(words.size, np.float32)
    _load().oracle_csr_from_words(R, S, words.size, _ptr(words), _ptr(colidx), _ptr(value))
    return colidx, value


def reference_fp16(x: np.ndarray, w: np.ndarray, mask: np.ndarray | None, stride: int, pad: int,
                   nthreads: int = 0):
    """Oracle result for the packed-word form of a layer ([T] Sec. 5.3): the CSR non-zeros
    are encoded as packed words, decoded again, and the list-form convolution runs on the
    decoded (fp16-rounded) weights with double accumulation.  Same dict as ``reference``
    plus ``words``; ``values`` are the fp16-rounded weights."""
    M, C, R, S = w.shape
    H, W = x.shape[2], x.shape[3]
    rowptr, colidx, value = csr_from_dense(w, mask)
    words = words_from_csr(colidx, value, C, R, S)
    colidx16, value16 = csr_from_words(words, R, S)
    y64, mag = conv_csr(x, rowptr, colidx16, value16, M, R, S, stride, pad, nthreads)
    return {"y": to_fp32(y64), "y64": y64, "mag": mag, "rowptr": rowptr, "colidx": colidx16,
            "offsets": stretch(colidx16, C, R, S, H, W), "values": value16, "words": words}


def within_tolerance(y_gpu: np.ndarray, y_ref64: np.ndarray, mag: np.ndarray, rel: float = 1e-5):
    """Boolean array: |y_gpu - y_ref| <= rel * mag per element; where mag == 0 the GPU value
    must be exactly 0.  Comparison in double precision."""
    d = np.abs(y_gpu.astype(np.float64) - y_ref64)
    ok = d <= rel * mag
    zero = mag == 0
    ok[zero] = y_gpu[zero] == 0
    return ok
