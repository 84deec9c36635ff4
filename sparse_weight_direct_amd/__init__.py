"""Python binding of libsparseconv.so (the C ABI in include/sparseconv.h).

Argument marshalling only: every step of packing and of the forward pass runs in the
native library (host C++ for packing, gfx950 HIP kernels for the convolution).  PyTorch is
used for device memory and streams.  There is no fallback: if the library is missing the
import fails, and the forward pass needs a ROCm device.

The functions keep the C names:
    sparseconv_pack, sparseconv_forward, sparseconv_forward_workspace,
    sparseconv_workspace_size, sparseconv_query, sparseconv_export_packed,
    sparseconv_export_words, sparseconv_destroy, sparseconv_last_error
plus ``Handle`` (owns a packed filter bank and destroys it when collected).  The dense
direct baseline is a Handle packed with SC_PACK_ALL_TAPS (every filter tap stored).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# torch first: it ships its own HIP runtime under the same soname (libamdhip64.so.7) as the
# system one this library links; loading torch first makes both use torch's runtime, so
# device pointers and streams from torch are valid here.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparseconv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                      " (or python sparse_weight_direct_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

SC_OK, SC_EINVAL, SC_ESHAPE, SC_ENOMEM, SC_EDEVICE, SC_EUNSUPPORTED = range(6)
SC_WEIGHTS_DENSE, SC_WEIGHTS_CSR = 0, 1
SC_PACK_HOST_ONLY = 1
SC_PACK_ALL_TAPS = 2
SC_PACK_FP16_WORD = 4
SC_PACK_ESCOIN_MAP = 8
SC_PACK_LDS_TILE = 16
MAPPING_LDS_TILE, MAPPING_ESCOIN, MAPPING_BAKED = 0, 1, 2
_STATUS_NAMES = {0: "SC_OK", 1: "SC_EINVAL", 2: "SC_ESHAPE", 3: "SC_ENOMEM", 4: "SC_EDEVICE",
                 5: "SC_EUNSUPPORTED"}

EXPORTED = ("sparseconv_pack", "sparseconv_forward", "sparseconv_forward_workspace", "sparseconv_workspace_size",
            "sparseconv_query", "sparseconv_export_packed", "sparseconv_export_words",
            "sparseconv_export_kernel_source", "sparseconv_launch_info", "sparseconv_device_status",
            "sparseconv_dense_forward", "sparseconv_forward_noalloc", "sparseconv_tune", "sparseconv_destroy",
            "sparseconv_last_error")


class sc_weights(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("values", ctypes.c_void_p), ("colidx", ctypes.c_void_p),
                ("rowptr", ctypes.c_void_p), ("mask", ctypes.c_void_p)]


class sc_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("M", "C", "R", "S", "H", "W", "stride", "pad", "E", "F")] + \
               [("nnz", ctypes.c_int64), ("packed_bytes", ctypes.c_int64), ("device_bytes", ctypes.c_int64)] + \
               [(n, ctypes.c_int32) for n in ("tile_pixels", "rows_per_wave", "row_groups", "chunk_channels",
                                               "lds_bytes", "max_wave_nnz", "waves_per_group",
                                               "pipeline_depth", "step_balance_permille",
                                               "split_pieces", "plan_variants", "entry_bytes", "mapping",
                                               "bake_groups", "bake_splits", "bake_units_per_wg",
                                               "bake_valid_lanes", "bake_pitch", "bake_depth", "bake_vgprs",
                                               "bake_lds_bytes", "bake_variants", "bake_stage",
                                               "bake_chunk_channels", "bake_buffers", "bake_sequential",
                                               "bake_shared_window")] + \
               [("bake_code_bytes", ctypes.c_int64)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class sc_launch(ctypes.Structure):
    _fields_ = [("mapping", ctypes.c_int32), ("variant", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("waves", ctypes.c_int64), ("pre_grid", ctypes.c_int64)] + \
               [(n, ctypes.c_int32) for n in ("block", "lds_bytes", "vgprs", "groups", "splits", "units_per_wg",
                                               "depth", "valid_lanes", "tile_pixels", "rows_per_wave",
                                               "chunk_channels", "quad", "stage")]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_vp, _i32, _u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32
_lib.sparseconv_pack.restype = _i32
_lib.sparseconv_pack.argtypes = [ctypes.POINTER(sc_weights)] + [_i32] * 8 + [_u32, ctypes.POINTER(_vp)]
_lib.sparseconv_forward.restype = _i32
_lib.sparseconv_forward.argtypes = [_vp, _vp, _vp] + [_i32] * 9 + [_vp]
_lib.sparseconv_forward_workspace.restype = _i32
_lib.sparseconv_forward_workspace.argtypes = [_vp, _vp, _vp] + [_i32] * 9 + [_vp, ctypes.c_int64, _vp]
_lib.sparseconv_workspace_size.restype = _i32
_lib.sparseconv_workspace_size.argtypes = [_vp, _i32, ctypes.POINTER(ctypes.c_int64)]
_lib.sparseconv_query.restype = _i32
_lib.sparseconv_query.argtypes = [_vp, ctypes.POINTER(sc_info)]
_lib.sparseconv_export_packed.restype = _i32
_lib.sparseconv_export_packed.argtypes = [_vp, _vp, _vp, _vp]
_lib.sparseconv_export_words.restype = _i32
_lib.sparseconv_export_words.argtypes = [_vp, _vp, _vp]
_lib.sparseconv_export_kernel_source.restype = _i32
_lib.sparseconv_export_kernel_source.argtypes = [_vp, ctypes.c_char_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
_lib.sparseconv_launch_info.restype = _i32
_lib.sparseconv_launch_info.argtypes = [_vp, _i32, ctypes.POINTER(sc_launch)]
_lib.sparseconv_device_status.restype = _i32
_lib.sparseconv_device_status.argtypes = [_vp, ctypes.POINTER(_u32), _i32]
_lib.sparseconv_dense_forward.restype = _i32
_lib.sparseconv_dense_forward.argtypes = [_vp, _vp, _vp] + [_i32] * 9 + [_vp]
_lib.sparseconv_forward_noalloc.restype = _i32
_lib.sparseconv_forward_noalloc.argtypes = [_vp, _vp, _vp] + [_i32] * 9 + [_vp]
_lib.sparseconv_tune.restype = _i32
_lib.sparseconv_tune.argtypes = [_vp, _vp, _vp] + [_i32] * 10 + [_vp, ctypes.POINTER(_i32)]
_lib.sparseconv_destroy.restype = None
_lib.sparseconv_destroy.argtypes = [_vp]
_lib.sparseconv_last_error.restype = ctypes.c_char_p
_lib.sparseconv_last_error.argtypes = []


class SparseConvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS_NAMES.get(status, status)}: {sparseconv_last_error()}")


def _check(status: int, where: str):
    if status != SC_OK:
        raise SparseConvError(status, where)


def _np_ptr(a, dtype):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a, dtype=dtype)
    return arr, arr.ctypes.data_as(_vp)


def _dev_ptr(t):
    """Device pointer of a contiguous fp32 torch tensor (or a raw int address)."""
    if isinstance(t, int):
        return t
    import torch
    if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
        raise ValueError("expected a contiguous float32 tensor on the GPU")
    return t.data_ptr()


_raw_stream = None  # torch's accessor of the current stream's raw handle (by device index)


def _stream_ptr(stream, device=None):
    """The HIP stream handle for ``stream``: a torch stream, a raw handle, or None for the
    current stream of ``device`` (a device index; the current device when None)."""
    global _raw_stream
    if stream is None:
        import torch
        if _raw_stream is None:
            _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
        if _raw_stream:
            return _raw_stream(torch.cuda.current_device() if device is None else device)
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def sparseconv_last_error() -> str:
    return _lib.sparseconv_last_error().decode()


def sparseconv_pack(M, C, R, S, H, W, stride, pad, *, values=None, mask=None, colidx=None, rowptr=None,
                    fmt=None, flags=0) -> int:
    """Pack weights; returns the raw handle address.  Dense: ``values`` (M*C*R*S fp32) and an
    optional ``mask`` (u8).  CSR: ``values``, ``colidx``, ``rowptr``."""
    if fmt is None:
        fmt = SC_WEIGHTS_CSR if rowptr is not None else SC_WEIGHTS_DENSE
    v, vp = _np_ptr(values, np.float32)
    m, mp = _np_ptr(mask, np.uint8)
    ci, cp = _np_ptr(colidx, np.int32)
    rp, rpp = _np_ptr(rowptr, np.int32)
    w = sc_weights(fmt, vp, cp, rpp, mp)
    out = _vp()
    st = _lib.sparseconv_pack(ctypes.byref(w), M, C, R, S, H, W, stride, pad, flags, ctypes.byref(out))
    del v, m, ci, rp
    _check(st, "sparseconv_pack")
    return out.value


def sparseconv_forward(handle: int, x, y, N, C, H, W, M, R, S, stride, pad, stream=None) -> None:
    _check(_lib.sparseconv_forward(handle, _dev_ptr(x), _dev_ptr(y), N, C, H, W, M, R, S, stride, pad,
                                   _stream_ptr(stream)), "sparseconv_forward")


def sparseconv_forward_workspace(handle: int, x, y, N, C, H, W, M, R, S, stride, pad, workspace, workspace_bytes,
                                 stream=None) -> None:
    """``workspace``: a device tensor (any dtype, contiguous), a raw address, or None."""
    if workspace is None:
        wp = None
    elif isinstance(workspace, int):
        wp = workspace
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the GPU")
        wp = workspace.data_ptr()
    _check(_lib.sparseconv_forward_workspace(handle, _dev_ptr(x), _dev_ptr(y), N, C, H, W, M, R, S, stride, pad, wp,
                                             int(workspace_bytes), _stream_ptr(stream)),
           "sparseconv_forward_workspace")


def sparseconv_forward_noalloc(handle: int, x, y, N, C, H, W, M, R, S, stride, pad, stream=None) -> None:
    _check(_lib.sparseconv_forward_noalloc(handle, _dev_ptr(x), _dev_ptr(y), N, C, H, W, M, R, S, stride, pad,
                                           _stream_ptr(stream)), "sparseconv_forward_noalloc")


def sparseconv_tune(handle: int, x, y, N, C, H, W, M, R, S, stride, pad, reps=5, stream=None) -> int:
    """Time the handle's kernels for N images on (x, y); later forwards of N use the fastest,
    whose index is returned."""
    chosen = _i32(-1)
    _check(_lib.sparseconv_tune(handle, _dev_ptr(x), _dev_ptr(y), N, C, H, W, M, R, S, stride, pad, reps,
                                _stream_ptr(stream), ctypes.byref(chosen)), "sparseconv_tune")
    return chosen.value


def sparseconv_workspace_size(handle: int, N: int) -> int:
    b = ctypes.c_int64()
    _check(_lib.sparseconv_workspace_size(handle, N, ctypes.byref(b)), "sparseconv_workspace_size")
    return b.value


def sparseconv_query(handle: int) -> dict:
    info = sc_info()
    _check(_lib.sparseconv_query(handle, ctypes.byref(info)), "sparseconv_query")
    return info.as_dict()


def sparseconv_export_packed(handle: int):
    """Canonical (rowptr, offsets, values) as numpy arrays."""
    info = sparseconv_query(handle)
    rowptr = np.zeros(info["M"] + 1, np.int32)
    off = np.zeros(info["nnz"], np.uint32)
    val = np.zeros(info["nnz"], np.float32)
    _check(_lib.sparseconv_export_packed(handle, rowptr.ctypes.data_as(_vp), off.ctypes.data_as(_vp),
                                         val.ctypes.data_as(_vp)), "sparseconv_export_packed")
    return rowptr, off, val


def sparseconv_export_words(handle: int):
    """(rowptr, words): the 32-bit packed words of an SC_PACK_FP16_WORD handle."""
    info = sparseconv_query(handle)
    rowptr = np.zeros(info["M"] + 1, np.int32)
    words = np.zeros(info["nnz"], np.uint32)
    _check(_lib.sparseconv_export_words(handle, rowptr.ctypes.data_as(_vp), words.ctypes.data_as(_vp)),
           "sparseconv_export_words")
    return rowptr, words


def sparseconv_export_kernel_source(handle: int) -> str:
    """Assembly of the handle's weights-in-code kernel."""
    n = ctypes.c_int64()
    _check(_lib.sparseconv_export_kernel_source(handle, None, 0, ctypes.byref(n)), "sparseconv_export_kernel_source")
    buf = ctypes.create_string_buffer(n.value)
    _check(_lib.sparseconv_export_kernel_source(handle, buf, n.value, ctypes.byref(n)),
           "sparseconv_export_kernel_source")
    return buf.value.decode()


def sparseconv_launch_info(handle: int, N: int) -> dict:
    """The launch a forward of N images makes (mapping, plan variant, grid, ...)."""
    out = sc_launch()
    _check(_lib.sparseconv_launch_info(handle, N, ctypes.byref(out)), "sparseconv_launch_info")
    return out.as_dict()


def sparseconv_device_status(handle: int, clear: bool = False) -> int:
    """The handle's device status word (bit 0: a bounded wait in the LDS-tile kernel gave up)."""
    st = _u32()
    _check(_lib.sparseconv_device_status(handle, ctypes.byref(st), 1 if clear else 0), "sparseconv_device_status")
    return st.value


def sparseconv_dense_forward(w, x, y, N, C, H, W, M, R, S, stride, pad, stream=None) -> None:
    """Dense direct baseline: ``w`` a device tensor (or address) of M*C*R*S fp32 weights."""
    _check(_lib.sparseconv_dense_forward(_dev_ptr(w), _dev_ptr(x), _dev_ptr(y), N, C, H, W, M, R, S, stride, pad,
                                         _stream_ptr(stream)), "sparseconv_dense_forward")


def dense_forward(w, x, out, stride: int, pad: int, stream=None):
    """Dense direct convolution of x (N, C, H, W) with every tap of w (M, C, R, S), both float32
    CUDA tensors, into out (N, M, E, F)."""
    if w.dim() != 4 or x.dim() != 4 or out.dim() != 4:
        raise ValueError("w, x and out must be 4-d tensors")
    M, C, R, S = (int(v) for v in w.shape)
    N, Cx, H, W = (int(v) for v in x.shape)
    if Cx != C:
        raise ValueError(f"input has {Cx} channels, the weights {C}")
    # the library writes N*M*E*F outputs: out must have exactly that shape
    E, F = (H + 2 * pad - R) // stride + 1, (W + 2 * pad - S) // stride + 1
    if tuple(out.shape) != (N, M, E, F):
        raise ValueError(f"output shape {tuple(out.shape)} is not ({N}, {M}, {E}, {F})")
    sparseconv_dense_forward(w, x, out, N, C, H, W, M, R, S, stride, pad, stream)
    return out


def sparseconv_destroy(handle) -> None:
    _lib.sparseconv_destroy(handle)


class Handle:
    """A packed filter bank for one layer geometry; destroyed with the object."""

    def __init__(self, M, C, R, S, H, W, stride, pad, *, values=None, mask=None, colidx=None,
                 rowptr=None, flags=0):
        self.geom = dict(M=M, C=C, R=R, S=S, H=H, W=W, stride=stride, pad=pad)
        self.ptr = sparseconv_pack(M, C, R, S, H, W, stride, pad, values=values, mask=mask,
                                   colidx=colidx, rowptr=rowptr, flags=flags)
        info = sparseconv_query(self.ptr)  # output extent as the library computes it
        self.E, self.F = info["E"], info["F"]
        # what forward compares and passes on every call
        self._chw, self._mef = (C, H, W), (M, self.E, self.F)
        self._dims = (C, H, W, M, R, S, stride, pad)

    @classmethod
    def from_dense(cls, w: np.ndarray, H: int, W: int, stride: int, pad: int, mask=None, flags=0):
        M, C, R, S = w.shape
        return cls(M, C, R, S, H, W, stride, pad, values=w, mask=mask, flags=flags)

    def info(self) -> dict:
        return sparseconv_query(self.ptr)

    def export(self):
        return sparseconv_export_packed(self.ptr)

    def export_words(self):
        return sparseconv_export_words(self.ptr)

    def kernel_source(self) -> str:
        return sparseconv_export_kernel_source(self.ptr)

    def launch_info(self, N: int) -> dict:
        return sparseconv_launch_info(self.ptr, N)

    def device_status(self, clear: bool = False) -> int:
        return sparseconv_device_status(self.ptr, clear)

    def workspace_size(self, N: int) -> int:
        return sparseconv_workspace_size(self.ptr, N)

    def forward(self, x, out=None, stream=None, workspace=None):
        """x: (N, C, H, W) float32 CUDA tensor; returns out (N, M, E, F).  With ``workspace``
        (a device tensor of at least workspace_size(N) bytes) the workspace entry point is
        used; handles packed with SC_PACK_ESCOIN_MAP need one."""
        import torch
        g = self.geom
        shp = x.shape
        if len(shp) != 4 or shp[1:] != self._chw:
            raise ValueError(f"input shape {tuple(shp)} is not (N, {g['C']}, {g['H']}, {g['W']})")
        N = shp[0]
        if out is None:
            out = torch.empty((N,) + self._mef, dtype=torch.float32, device=x.device)
        elif out.shape[1:] != self._mef or out.shape[0] != N:
            raise ValueError(f"output shape {tuple(out.shape)} is not ({N}, {g['M']}, {self.E}, {self.F})")
        for name, t in (("input", x), ("output", out)):
            if t.dtype is not torch.float32 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous float32 tensor on the GPU")
        if workspace is None:
            # arguments checked above: straight to the library
            _check(_lib.sparseconv_forward(self.ptr, x.data_ptr(), out.data_ptr(), N, *self._dims,
                                           _stream_ptr(stream, x.get_device())), "sparseconv_forward")
        else:
            sparseconv_forward_workspace(self.ptr, x, out, N, g["C"], g["H"], g["W"], g["M"], g["R"], g["S"],
                                         g["stride"], g["pad"], workspace,
                                         workspace.numel() * workspace.element_size(), stream)
        return out

    def tune(self, x, out=None, reps: int = 5, stream=None) -> int:
        """Choose by measurement the kernel forwards of x.shape[0] images launch (see
        sparseconv_tune); returns its index.  out receives the convolution."""
        import torch
        g = self.geom
        if x.dim() != 4 or tuple(x.shape[1:]) != (g["C"], g["H"], g["W"]):
            raise ValueError(f"input shape {tuple(x.shape)} is not (N, {g['C']}, {g['H']}, {g['W']})")
        N = x.shape[0]
        if out is None:
            out = torch.empty((N, g["M"], self.E, self.F), dtype=torch.float32, device=x.device)
        elif tuple(out.shape) != (N, g["M"], self.E, self.F):
            raise ValueError(f"output shape {tuple(out.shape)} is not ({N}, {g['M']}, {self.E}, {self.F})")
        return sparseconv_tune(self.ptr, x, out, N, g["C"], g["H"], g["W"], g["M"], g["R"], g["S"], g["stride"],
                               g["pad"], reps, stream)

    def close(self):
        if getattr(self, "ptr", None):
            sparseconv_destroy(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
