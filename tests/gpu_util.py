"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare with
the oracle element by element (|gpu - oracle| <= 1e-5 * sum|w*x|, exact zero where that
sum is zero)."""
import numpy as np
import torch

import oracle
import sparse_weight_direct_amd as sc

REL_TOL = 1e-5


# Every wait inside the kernel is bounded (about 0.1 s of spinning before it gives up), so a
# synchronisation mistake can leave results right and only make the forward slow.  Each
# forward here is therefore also timed: none of the test layers takes a millisecond.
MAX_FORWARD_MS = 100.0


def gpu_sparse(x, w, mask, stride, pad, handle=None, poison=True, stream=None, flags=0):
    N, C, H, W = x.shape
    M, _, R, S = w.shape
    if handle is None:
        handle = sc.Handle(M, C, R, S, H, W, stride, pad, values=w, mask=mask, flags=flags)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out = torch.full((N, M, handle.E, handle.F), float("nan") if poison else 0.0, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream() if stream is None else stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    handle.forward(xd, out, stream=stream)  # the first launch of a kernel also loads it
    e0.record(s)
    handle.forward(xd, out, stream=stream)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert ms < MAX_FORWARD_MS, f"forward took {ms:.1f} ms: a bounded wait in the kernel timed out"
    assert handle.device_status() == 0, "a bounded wait in the kernel gave up (device status word)"
    return out.cpu().numpy(), handle


def gpu_all_taps(x, w_masked, stride, pad):
    """A handle storing every filter tap (SC_PACK_ALL_TAPS), zeros included."""
    N, C, H, W = x.shape
    h = sc.Handle.from_dense(np.ascontiguousarray(w_masked), H, W, stride, pad, flags=sc.SC_PACK_ALL_TAPS)
    y, _ = gpu_sparse(x, w_masked, None, stride, pad, handle=h)
    return y


def assert_parity(y_gpu, y64, mag, what=""):
    assert y_gpu.shape == y64.shape, (y_gpu.shape, y64.shape)
    assert np.isfinite(y_gpu).all(), f"{what}: {int((~np.isfinite(y_gpu)).sum())} outputs not written / not finite"
    ok = oracle.within_tolerance(y_gpu, y64, mag, REL_TOL)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} outside tolerance; first at {i}: gpu={y_gpu[i]!r} "
                             f"oracle={y64[i]!r} mag={mag[i]!r}")


# Oracle results of the full-size workload layers, computed once per test process and shared
# by every kernel variant compared against them (the list form takes well under a second per
# 112x112 batch on 16 threads).
_REF = {}


def layer_check(name):
    """(None, y64, mag) for a named workload: the oracle on every output, shaped (N, M, E, F)."""
    if name not in _REF:
        import workloads
        d = workloads.make(name)
        L = d["layer"]
        r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
        _REF[name] = (None, r["y64"], r["mag"])
    return _REF[name]


def assert_layer_parity(name, y, what):
    """Compare a full-size output with the cached oracle result of the named layer."""
    planes, y64, mag = layer_check(name)
    if planes is None:
        assert_parity(y, y64, mag, what)
    else:
        N, M, E, F = y.shape
        assert np.isfinite(y).all(), f"{what}: outputs not written"
        assert_parity(y.reshape(N * M, E, F)[planes], y64, mag, what)
