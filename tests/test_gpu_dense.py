"""GPU parity of the dense direct baseline (sparseconv_dense_forward): every filter tap of a
dense weight tensor on the device, checked against the oracle with every weight kept (0%
sparsity) on every output element.

Bar: |gpu - oracle| <= 1e-5 * sum|w*x| per output element, exact +0 where no term
contributes.  The kernel sums per output over filter rows, then input channels, then filter
columns, an order the oracle does not share, so agreement is to rounding."""
import numpy as np
import pytest
import torch

import oracle
import sparse_weight_direct_amd as sc
import workloads
from gpu_util import assert_parity

pytestmark = pytest.mark.gpu


def dense_gpu(x, w, stride, pad, poison=True):
    N, C, H, W = x.shape
    M, _, R, S = w.shape
    E, F = (H + 2 * pad - R) // stride + 1, (W + 2 * pad - S) // stride + 1
    wd = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).cuda()
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    out = torch.full((N, M, E, F), float("nan") if poison else 0.0, device="cuda")
    sc.dense_forward(wd, xd, out, stride, pad)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(x, w, stride, pad, what):
    r = oracle.reference(x, w, None if np.all(w != 0) else np.ones(w.shape, np.uint8), stride, pad)
    y = dense_gpu(x, w, stride, pad)
    assert_parity(y, r["y64"], r["mag"], what)
    return y


@pytest.mark.parametrize("name", ["tiny", "mid", "late", "first11", "pw1x1"])
def test_workload_layers_every_tap(name):
    """The workload layers with every tap kept (0% sparsity), full batch."""
    d = workloads.make(name)
    L = d["layer"]
    _check(d["x"], d["w"], L.stride, L.pad, "dense " + name)


def test_full_size_112x112_every_output():
    """The 112x112, 128 -> 128 channel, 3x3 layer at its full batch of 8 with every tap kept:
    the launch the benchmark times, every output against the oracle."""
    d = workloads.make("imb95")
    L = d["layer"]
    _check(d["x"], d["w"], L.stride, L.pad, "dense 112x112")


def _cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        R, S = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        st, pad = int(rng.integers(1, 5)), int(rng.integers(0, 4))
        H = int(rng.integers(max(1, R - 2 * pad), 40))
        W = int(rng.integers(max(1, S - 2 * pad), 40))
        N, C = int(rng.integers(1, 4)), int(rng.choice([1, 3, 8, 21]))
        M = int(rng.choice([1, 5, 16, 17, 33, 70]))
        E, F = (H + 2 * pad - R) // st + 1, (W + 2 * pad - S) // st + 1
        if C * M * R * S * N * E * F > 3e7:
            continue
        out.append((N, C, H, W, M, R, S, st, pad, seed * 1000 + len(out)))
    return out


def test_random_shapes():
    """80 seeded shapes: filters 1..11 in each axis (every column-pass width, partial last
    passes), stride 1..4, pad 0..3, channel counts that leave a partial last channel group,
    position counts that leave a ragged last tile; failures listed together."""
    failures = []
    for c in _cases(80, 4242):
        N, C, H, W, M, R, S, st, pad, seed = c
        rng = np.random.default_rng(seed)
        x = rng.uniform(-1, 1, (N, C, H, W)).astype(np.float32)
        w = rng.uniform(-1, 1, (M, C, R, S)).astype(np.float32)
        r = oracle.reference(x, w, np.ones(w.shape, np.uint8), st, pad)
        y = dense_gpu(x, w, st, pad)
        ok = np.isfinite(y) & oracle.within_tolerance(y, r["y64"], r["mag"], 1e-5)
        if not ok.all():
            failures.append((c, int((~ok).sum())))
    assert not failures, failures[:5]


def test_zero_weights_and_padding_only_windows_give_plus_zero():
    """Zero weights contribute exact +0, and outputs whose window lies wholly in the padding
    are +0 (no term is evaluated outside the image)."""
    rng = np.random.default_rng(9)
    x = rng.uniform(-1, 1, (2, 3, 5, 6)).astype(np.float32)
    w = np.zeros((7, 3, 3, 3), np.float32)
    y = dense_gpu(x, w, 1, 1)
    assert np.all(y == 0) and not np.signbit(y).any()
    w = rng.uniform(-1, 1, (4, 3, 2, 2)).astype(np.float32)
    y = _check(x, w, 3, 3, "padding-only windows")
    # stride 3, pad 3: output row 0 reads input rows -3..-2, all padding
    assert np.all(y[:, :, 0, :] == 0) and not np.signbit(y[:, :, 0, :]).any()


def test_agrees_with_a_handle_holding_every_tap():
    """The dense entry point and a packed handle with every tap (SC_PACK_ALL_TAPS) compute the
    same sums in different orders: both within the oracle's tolerance and close to each other."""
    d = workloads.make("mid")
    L = d["layer"]
    w = d["w"]
    r = oracle.reference(d["x"], w, np.ones(w.shape, np.uint8), L.stride, L.pad)
    y = dense_gpu(d["x"], w, L.stride, L.pad)
    h = sc.Handle.from_dense(w, L.H, L.W, L.stride, L.pad, flags=sc.SC_PACK_ALL_TAPS)
    xd = torch.from_numpy(d["x"]).cuda()
    y2 = h.forward(xd).cpu().numpy()
    assert_parity(y, r["y64"], r["mag"], "dense entry point")
    assert_parity(y2, r["y64"], r["mag"], "all-taps handle")
    assert np.all(np.abs(y - y2) <= 2e-5 * r["mag"])


def test_stream_and_graph_replay():
    """Launches on a side stream and replays from a HIP graph equal the eager result bit for
    bit (the entry point allocates nothing and records one kernel)."""
    d = workloads.make("mid")
    L = d["layer"]
    wd = torch.from_numpy(d["w"]).cuda()
    x = torch.from_numpy(d["x"]).cuda()
    y = torch.empty((L.N, L.M, L.E, L.F), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sc.dense_forward(wd, x, y, L.stride, L.pad, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = y.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sc.dense_forward(wd, x, y, L.stride, L.pad)
    for _ in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), eager.view(np.uint32))
        torch.ones(1000, device="cuda").sum()


def test_errors_before_launch():
    d = workloads.make("tiny")
    L = d["layer"]
    wd = torch.from_numpy(d["w"]).cuda()
    x = torch.from_numpy(d["x"]).cuda()
    y = torch.zeros((L.N, L.M, L.E, L.F), device="cuda")
    with pytest.raises(sc.SparseConvError) as e:  # weights overlap the output
        sc.sparseconv_dense_forward(y.data_ptr(), x, y, L.N, L.C, L.H, L.W, L.M, L.R, L.S, L.stride, L.pad)
    assert e.value.status == sc.SC_EINVAL
    with pytest.raises(sc.SparseConvError) as e:  # misaligned input
        sc.sparseconv_dense_forward(wd, x.data_ptr() + 2, y, L.N, L.C, L.H, L.W, L.M, L.R, L.S, L.stride, L.pad)
    assert e.value.status == sc.SC_EINVAL
    with pytest.raises(ValueError):  # output of the wrong extent, caught by the binding
        sc.dense_forward(wd, x, torch.zeros((L.N, L.M, L.E - 1, L.F), device="cuda"), L.stride, L.pad)
