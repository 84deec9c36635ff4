"""GPU parity of the second mapping (SC_PACK_ESCOIN_MAP: the "Escoin" dataflow with a
pad_in kernel, one output channel per workgroup, weights stationary in LDS, input through
the caches) against the oracle, through sparseconv_forward_workspace.  Same bar as the
default mapping: |gpu - oracle| <= 1e-5 * sum|w*x|, exact +0 where no term contributes."""
import numpy as np
import pytest
import torch

import oracle
import sparse_weight_direct_amd as sc
import workloads
from gpu_util import MAX_FORWARD_MS, assert_layer_parity, assert_parity

pytestmark = pytest.mark.gpu


def _escoin_handle(w, mask, H, W, stride, pad, **kw):
    M, C, R, S = w.shape
    return sc.Handle(M, C, R, S, H, W, stride, pad, values=w, mask=mask, flags=sc.SC_PACK_ESCOIN_MAP, **kw)


def gpu_escoin(x, h, poison=True):
    N = x.shape[0]
    g = h.geom
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out = torch.full((N, g["M"], h.E, h.F), float("nan") if poison else 0.0, dtype=torch.float32, device="cuda")
    ws = torch.full((max(1, h.workspace_size(N)) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    h.forward(xd, out, workspace=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    h.forward(xd, out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) < MAX_FORWARD_MS
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "mid", "late", "first11", "pw1x1"])
def test_layer_full_parity_escoin(name):
    d = workloads.make(name)
    L = d["layer"]
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    h = _escoin_handle(d["w"], d["mask"], L.H, L.W, L.stride, L.pad)
    assert h.info()["mapping"] == 1
    assert_parity(gpu_escoin(d["x"], h), r["y64"], r["mag"], name + " escoin")


@pytest.mark.parametrize("name", ["imb80", "imb90", "imb95", "imb99"])
def test_full_size_escoin(name):
    """Full-size layers through the "Escoin" mapping against the oracle on every output
   ."""
    d = workloads.make(name)
    L = d["layer"]
    h = _escoin_handle(d["w"], d["mask"], L.H, L.W, L.stride, L.pad)
    y = gpu_escoin(d["x"], h)
    assert_layer_parity(name, y, name + " escoin")


def _cases(count, seed0):
    rng = np.random.default_rng(seed0)
    out = []
    for i in range(count):
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        st, p = int(rng.integers(1, 5)), int(rng.integers(0, 3))
        H = int(rng.integers(max(1, R - 2 * p), 40))
        W = int(rng.integers(max(1, S - 2 * p), 40))
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 9)), H, W, int(rng.integers(1, 40)), R, S, st, p,
                    [0.9, 0.5, 0.1, 0.0, 1.0][i % 5], 5000 + i))
    return out


@pytest.mark.parametrize("c", _cases(16, 11), ids=lambda c: "N{}C{}H{}W{}M{}R{}S{}st{}p{}k{}".format(*c[:10]))
def test_random_shapes_escoin(c):
    N, C, H, W, M, R, S, st, p, keep, seed = c
    d = workloads.make_custom(N, C, H, W, M, R, S, st, p, keep, seed)
    r = oracle.reference(d["x"], d["w"], d["mask"], st, p)
    h = _escoin_handle(d["w"], d["mask"], H, W, st, p)
    assert_parity(gpu_escoin(d["x"], h), r["y64"], r["mag"], "escoin")


def test_rows_longer_than_the_lds_buffer():
    """Dense rows of 512 * 9 = 4608 entries are walked in two LDS passes."""
    d = workloads.make_custom(1, 512, 6, 6, 3, 3, 3, 1, 1, 1.0, 77)
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, 1)
    h = _escoin_handle(d["w"], d["mask"], 6, 6, 1, 1)
    assert h.info()["max_wave_nnz"] == 4608
    assert_parity(gpu_escoin(d["x"], h), r["y64"], r["mag"], "escoin long rows")


def test_empty_rows_and_all_zero_weights_escoin():
    d = workloads.make_custom(2, 8, 12, 12, 40, 3, 3, 1, 1, 0.2, 21)
    mask = d["mask"].copy()
    mask[::3] = 0
    y = gpu_escoin(d["x"], _escoin_handle(d["w"], mask, 12, 12, 1, 1))
    assert np.all(y[:, ::3] == 0) and not np.signbit(y[:, ::3]).any()
    y0 = gpu_escoin(d["x"], _escoin_handle(d["w"], np.zeros_like(mask), 12, 12, 1, 1))
    assert np.all(y0 == 0) and not np.signbit(y0).any()


def test_workspace_errors_and_default_handles():
    d = workloads.make("tiny")
    L = d["layer"]
    h = _escoin_handle(d["w"], d["mask"], L.H, L.W, L.stride, L.pad)
    xd = torch.from_numpy(d["x"]).cuda()
    out = torch.zeros((L.N, L.M, L.E, L.F), device="cuda")
    with pytest.raises(sc.SparseConvError) as e:
        h.forward(xd, out)  # no workspace
    assert e.value.status == sc.SC_EINVAL
    need = h.workspace_size(L.N)
    small = torch.zeros(need // 4 - 1, device="cuda")
    with pytest.raises(sc.SparseConvError) as e:
        h.forward(xd, out, workspace=small)
    assert e.value.status == sc.SC_EINVAL and "workspace" in str(e.value)
    big = torch.zeros(need // 4 + L.N * L.C * L.H * L.W, device="cuda")
    with pytest.raises(sc.SparseConvError) as e:  # workspace overlapping the input
        sc.sparseconv_forward_workspace(h.ptr, big[:L.N * L.C * L.H * L.W], out, L.N, L.C, L.H, L.W, L.M, L.R, L.S,
                                        L.stride, L.pad, big.data_ptr() + 4 * 16, need)
    assert e.value.status == sc.SC_EINVAL
    # a default-mapping handle runs through the workspace entry point unchanged
    hd = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"])
    assert hd.workspace_size(L.N) == 0
    y1 = hd.forward(xd).cpu().numpy()
    y2 = torch.zeros_like(out)
    sc.sparseconv_forward_workspace(hd.ptr, xd, y2, L.N, L.C, L.H, L.W, L.M, L.R, L.S, L.stride, L.pad, None, 0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y1.view(np.uint32), y2.cpu().numpy().view(np.uint32))
