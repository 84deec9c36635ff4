"""The entry point that allocates nothing (sparseconv_forward_noalloc), through the C ABI,
against the workspace entry point it stands in for: handles packed with the "Escoin" mapping
keep the padded input in the library's static device array instead of a caller workspace.

Bar: the same kernels on the same inputs, so the outputs must equal the workspace entry
point's bit for bit, and the oracle's within |gpu - oracle| <= 1e-5 * sum|w*x|.  Two calls in
a row, the second with a smaller batch, show that a call does not depend on what the previous
one left in the shared array."""
import numpy as np
import pytest
import torch

import oracle
import sparse_weight_direct_amd as sc
import workloads
from gpu_util import assert_parity

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20  # SC_NOALLOC_SCRATCH_BYTES


def _run(h, L, x, entry):
    N = x.shape[0]
    y = torch.full((N, L.M, L.E, L.F), float("nan"), device="cuda")
    if entry == "noalloc":
        sc.sparseconv_forward_noalloc(h.ptr, x, y, N, L.C, L.H, L.W, L.M, L.R, L.S, L.stride, L.pad)
    else:
        ws = torch.empty(max(h.workspace_size(N), 4) // 4, dtype=torch.float32, device="cuda")
        h.forward(x, y, workspace=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("name,n1,n2", [("mid", 2, 1), ("late", 32, 5), ("first11", 16, 3)])
def test_noalloc_equals_workspace_entry_point(name, n1, n2):
    d = workloads.make(name)
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                  flags=sc.SC_PACK_ESCOIN_MAP)
    assert h.info()["mapping"] == sc.MAPPING_ESCOIN
    for n in (n1, n2):  # the second call is smaller than the first
        assert 0 < h.workspace_size(n) <= SCRATCH_BYTES
        xh = np.ascontiguousarray(d["x"][:n])
        x = torch.from_numpy(xh).cuda()
        y = _run(h, L, x, "noalloc")
        ref = _run(h, L, x, "workspace")
        np.testing.assert_array_equal(y.view(np.uint32), ref.view(np.uint32))
        r = oracle.reference(xh, d["w"], d["mask"], L.stride, L.pad)
        assert_parity(y, r["y64"], r["mag"], f"noalloc {name} N={n}")


def test_noalloc_rejects_a_batch_beyond_the_static_array():
    """The 112x112, 128-channel layer's padded input is 6.65 MB per image: 4 images fit the
    32 MiB array, 6 do not; the call is rejected before any launch and the output is left as
    it was."""
    d = workloads.make("imb95", n_override=6)
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                  flags=sc.SC_PACK_ESCOIN_MAP)
    assert h.workspace_size(4) <= SCRATCH_BYTES < h.workspace_size(6)
    x = torch.from_numpy(d["x"]).cuda()
    y = torch.full((6, L.M, L.E, L.F), 7.0, device="cuda")
    with pytest.raises(sc.SparseConvError) as e:
        sc.sparseconv_forward_noalloc(h.ptr, x, y, 6, L.C, L.H, L.W, L.M, L.R, L.S, L.stride, L.pad)
    assert e.value.status == sc.SC_EUNSUPPORTED and "static" in str(e.value)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    y4 = _run(h, L, x[:4], "noalloc")
    r = oracle.reference(d["x"][:4], d["w"], d["mask"], L.stride, L.pad)
    assert_parity(y4, r["y64"], r["mag"], "noalloc imb95 N=4")


def test_noalloc_on_a_handle_that_needs_no_workspace():
    """Handles of the other mappings need no workspace: the call is the plain forward."""
    d = workloads.make("mid")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"])
    x = torch.from_numpy(d["x"]).cuda()
    y = _run(h, L, x, "noalloc")
    ref = h.forward(x).cpu().numpy()
    np.testing.assert_array_equal(y.view(np.uint32), ref.view(np.uint32))
