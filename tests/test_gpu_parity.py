"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Bar: |gpu - oracle| <= 1e-5 * sum|w*x| per output element (fp32 accumulation in any order
stays well inside it; see the tolerance derivation in the design notes), exact +0 where
no term contributes, and bit-exact results for the closed forms (one non-zero per output:
the GPU's fma(w, x, 0) and the oracle's rounded double product are the same fp32 value)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_weight_direct_amd as sc
import workloads
from gpu_util import assert_layer_parity, assert_parity, gpu_all_taps, gpu_sparse

pytestmark = pytest.mark.gpu

FULL_LAYERS = ["tiny", "mid", "late", "first11", "pw1x1"]
# the two kernels for fp32 weights: the default weights-in-code kernel and the LDS-tile kernel
MAPPINGS = {"baked": 0, "lds_tile": sc.SC_PACK_LDS_TILE}
MAPPING_ID = {"baked": sc.MAPPING_BAKED, "lds_tile": sc.MAPPING_LDS_TILE}


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
@pytest.mark.parametrize("name", FULL_LAYERS)
def test_layer_full_parity(name, mapping):
    d = workloads.make(name)
    L = d["layer"]
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad, flags=MAPPINGS[mapping])
    assert h.launch_info(L.N)["mapping"] == MAPPING_ID[mapping]
    assert_parity(y, r["y64"], r["mag"], f"{name} {mapping}")
    # packed offsets exported by the device handle are the canonical ones, bit for bit
    rowptr, off, val = h.export()
    np.testing.assert_array_equal(rowptr, r["rowptr"])
    np.testing.assert_array_equal(off, r["offsets"])
    np.testing.assert_array_equal(val.view(np.uint32), r["values"].view(np.uint32))


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
@pytest.mark.parametrize("name", ["imb80", "imb90", "imb95", "imb99"])
def test_imbalance_sweep_full_size(name, mapping):
    """The 112x112 batch-8 layers in the benchmark's launch configuration, against the oracle
    on every output; empty channels exact +0."""
    d = workloads.make(name)
    L = d["layer"]
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad, flags=MAPPINGS[mapping])
    assert h.launch_info(L.N)["mapping"] == MAPPING_ID[mapping]
    assert_layer_parity(name, y, f"{name} {mapping}")
    rows = np.diff(oracle.csr_from_dense(d["w"], d["mask"])[0])
    for m in np.flatnonzero(rows == 0):
        assert np.all(y[:, m] == 0) and not np.signbit(y[:, m]).any()


def _tiny_cases(count, seed0):
    rng = np.random.default_rng(seed0)
    keeps = [0.9, 0.5, 0.1, 0.0, 1.0]
    out = []
    for i in range(count):
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        stride, pad = int(rng.integers(1, 5)), int(rng.integers(0, 3))
        H = int(rng.integers(max(1, R - 2 * pad), 40))
        W = int(rng.integers(max(1, S - 2 * pad), 40))
        out.append(dict(N=int(rng.integers(1, 4)), C=int(rng.integers(1, 40)), H=H, W=W,
                        M=int(rng.integers(1, 70)), R=R, S=S, stride=stride, pad=pad, keep=keeps[i % 5],
                        seed=5000 + i))
    return out


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
@pytest.mark.parametrize("c", _tiny_cases(40, 3), ids=lambda c: "N{N}C{C}H{H}W{W}M{M}R{R}S{S}st{stride}p{pad}k{keep}".format(**c))
def test_random_shapes(c, mapping):
    d = workloads.make_custom(c["N"], c["C"], c["H"], c["W"], c["M"], c["R"], c["S"], c["stride"], c["pad"],
                              c["keep"], c["seed"])
    r = oracle.reference(d["x"], d["w"], d["mask"], c["stride"], c["pad"])
    y, _ = gpu_sparse(d["x"], d["w"], d["mask"], c["stride"], c["pad"], flags=MAPPINGS[mapping])
    assert_parity(y, r["y64"], r["mag"], str(c))


@pytest.mark.parametrize("plan", ["K=1,OCW=1", "K=2,OCW=5", "K=7,OCW=9", "K=4,OCW=2,CC=3", "K=8,OCW=5,D=2",
                                  "K=2,OCW=3,D=3", "K=1,OCW=9,D=4,CC=1", "K=16,OCW=3,D=4", "K=12,OCW=5,D=3",
                                  "K=6,OCW=9,D=2,CC=1"])
def test_every_plan_shape(plan, monkeypatch):
    """The same layer through several launch plans (positions per lane, slots per wave,
    wavefronts per workgroup, pipeline depth, channel chunk), including chunking that
    leaves a ragged last chunk."""
    monkeypatch.setenv("SPARSECONV_PLAN", plan)
    d = workloads.make_custom(3, 20, 23, 37, 50, 3, 3, 1, 1, 0.15, 77)
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, 1)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1)
    assert_parity(y, r["y64"], r["mag"], plan)


@pytest.mark.parametrize("plan", ["K=7,OCW=9", "K=4,OCW=2,CC=3,D=3", "K=2,OCW=5,D=4", "K=1,OCW=9,CC=1",
                                  "NARROW,K=4,OCW=5"])
@pytest.mark.parametrize("pad", [0, 1, 2])
def test_wide_layout_plans(plan, pad, monkeypatch):
    """Stride 1 with W % 4 == 0 and pad <= 2 uses the wide layout (input column x at phase
    column x + 4, 16-byte staging loads); NARROW forces the padded layout for the same layer."""
    monkeypatch.setenv("SPARSECONV_PLAN", plan)
    d = workloads.make_custom(3, 20, 23, 36, 50, 3, 3, 1, pad, 0.15, 78 + pad)
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, pad)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], 1, pad)
    assert_parity(y, r["y64"], r["mag"], f"{plan} pad {pad}")


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_misaligned_input_pointer(name, mapping):
    """An input that is 4-byte but not 16-byte aligned: the LDS-tile kernel's wide layout is
    then staged with 4-byte loads (same LDS layout); the output is also written through an
    offset view."""
    d = workloads.make(name)
    L = d["layer"]
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                  flags=MAPPINGS[mapping])
    xs = torch.empty(d["x"].size + 1, dtype=torch.float32, device="cuda")
    x = xs[1:].view(d["x"].shape)
    x.copy_(torch.from_numpy(d["x"]))
    assert x.data_ptr() % 16 != 0
    ys = torch.full((r["y64"].size + 3,), float("nan"), dtype=torch.float32, device="cuda")
    y = ys[3:].view(r["y64"].shape)
    h.forward(x, y)
    torch.cuda.synchronize()
    assert_parity(y.cpu().numpy(), r["y64"], r["mag"], "misaligned " + name)


@pytest.mark.parametrize("plan", ["K=1,OCW=3,D=4", "K=1,OCW=5,D=2", "K=2,OCW=2,D=3"])
def test_persistent_runs_of_many_units(plan, monkeypatch):
    """More work units than resident workgroups: each persistent workgroup walks a run of
    several tiles, with the staging pipeline crossing tile boundaries."""
    monkeypatch.setenv("SPARSECONV_PLAN", plan)
    d = workloads.make_custom(6, 5, 60, 60, 20, 3, 3, 1, 1, 0.3, 91)
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, 1)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1)
    assert_parity(y, r["y64"], r["mag"], plan)


@pytest.mark.parametrize("plan", ["", "QUAD=1", "K=8,OCW=5", "NARROW"])
@pytest.mark.parametrize("N,C,H,W,M,R,S,pad", [(1, 62, 37, 20, 114, 3, 1, 1), (1, 16, 26, 32, 123, 1, 1, 1),
                                               (4, 20, 6, 12, 87, 1, 2, 2), (2, 8, 9, 16, 20, 2, 2, 2),
                                               (2, 8, 9, 16, 20, 1, 3, 2)])
def test_padding_at_least_the_filter_width(N, C, H, W, M, R, S, pad, plan, monkeypatch):
    """Stride 1, W % 4 == 0 and pad >= S: the output is wider than the input (F = W + 2 pad -
    S + 1 > W), so the last output columns lie past the input row.  (The 16-byte staging
    layout cannot hold them and must not be used; these shapes once left the last column
    unwritten.)  The last case has pad < S for contrast."""
    if plan:
        monkeypatch.setenv("SPARSECONV_PLAN", plan)
    d = workloads.make_custom(N, C, H, W, M, R, S, 1, pad, 0.1, 9100 + W + S)
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, pad)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], 1, pad)
    assert_parity(y, r["y64"], r["mag"], f"pad {pad} S {S} {plan}")


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
@pytest.mark.parametrize("R,S,stride,pad,H,W", [(3, 3, 1, 1, 30, 41), (11, 11, 4, 0, 67, 59), (5, 3, 2, 2, 17, 23),
                                                (1, 1, 1, 0, 7, 7)])
def test_single_nonzero_bit_exact(R, S, stride, pad, H, W, mapping):
    rng = np.random.default_rng(R * 31 + W)
    N, C, M = 2, 5, 6
    x = rng.uniform(-1, 1, (N, C, H, W)).astype(np.float32)
    w = np.zeros((M, C, R, S), np.float32)
    w[2, 4, R - 1, 0] = np.float32(0.8125)
    w[5, 0, 0, S - 1] = np.float32(-1.3)
    r = oracle.reference(x, w, None, stride, pad)
    y, _ = gpu_sparse(x, w, None, stride, pad, flags=MAPPINGS[mapping])
    np.testing.assert_array_equal(y.view(np.uint32), r["y"].view(np.uint32))


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
def test_delta_kernel_identity_bit_exact(mapping):
    d = workloads.make_custom(2, 24, 31, 29, 24, 3, 3, 1, 1, 0.0, 8)
    w = np.zeros((24, 24, 3, 3), np.float32)
    for m in range(24):
        w[m, m, 1, 1] = 1.0
    y, _ = gpu_sparse(d["x"], w, None, 1, 1, flags=MAPPINGS[mapping])
    np.testing.assert_array_equal(y.view(np.uint32), d["x"].view(np.uint32))


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
def test_all_zero_weights_and_empty_rows(mapping):
    d = workloads.make_custom(2, 8, 12, 12, 40, 3, 3, 1, 1, 0.2, 21)
    mask = d["mask"].copy()
    mask[::3] = 0
    y, _ = gpu_sparse(d["x"], d["w"], mask, 1, 1, flags=MAPPINGS[mapping])
    assert np.all(y[:, ::3] == 0) and not np.signbit(y[:, ::3]).any()
    y0, _ = gpu_sparse(d["x"], d["w"], np.zeros_like(mask), 1, 1, flags=MAPPINGS[mapping])
    assert np.all(y0 == 0) and not np.signbit(y0).any()


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
def test_skewed_rows_one_dense_channel(mapping):
    """One fully dense output channel among nearly empty ones (worst case for balance)."""
    d = workloads.make_custom(2, 64, 20, 20, 32, 3, 3, 1, 1, 0.02, 31)
    mask = d["mask"].copy()
    mask[7] = 1
    r = oracle.reference(d["x"], d["w"], mask, 1, 1)
    y, _ = gpu_sparse(d["x"], d["w"], mask, 1, 1, flags=MAPPINGS[mapping])
    assert_parity(y, r["y64"], r["mag"], "skewed")


@pytest.mark.parametrize("plan", ["", "K=1,OCW=3,D=4", "K=2,OCW=2,D=2"])
def test_split_rows_many_units(plan, monkeypatch):
    """Dense channels split over several wavefronts, with many work units per workgroup, so
    the partial-sum buffers are reused from unit to unit; run twice to check that the fixed
    combine order makes the result identical."""
    if plan:
        monkeypatch.setenv("SPARSECONV_PLAN", plan)
    d = workloads.make_custom(6, 24, 40, 40, 36, 3, 3, 1, 1, 0.03, 41)
    mask = d["mask"].copy()
    mask[3] = 1
    mask[20] = 1
    r = oracle.reference(d["x"], d["w"], mask, 1, 1)
    y, h = gpu_sparse(d["x"], d["w"], mask, 1, 1, flags=sc.SC_PACK_LDS_TILE)
    assert h.info()["split_pieces"] > 0
    assert_parity(y, r["y64"], r["mag"], "split " + plan)
    y2, _ = gpu_sparse(d["x"], d["w"], mask, 1, 1, handle=h)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("name,plan", [("mid", "K=1,OCW=1"), ("pw1x1", "K=1,OCW=2"), ("tiny", "K=1,OCW=1,D=2")])
def test_split_rows_in_some_groups_finish_promptly(name, plan, monkeypatch):
    """Several groups of output channels per tile, where only some groups split rows: a
    group's partial-sum buffers are used only in that group's units, so the waits on them
    must follow that group's units alone.  (Counted over all units they wait for a use that
    never comes, until the bounded spin gives up about 0.1 s later.)"""
    monkeypatch.setenv("SPARSECONV_PLAN", plan)
    d = workloads.make(name)
    L = d["layer"]
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad)
    info = h.info()
    assert info["row_groups"] > 1 and info["split_pieces"] > 0
    assert_parity(y, r["y64"], r["mag"], f"{name} {plan}")
    xd = torch.from_numpy(d["x"]).cuda()
    out = torch.empty((L.N, L.M, L.E, L.F), dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h.forward(xd, out)
    e0.record()
    h.forward(xd, out)
    e1.record()
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) < 20.0, f"forward took {e0.elapsed_time(e1):.1f} ms"


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
def test_fewer_channels_than_wavefronts(mapping):
    """M = 4 output channels: on the LDS-tile kernel's 15 computing wavefronts every channel
    is split; the weights-in-code kernel holds all four in one wavefront."""
    d = workloads.make_custom(2, 16, 30, 30, 4, 3, 3, 1, 1, 0.5, 42)
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, 1)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1, flags=MAPPINGS[mapping])
    assert h.info()["split_pieces"] > 0
    assert_parity(y, r["y64"], r["mag"], "M=4")


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
def test_csr_input_path_and_determinism(mapping):
    d = workloads.make("mid")
    L = d["layer"]
    rowptr, colidx, value = oracle.csr_from_dense(d["w"], d["mask"])
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=value, colidx=colidx, rowptr=rowptr,
                  flags=MAPPINGS[mapping])
    y1, _ = gpu_sparse(d["x"], d["w"], None, L.stride, L.pad, handle=h)
    y2, _ = gpu_sparse(d["x"], d["w"], None, L.stride, L.pad, handle=h)
    np.testing.assert_array_equal(y1.view(np.uint32), y2.view(np.uint32))
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    assert_parity(y1, r["y64"], r["mag"], "csr")


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
def test_batch_sizes_share_one_handle(mapping):
    """N is a forward-time argument: one handle, several batch sizes, incl. N = 0 (the
    weights-in-code handle launches different kernels of its set for different N)."""
    d = workloads.make("late")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                  flags=MAPPINGS[mapping])
    for n in (1, 3, 32):
        x = d["x"][:n]
        r = oracle.reference(x, d["w"], d["mask"], L.stride, L.pad)
        y, _ = gpu_sparse(x, d["w"], d["mask"], L.stride, L.pad, handle=h)
        assert_parity(y, r["y64"], r["mag"], f"late N={n}")
    xd = torch.zeros((0, L.C, L.H, L.W), device="cuda")
    out = torch.zeros((0, L.M, L.E, L.F), device="cuda")
    h.forward(xd, out)


def test_forward_rejects_mismatched_dims_and_overlap():
    d = workloads.make("tiny")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"])
    x = torch.zeros((1, L.C, L.H, L.W), device="cuda")
    y = torch.zeros((1, L.M, L.E, L.F), device="cuda")
    with pytest.raises(sc.SparseConvError) as e:
        sc.sparseconv_forward(h.ptr, x, y, 1, L.C, L.H + 1, L.W, L.M, L.R, L.S, L.stride, L.pad)
    assert e.value.status == sc.SC_ESHAPE
    big = torch.zeros(L.M * L.E * L.F + L.C * L.H * L.W, device="cuda")
    with pytest.raises(sc.SparseConvError) as e:
        sc.sparseconv_forward(h.ptr, big.data_ptr(), big.data_ptr() + 64, 1, L.C, L.H, L.W, L.M, L.R, L.S,
                              L.stride, L.pad)
    assert e.value.status == sc.SC_EINVAL


@pytest.mark.parametrize("name", ["tiny", "mid", "first11"])
def test_all_taps_handle_parity(name):
    d = workloads.make(name, n_override=2)
    L = d["layer"]
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    y = gpu_all_taps(d["x"], d["w_masked"], L.stride, L.pad)
    assert_parity(y, r["y64"], r["mag"], "all taps " + name)


@pytest.mark.parametrize("mapping", sorted(MAPPINGS))
def test_side_stream(mapping):
    d = workloads.make("mid")
    L = d["layer"]
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y, _ = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad, stream=s, flags=MAPPINGS[mapping])
    assert_parity(y, r["y64"], r["mag"], "stream")


def _sweep_cases(count, seed):
    """Seeded shapes over wide ranges: filters 1..11 (R != S), stride 1..4, pad 0..3, 1..300
    channels, densities 0..1, one dense row in some (split across wavefronts)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        R = int(rng.choice([1, 1, 2, 3, 3, 3, 5, 7, 11]))
        S = int(rng.choice([1, 1, 2, 3, 3, 3, 5, 7, 11]))
        st, pad = int(rng.integers(1, 5)), int(rng.integers(0, 4))
        H = int(rng.integers(max(1, R - 2 * pad), 36))
        W = int(rng.integers(max(1, S - 2 * pad), 36))
        N = int(rng.integers(1, 6))
        C = int(rng.choice([1, 3, 16, 40, 130, 300]))
        M = int(rng.choice([1, 7, 33, 140, 300]))
        keep = float(rng.choice([0.0, 0.01, 0.05, 0.2, 0.6, 1.0]))
        dense_row = int(rng.integers(0, M)) if (rng.random() < 0.3 and M > 2) else -1
        E, F = (H + 2 * pad - R) // st + 1, (W + 2 * pad - S) // st + 1
        if C * M * R * S > 400_000 or N * C * H * W > 200_000 or N * M * E * F > 300_000:
            continue
        if (keep * C * M * R * S + C * R * S) * N * E * F > 5e7:  # keeps the oracle quick
            continue
        out.append((N, C, H, W, M, R, S, st, pad, keep, dense_row, seed * 1000 + len(out)))
    return out


@pytest.mark.parametrize("plan", ["", "QUAD=1", "NARROW"])
def test_random_sweep_wide_ranges(plan, monkeypatch):
    """150 seeded shapes per plan kind against the oracle, failures listed together (a sweep
    like this one found the wide-layout bug with pad >= S).  A forced quad plan may not fit
    the LDS on large stride-4 phase planes; such shapes are refused at pack (SC_EUNSUPPORTED)
    and skipped, the default plans must take every shape."""
    if plan:
        monkeypatch.setenv("SPARSECONV_PLAN", plan)
    failures, ran = [], 0
    for c in _sweep_cases(150, 4711):
        N, C, H, W, M, R, S, st, pad, keep, dense_row, seed = c
        d = workloads.make_custom(N, C, H, W, M, R, S, st, pad, keep, seed)
        mask = d["mask"].copy()
        if dense_row >= 0:
            mask[dense_row] = 1
        try:
            y, _ = gpu_sparse(d["x"], d["w"], mask, st, pad)
        except sc.SparseConvError as e:
            if plan and e.status == sc.SC_EUNSUPPORTED:
                continue
            raise
        ran += 1
        r = oracle.reference(d["x"], d["w"], mask, st, pad)
        ok = oracle.within_tolerance(y, r["y64"], r["mag"], 1e-5)
        if not ok.all():
            failures.append((c, int((~ok).sum())))
    assert ran >= 140, ran
    assert not failures, failures[:5]


def test_bounded_wait_give_up_is_reported(monkeypatch):
    """Every wait of the LDS-tile kernel is bounded; one that gives up sets the handle's
    device status word.  A spin limit of one sleep, set from the host, makes waits give up
    in a normal launch (the kernel still ends: its loops have fixed trip counts); the status
    reports it, and after clearing, a launch with the normal limit is clean and correct."""
    d = workloads.make("mid")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                  flags=sc.SC_PACK_LDS_TILE)
    x = torch.from_numpy(d["x"]).cuda()
    y = torch.empty((L.N, L.M, L.E, L.F), device="cuda")
    assert h.device_status() == 0
    monkeypatch.setenv("SPARSECONV_SPIN_LIMIT", "1")
    h.forward(x, y)
    torch.cuda.synchronize()
    assert h.device_status(clear=True) & 1
    assert h.device_status() == 0
    monkeypatch.delenv("SPARSECONV_SPIN_LIMIT")
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    got, _ = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad, handle=h)
    assert_parity(got, r["y64"], r["mag"], "after clearing")
