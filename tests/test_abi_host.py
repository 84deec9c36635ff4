"""The C-ABI library on the host (CPU only, no GPU calls): symbols, packing, validation.

Packing with SC_PACK_HOST_ONLY runs the whole host part of the packer (CSR, stretched
offsets, schedule, kernel encoding) without a device, so the canonical packed form can be
checked bit-exactly against the oracle's independent CSR builder and stretch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import sparse_weight_direct_amd as sc
import workloads

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sparseconv.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparseconv_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) == len(sc.EXPORTED) >= 10
    lib = ctypes.CDLL(sc.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(sc.EXPORTED) == names
    for n in names:
        assert callable(getattr(sc, n))


def _pack_host(d, L, **kw):
    return sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                     flags=sc.SC_PACK_HOST_ONLY, **kw)


@pytest.mark.parametrize("name", ["tiny", "mid", "late", "imb95", "first11", "pw1x1"])
def test_canonical_export_bit_exact_vs_oracle(name):
    d = workloads.make(name, n_override=1)
    L = d["layer"]
    h = _pack_host(d, L)
    rowptr, off, val = h.export()
    o_rowptr, o_col, o_val = oracle.csr_from_dense(d["w"], d["mask"])
    o_off = oracle.stretch(o_col, L.C, L.R, L.S, L.H, L.W)
    np.testing.assert_array_equal(rowptr, o_rowptr)
    np.testing.assert_array_equal(off, o_off)
    np.testing.assert_array_equal(val.view(np.uint32), o_val.view(np.uint32))
    info = h.info()
    nnz = int(d["mask"].sum())
    assert info["nnz"] == nnz
    assert info["packed_bytes"] == (2 * nnz + L.M + 1) * 4
    assert (info["E"], info["F"]) == (L.E, L.F)


def test_dense_mask_and_csr_inputs_give_identical_handles():
    d = workloads.make("tiny")
    L = d["layer"]
    h1 = _pack_host(d, L)
    rowptr, col, val = oracle.csr_from_dense(d["w"], d["mask"])
    # shuffle columns within rows: the packer must sort them, moving values along
    rng = np.random.default_rng(0)
    col_s, val_s = col.copy(), val.copy()
    for m in range(L.M):
        b, e = rowptr[m], rowptr[m + 1]
        perm = rng.permutation(e - b) + b
        col_s[b:e], val_s[b:e] = col[perm], val[perm]
    h2 = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=val_s, colidx=col_s, rowptr=rowptr,
                   flags=sc.SC_PACK_HOST_ONLY)
    for a, b in zip(h1.export(), h2.export()):
        np.testing.assert_array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))
    assert h1.info() == h2.info()


def test_no_mask_storage_rule_and_explicit_zeros():
    w = np.array([0.0, 1.5, -0.0, np.nan, 2.0, 0.0, 0.0, 3.0], np.float32).reshape(2, 1, 2, 2)
    h = sc.Handle.from_dense(w, 3, 3, 1, 0, flags=sc.SC_PACK_HOST_ONLY)
    rowptr, off, val = h.export()
    assert rowptr.tolist() == [0, 2, 4]
    # columns 1, 3 | 0, 3 -> (r, s) = (0,1), (1,1) | (0,0), (1,1) with W = 3
    assert off.tolist() == [1, 4, 0, 4]
    assert val[0] == 1.5 and np.isnan(val[1]) and val[2] == 2.0 and val[3] == 3.0
    mask = np.array([0, 1, 1, 0, 1, 0, 0, 0], np.uint8).reshape(2, 1, 2, 2)
    h = sc.Handle.from_dense(w, 3, 3, 1, 0, mask=mask, flags=sc.SC_PACK_HOST_ONLY)
    rowptr, off, val = h.export()
    assert rowptr.tolist() == [0, 2, 3]
    assert np.signbit(val[1]) and val[1] == 0.0


def _status(fn):
    try:
        fn()
    except sc.SparseConvError as e:
        return e.status, str(e)
    return sc.SC_OK, ""


@pytest.mark.parametrize("bad,expect", [
    ("rowptr_decreasing", sc.SC_EINVAL), ("rowptr0_nonzero", sc.SC_EINVAL), ("col_out_of_range", sc.SC_EINVAL),
    ("col_negative", sc.SC_EINVAL), ("duplicate", sc.SC_EINVAL),
])
def test_invalid_csr_rejected(bad, expect):
    M, C, R, S = 2, 2, 3, 3
    rowptr = np.array([0, 2, 4], np.int32)
    col = np.array([0, 5, 3, 17], np.int32)
    val = np.ones(4, np.float32)
    if bad == "rowptr_decreasing":
        rowptr = np.array([0, 3, 2], np.int32)
    elif bad == "rowptr0_nonzero":
        rowptr = np.array([1, 2, 4], np.int32)
    elif bad == "col_out_of_range":
        col[3] = C * R * S
    elif bad == "col_negative":
        col[0] = -1
    elif bad == "duplicate":
        col[1] = 0
    st, msg = _status(lambda: sc.sparseconv_pack(M, C, R, S, 5, 5, 1, 1, values=val, colidx=col, rowptr=rowptr,
                                                 flags=sc.SC_PACK_HOST_ONLY))
    assert st == expect and "CSR" in msg


def test_shape_and_limit_errors():
    w = np.ones((2, 1, 3, 3), np.float32)
    st, _ = _status(lambda: sc.sparseconv_pack(0, 1, 3, 3, 5, 5, 1, 1, values=w, flags=sc.SC_PACK_HOST_ONLY))
    assert st == sc.SC_ESHAPE
    st, _ = _status(lambda: sc.sparseconv_pack(2, 1, 3, 3, 2, 2, 1, 0, values=w, flags=sc.SC_PACK_HOST_ONLY))
    assert st == sc.SC_ESHAPE  # output would be empty
    st, _ = _status(lambda: sc.sparseconv_pack(2, 1, 3, 3, 5, 5, 0, 1, values=w, flags=sc.SC_PACK_HOST_ONLY))
    assert st == sc.SC_ESHAPE  # stride 0
    big = np.ones((1, 1, 1, 1), np.float32)
    st, msg = _status(lambda: sc.sparseconv_pack(1, 1, 1, 1, 65536, 65536, 1, 0, values=big,
                                                 flags=sc.SC_PACK_HOST_ONLY))
    assert st == sc.SC_EUNSUPPORTED and "2^32" in msg
    st, _ = _status(lambda: sc.sparseconv_pack(2, 1, 3, 3, 5, 5, 1, 1, values=w, flags=1 << 10))
    assert st == sc.SC_EINVAL


def test_forward_validation_without_device():
    d = workloads.make("tiny")
    L = d["layer"]
    h = _pack_host(d, L)
    st, msg = _status(lambda: sc.sparseconv_forward(h.ptr, 1 << 20, 1 << 24, 1, L.C, L.H, L.W, L.M, L.R, L.S,
                                                    L.stride, L.pad, stream=0))
    assert st == sc.SC_EINVAL and "HOST_ONLY" in msg
    st, _ = _status(lambda: sc.sparseconv_forward(0, 1 << 20, 1 << 24, 1, L.C, L.H, L.W, L.M, L.R, L.S,
                                                  L.stride, L.pad, stream=0))
    assert st == sc.SC_EINVAL
    assert sc.sparseconv_last_error() != ""
    sc.sparseconv_destroy(None)  # no-op


def test_all_taps_flag_stores_every_position():
    d = workloads.make("tiny")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w_masked"],
                  flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_ALL_TAPS)
    rowptr, off, val = h.export()
    crs = L.C * L.R * L.S
    assert rowptr.tolist() == [m * crs for m in range(L.M + 1)]
    np.testing.assert_array_equal(val, d["w_masked"].reshape(-1))
    o_off = oracle.stretch(np.tile(np.arange(crs, dtype=np.int32), L.M), L.C, L.R, L.S, L.H, L.W)
    np.testing.assert_array_equal(off, o_off)
    rp, col, v = oracle.csr_from_dense(d["w"], d["mask"])
    st, _ = _status(lambda: sc.sparseconv_pack(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=v, colidx=col,
                                               rowptr=rp, flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_ALL_TAPS))
    assert st == sc.SC_EINVAL


def test_injected_allocation_failure(monkeypatch):
    d = workloads.make("tiny")
    L = d["layer"]
    monkeypatch.setenv("SPARSECONV_TEST_FAIL_ALLOC", "1")
    st, msg = _status(lambda: _pack_host(d, L))
    assert st == sc.SC_ENOMEM and "injected" in msg


@pytest.mark.parametrize("name", ["imb80", "imb95", "imb99"])
def test_schedule_balances_wavefronts_by_nnz(name):
    d = workloads.make(name, n_override=1)
    L = d["layer"]
    info = _pack_host(d, L).info()
    nnz = int(d["mask"].sum())
    waves = info["row_groups"] * info["waves_per_group"]
    rows = d["mask"].reshape(L.M, -1).sum(1)
    # the heaviest wavefront exceeds the mean by less than one row, and the per-chunk
    # synchronisation costs little over the mean (rows are dealt chunk-balanced)
    assert info["max_wave_nnz"] <= nnz / waves + rows.max()
    assert info["max_wave_nnz"] <= 1.15 * nnz / waves
    assert 1000 <= info["step_balance_permille"] <= {"imb80": 1100, "imb95": 1150, "imb99": 1250}[name]


@pytest.mark.parametrize("dense_rows", [1, 3])
def test_long_rows_are_split_across_wavefronts(dense_rows):
    """Rows longer than a wavefront's fair share are split into pieces on different
    wavefronts: the heaviest wavefront stays near the mean instead of carrying a whole dense
    row, and the canonical export is unchanged."""
    d = workloads.make_custom(1, 32, 20, 20, 40, 3, 3, 1, 1, 0.05, 5)
    mask = d["mask"].copy()
    mask[7:7 + dense_rows] = 1
    h = sc.Handle(40, 32, 3, 3, 20, 20, 1, 1, values=d["w"], mask=mask, flags=sc.SC_PACK_HOST_ONLY)
    info = h.info()
    nnz = int(mask.sum())
    waves = info["row_groups"] * info["waves_per_group"]
    assert info["split_pieces"] > 0
    assert info["max_wave_nnz"] < 32 * 9  # no wavefront holds a whole dense row
    assert info["max_wave_nnz"] <= 1.5 * nnz / waves
    rowptr, off, val = h.export()
    r = oracle.reference(d["x"][:1], d["w"], mask, 1, 1)
    assert np.array_equal(rowptr, r["rowptr"]) and np.array_equal(off, r["offsets"])
    assert np.array_equal(val.view(np.uint32), r["values"].view(np.uint32))


def test_no_split_for_balanced_layers():
    for name in ("imb80", "imb95", "tiny", "late"):
        d = workloads.make(name, n_override=1)
        assert _pack_host(d, d["layer"]).info()["split_pieces"] == 0, name


def test_chain_rejects_mismatched_shapes():
    from sparse_weight_direct_amd.chain import LayerChain
    a = sc.Handle(8, 4, 3, 3, 10, 10, 1, 1, values=np.ones((8, 4, 3, 3), np.float32), flags=sc.SC_PACK_HOST_ONLY)
    b = sc.Handle(8, 6, 3, 3, 10, 10, 1, 1, values=np.ones((8, 6, 3, 3), np.float32), flags=sc.SC_PACK_HOST_ONLY)
    with pytest.raises(ValueError):
        LayerChain([a, b], N=1)


def test_escoin_mapping_handle_on_host():
    """SC_PACK_ESCOIN_MAP: same canonical export, its own info and workspace size, and the
    combinations the header rejects."""
    d = workloads.make("mid", n_override=1)
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                  flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_ESCOIN_MAP)
    rowptr, off, val = h.export()
    o_rowptr, o_col, o_val = oracle.csr_from_dense(d["w"], d["mask"])
    np.testing.assert_array_equal(rowptr, o_rowptr)
    np.testing.assert_array_equal(off, oracle.stretch(o_col, L.C, L.R, L.S, L.H, L.W))
    np.testing.assert_array_equal(val.view(np.uint32), o_val.view(np.uint32))
    info = h.info()
    assert info["mapping"] == 1 and info["max_wave_nnz"] == int(np.diff(o_rowptr).max())
    for n in (0, 1, 3):
        want = n * L.C * (L.H + 2 * L.pad) * (L.W + 2 * L.pad) * 4
        assert h.workspace_size(n) == (want + 255) // 256 * 256
    assert _pack_host(d, L).workspace_size(5) == 0 and _pack_host(d, L).info()["mapping"] == sc.MAPPING_BAKED
    assert _pack_host(d, L, ).info()["bake_groups"] >= 1
    lds = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                    flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_LDS_TILE)
    assert lds.info()["mapping"] == sc.MAPPING_LDS_TILE and lds.info()["bake_groups"] == 0
    st, msg = _status(lambda: sc.sparseconv_pack(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"],
                                                 mask=d["mask"], flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_ESCOIN_MAP
                                                 | sc.SC_PACK_LDS_TILE))
    assert st == sc.SC_EINVAL
    st, msg = _status(lambda: sc.sparseconv_pack(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"],
                                                 mask=d["mask"], flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_ESCOIN_MAP
                                                 | sc.SC_PACK_FP16_WORD))
    assert st == sc.SC_EINVAL and "ESCOIN" in msg
    st, _ = _status(lambda: h.workspace_size(-1))
    assert st == sc.SC_ESHAPE
    st, msg = _status(lambda: sc.sparseconv_forward_workspace(h.ptr, 1 << 20, 1 << 24, 1, L.C, L.H, L.W, L.M, L.R,
                                                              L.S, L.stride, L.pad, 1 << 28, 1 << 24, stream=0))
    assert st == sc.SC_EINVAL and "HOST_ONLY" in msg


def test_destroyed_and_foreign_handles_are_rejected():
    """The library keeps a registry of live handles: a destroyed handle, a second destroy and
    a pointer that never was a handle are reported (or ignored by destroy), never read."""
    d = workloads.make("tiny")
    L = d["layer"]
    h = _pack_host(d, L)
    ptr = h.ptr
    assert sc.sparseconv_query(ptr)["M"] == L.M
    sc.sparseconv_destroy(ptr)
    h.ptr = None
    st, msg = _status(lambda: sc.sparseconv_query(ptr))
    assert st == sc.SC_EINVAL and "destroyed" in msg
    sc.sparseconv_destroy(ptr)  # second destroy: ignored
    buf = np.zeros(64, np.uint8)
    fake = buf.ctypes.data
    st, _ = _status(lambda: sc.sparseconv_query(fake))
    assert st == sc.SC_EINVAL
    sc.sparseconv_destroy(fake)  # not a handle: ignored
    st, _ = _status(lambda: sc.sparseconv_export_packed(fake))
    assert st == sc.SC_EINVAL


def test_binding_checks_tensor_shapes_before_launch():
    """Handle.forward rejects an input or output whose shape differs from the handle's
    geometry before any pointer reaches the library (so a wrong-sized tensor cannot make the
    kernel read or write past it); output sizes come from the library's own E and F."""
    import torch
    d = workloads.make("tiny")
    L = d["layer"]
    h = _pack_host(d, L)
    assert (h.E, h.F) == (L.E, L.F)
    good_x = torch.zeros((1, L.C, L.H, L.W))
    with pytest.raises(ValueError, match="input shape"):
        h.forward(torch.zeros((1, L.C, L.H + 1, L.W)))
    with pytest.raises(ValueError, match="input shape"):
        h.forward(torch.zeros((L.C, L.H, L.W)))
    with pytest.raises(ValueError, match="output shape"):
        h.forward(good_x, torch.zeros((1, L.M, L.E, L.F + 1)))
    with pytest.raises(ValueError, match="output shape"):
        h.forward(good_x, torch.zeros((2, L.M, L.E, L.F)))
    with pytest.raises(ValueError, match="float32"):
        h.forward(good_x.double(), torch.zeros((1, L.M, L.E, L.F)))


def test_dense_forward_checks_before_any_device_work():
    """sparseconv_dense_forward validates shapes, pointers, alignment, overlap and the 32-bit
    limits on the host and returns before touching a device; N = 0 is a no-op."""
    base = 1 << 40  # never dereferenced: every call below fails (or returns) before a launch
    a = dict(N=2, C=3, H=10, W=12, M=4, R=3, S=3, stride=1, pad=1)

    def call(w=base, x=base + (1 << 30), y=base + (2 << 30), **kw):
        g = dict(a, **kw)
        return _status(lambda: sc.sparseconv_dense_forward(w, x, y, g["N"], g["C"], g["H"], g["W"], g["M"],
                                                           g["R"], g["S"], g["stride"], g["pad"], 0))

    assert call(N=0) == (sc.SC_OK, "")
    assert call(N=0, w=0, x=0, y=0) == (sc.SC_OK, "")
    assert call(N=-1)[0] == sc.SC_ESHAPE
    assert call(R=13)[0] == sc.SC_ESHAPE          # filter taller than the padded input
    assert call(stride=0)[0] == sc.SC_ESHAPE
    assert call(pad=-1)[0] == sc.SC_ESHAPE
    assert call(M=0)[0] == sc.SC_ESHAPE
    assert call(w=0)[0] == sc.SC_EINVAL
    assert call(x=base + (1 << 30) + 2)[0] == sc.SC_EINVAL          # misaligned
    assert call(y=base + (1 << 30) + 64)[0] == sc.SC_EINVAL         # output overlaps input
    assert call(y=base)[0] == sc.SC_EINVAL                          # output overlaps the weights
    assert call(N=1 << 20, C=64, H=64, W=64)[0] == sc.SC_EUNSUPPORTED  # input >= 2^31 bytes
    assert call(M=1 << 16, C=1 << 12, R=3, S=3, N=1)[0] == sc.SC_EUNSUPPORTED  # M*C*R*S >= 2^31


def test_tune_checks_arguments_before_any_device_work():
    """sparseconv_tune rejects a host-only handle, a bad repetition count and N < 1 without
    launching anything."""
    d = workloads.make("tiny")
    L = d["layer"]
    h = _pack_host(d, L)
    fake = 1 << 40
    args = (L.C, L.H, L.W, L.M, L.R, L.S, L.stride, L.pad)
    st, msg = _status(lambda: sc.sparseconv_tune(h.ptr, fake, fake + (1 << 30), 1, *args, reps=5, stream=0))
    assert st == sc.SC_EINVAL and "HOST_ONLY" in msg
    st, _ = _status(lambda: sc.sparseconv_tune(h.ptr, fake, fake + (1 << 30), 1, *args, reps=0, stream=0))
    assert st == sc.SC_EINVAL
    st, _ = _status(lambda: sc.sparseconv_tune(h.ptr, fake, fake + (1 << 30), 0, *args, reps=3, stream=0))
    assert st == sc.SC_ESHAPE


def test_launch_rule_for_the_large_layers():
    """Which weights-in-code kernel a forward launches (host-only handles assume 256 compute
    units): where the staged kernels give every SIMD a wavefront they are launched, the one
    whose workgroups share their window between two groups on layers with at least 64
    non-zeros per output channel, the one-group one below; a batch of one image leaves SIMDs
    idle and launches an unstaged kernel."""
    seen = {}
    for name in ("imb95", "imb90"):
        d = workloads.make(name)
        L = d["layer"]
        h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                      flags=sc.SC_PACK_HOST_ONLY)
        nnz_per_channel = h.info()["nnz"] / L.M
        big = h.launch_info(L.N)
        assert big["stage"] == 1 and big["waves"] >= 4 * 256
        assert (big["groups"] == 2 and big["block"] == 512) == (nnz_per_channel >= 64), (name, big)
        small = h.launch_info(1)
        assert small["stage"] == 0, (name, small)
        seen[name] = big["groups"]
    assert seen == {"imb95": 1, "imb90": 2}
