"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties the oracle to a fact fixed by the pages or by mathematics:
  * brute force in a different formulation (scatter from inputs instead of gather to outputs);
  * torch's float64 conv2d (a library routine the oracle does not use) on masked weights;
  * closed forms: delta kernel, shifted / scaled single non-zero, 1x1, the worked two-non-zero
    example after "Escoin" Fig. 5;
  * invariants: linearity over disjoint masks, exact zeros, the CSR size (2*nnz+M+1)*4 bytes
    ("Escoin", CSR section), the layout-function additivity f(c,y+r,x+s) = f(c,y,x) + f(0,r,s)
    and the stretched-offset gather ("Escoin", dynamic indexing / weight stretching);
  * the output-size formula (Tuteja et al., Sec. 3 Eq. (2)) against torch's output shapes.
"""
import os

import numpy as np
import pytest
import scipy.sparse
import torch

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _brute_scatter(x, w, mask, stride, pad):
    """All taps, scattered from each input element to the outputs it feeds (pure Python)."""
    N, C, H, W = x.shape
    M, _, R, S = w.shape
    E = (H + 2 * pad - R) // stride + 1
    F = (W + 2 * pad - S) // stride + 1
    y = np.zeros((N, M, E, F), np.float64)
    for n in range(N):
        for c in range(C):
            for iy in range(H):
                for ix in range(W):
                    xv = float(x[n, c, iy, ix])
                    for m in range(M):
                        for r in range(R):
                            ey = iy + pad - r
                            if ey < 0 or ey % stride:
                                continue
                            e = ey // stride
                            if e >= E:
                                continue
                            for s in range(S):
                                if not mask[m, c, r, s]:
                                    continue
                                fx = ix + pad - s
                                if fx < 0 or fx % stride:
                                    continue
                                f = fx // stride
                                if f >= F:
                                    continue
                                y[n, m, e, f] += float(w[m, c, r, s]) * xv
    return y


def _torch_ref(x, w_masked, stride, pad):
    return torch.nn.functional.conv2d(torch.from_numpy(x).double(), torch.from_numpy(w_masked).double(),
                                      stride=stride, padding=pad).numpy()


def _tiny_cases(count, seed0):
    rng = np.random.default_rng(seed0)
    cases = []
    keeps = [1.0, 0.5, 0.1, 0.0]
    for i in range(count):
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        stride, pad = int(rng.integers(1, 5)), int(rng.integers(0, 3))
        H = int(rng.integers(max(1, R - 2 * pad), 10))
        W = int(rng.integers(max(1, S - 2 * pad), 10))
        cases.append(dict(N=int(rng.integers(1, 3)), C=int(rng.integers(1, 6)), H=H, W=W,
                          M=int(rng.integers(1, 7)), R=R, S=S, stride=stride, pad=pad,
                          keep=keeps[i % 4], seed=seed0 * 100 + i))
    return cases


@pytest.mark.parametrize("case", _tiny_cases(16, 7), ids=lambda c: "N{N}C{C}H{H}W{W}M{M}R{R}S{S}st{stride}p{pad}k{keep}".format(**c))
def test_def_and_list_forms_match_scatter_brute_force(case):
    d = workloads.make_custom(case["N"], case["C"], case["H"], case["W"], case["M"], case["R"], case["S"],
                              case["stride"], case["pad"], case["keep"], case["seed"])
    y_ref = _brute_scatter(d["x"], d["w"], d["mask"], case["stride"], case["pad"])
    y_def, mag_def = oracle.conv_def(d["x"], d["w"], d["mask"], case["stride"], case["pad"])
    r = oracle.reference(d["x"], d["w"], d["mask"], case["stride"], case["pad"])
    assert y_def.shape == y_ref.shape == r["y64"].shape
    tol = 1e-12 * (mag_def + 1e-300)
    assert np.all(np.abs(y_def - y_ref) <= tol)
    assert np.all(np.abs(r["y64"] - y_ref) <= tol)
    np.testing.assert_array_equal(mag_def, r["mag"]) if case["R"] * case["S"] == 1 else \
        np.testing.assert_allclose(mag_def, r["mag"], rtol=1e-12, atol=0)


@pytest.mark.parametrize("case", _tiny_cases(24, 11), ids=lambda c: "N{N}C{C}H{H}W{W}M{M}R{R}S{S}st{stride}p{pad}k{keep}".format(**c))
def test_matches_torch_conv2d_float64(case):
    d = workloads.make_custom(case["N"], case["C"], case["H"], case["W"], case["M"], case["R"], case["S"],
                              case["stride"], case["pad"], case["keep"], case["seed"])
    r = oracle.reference(d["x"], d["w"], d["mask"], case["stride"], case["pad"])
    t = _torch_ref(d["x"], d["w_masked"], case["stride"], case["pad"])
    assert t.shape == r["y64"].shape
    assert np.all(np.abs(t - r["y64"]) <= 1e-12 * r["mag"] + 1e-300)


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_named_layers_match_torch(name):
    d = workloads.make(name)
    L = d["layer"]
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    t = _torch_ref(d["x"], d["w_masked"], L.stride, L.pad)
    assert np.all(np.abs(t - r["y64"]) <= 1e-12 * r["mag"] + 1e-300)
    # the definitional 7-loop form agrees with the list form on the small layer
    if name == "tiny":
        y_def, mag_def = oracle.conv_def(d["x"], d["w"], d["mask"], L.stride, L.pad)
        assert np.all(np.abs(y_def - r["y64"]) <= 1e-12 * mag_def + 1e-300)


def test_zero_sparsity_equals_dense_conv():
    d = workloads.make_custom(2, 4, 9, 7, 5, 3, 3, 1, 1, 1.0, 42)
    assert d["mask"].all()
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, 1)
    t = _torch_ref(d["x"], d["w"], 1, 1)
    assert np.all(np.abs(t - r["y64"]) <= 1e-12 * r["mag"])


@pytest.mark.parametrize("R,pad", [(3, 1), (5, 2), (1, 0)])
def test_delta_kernel_is_identity_bit_exact(R, pad):
    d = workloads.make_custom(2, 6, 11, 9, 6, R, R, 1, pad, 0.0, 5)
    w = np.zeros((6, 6, R, R), np.float32)
    for m in range(6):
        w[m, m, R // 2, R // 2] = 1.0
    r = oracle.reference(d["x"], w, None, 1, pad)
    np.testing.assert_array_equal(r["y"].view(np.uint32), d["x"].view(np.uint32))


@pytest.mark.parametrize("R,S,stride,pad,H,W", [(3, 3, 1, 1, 10, 12), (3, 5, 2, 2, 13, 9),
                                                (11, 11, 4, 0, 35, 39), (4, 2, 3, 1, 12, 10)])
def test_single_nonzero_is_shifted_scaled_copy(R, S, stride, pad, H, W):
    rng = np.random.default_rng(R * 100 + S)
    N, C, M = 2, 3, 4
    x = rng.uniform(-1, 1, (N, C, H, W)).astype(np.float32)
    for m0, c0, r0, s0 in [(1, 2, R - 1, 0), (3, 0, 0, S - 1), (0, 1, R // 2, S // 2)]:
        a = np.float32(rng.uniform(-2, 2))
        w = np.zeros((M, C, R, S), np.float32)
        w[m0, c0, r0, s0] = a
        r = oracle.reference(x, w, None, stride, pad)
        E, F = r["y"].shape[2:]
        exp = np.zeros((N, M, E, F), np.float32)
        for e in range(E):
            for f in range(F):
                iy, ix = e * stride - pad + r0, f * stride - pad + s0
                if 0 <= iy < H and 0 <= ix < W:
                    exp[:, m0, e, f] = a * x[:, c0, iy, ix]  # one fp32 rounding of the product
        np.testing.assert_array_equal(r["y"].view(np.uint32), exp.view(np.uint32))


@pytest.mark.parametrize("stride", [1, 2])
def test_1x1_single_nonzero(stride):
    rng = np.random.default_rng(3)
    x = rng.uniform(-1, 1, (3, 5, 7, 8)).astype(np.float32)
    w = np.zeros((4, 5, 1, 1), np.float32)
    a = np.float32(-0.375)
    w[2, 4, 0, 0] = a
    r = oracle.reference(x, w, None, stride, 0)
    exp = np.zeros_like(r["y"])
    exp[:, 2] = a * x[:, 4, ::stride, ::stride]
    np.testing.assert_array_equal(r["y"].view(np.uint32), exp.view(np.uint32))


def test_escoin_fig5_worked_example():
    g = np.loadtxt(os.path.join(GOLD, "escoin_fig5.txt"), dtype=np.float64)
    x = (6 * np.arange(6)[:, None] + np.arange(6)[None, :]).astype(np.float32).reshape(1, 1, 6, 6)
    w = np.zeros((1, 1, 3, 3), np.float32)
    w[0, 0, 0, 0] = 2.0
    w[0, 0, 1, 2] = 3.0
    r = oracle.reference(x, w, None, 1, 0)
    np.testing.assert_array_equal(r["y"][0, 0], g.astype(np.float32))
    y_def, _ = oracle.conv_def(x, w, None, 1, 0)
    np.testing.assert_array_equal(y_def[0, 0], g)


def test_linearity_over_disjoint_masks():
    d = workloads.make_custom(2, 5, 10, 11, 6, 3, 4, 2, 1, 0.6, 77)
    rng = np.random.default_rng(1)
    split = rng.random(d["mask"].shape) < 0.5
    m1 = (d["mask"] & split).astype(np.uint8)
    m2 = (d["mask"] & ~split).astype(np.uint8)
    r = oracle.reference(d["x"], d["w"], d["mask"], 2, 1)
    r1 = oracle.reference(d["x"], d["w"], m1, 2, 1)
    r2 = oracle.reference(d["x"], d["w"], m2, 2, 1)
    assert np.all(np.abs(r1["y64"] + r2["y64"] - r["y64"]) <= 1e-12 * r["mag"] + 1e-300)
    np.testing.assert_allclose(r1["mag"] + r2["mag"], r["mag"], rtol=1e-12, atol=0)


def test_all_zero_and_empty_rows_give_positive_zero():
    d = workloads.make_custom(2, 3, 8, 8, 5, 3, 3, 1, 1, 0.3, 9)
    mask = d["mask"].copy()
    mask[1] = 0
    mask[3] = 0
    r = oracle.reference(d["x"], d["w"], mask, 1, 1)
    for m in (1, 3):
        assert np.all(r["y"][:, m] == 0) and not np.signbit(r["y"][:, m]).any()
        assert np.all(r["mag"][:, m] == 0)
    r0 = oracle.reference(d["x"], d["w"], np.zeros_like(mask), 1, 1)
    assert np.all(r0["y"] == 0) and not np.signbit(r0["y"]).any()
    assert r0["rowptr"].tolist() == [0] * 6


def test_csr_against_scipy_and_size_invariant():
    for name in ["tiny", "mid"]:
        d = workloads.make(name)
        L = d["layer"]
        rowptr, colidx, value = oracle.csr_from_dense(d["w"], d["mask"])
        sp = scipy.sparse.csr_matrix(d["w_masked"].reshape(L.M, -1))
        sp.sort_indices()
        np.testing.assert_array_equal(rowptr, sp.indptr)
        np.testing.assert_array_equal(colidx, sp.indices)
        np.testing.assert_array_equal(value, sp.data)
        nnz = colidx.size
        assert nnz == int(d["mask"].sum())
        # "Escoin", CSR section: (2*nnz + M + 1) * 4 bytes
        assert rowptr.nbytes + colidx.nbytes + value.nbytes == (2 * nnz + L.M + 1) * 4


def _read_kv(path):
    out = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *v = line.split()
        out[k] = v
    return out


def test_csr_storage_rules_fixture():
    g = _read_kv(os.path.join(GOLD, "csr_rules.txt"))
    w = np.array([[0.0, 1.5, -0.0, np.nan], [2.0, 0.0, 0.0, 3.0]], np.float32)
    rowptr, colidx, value = oracle.csr_from_dense(w, None)
    assert rowptr.tolist() == [int(v) for v in g["rowptr"]]
    assert colidx.tolist() == [int(v) for v in g["colidx"]]
    np.testing.assert_array_equal(value, np.array([float(v) for v in g["value"]], np.float32))
    mask = np.array([[0, 1, 1, 0], [1, 0, 0, 0]], np.uint8)
    rowptr, colidx, value = oracle.csr_from_dense(w, mask)
    assert rowptr.tolist() == [int(v) for v in g["mask_rowptr"]]
    assert colidx.tolist() == [int(v) for v in g["mask_colidx"]]
    exp = np.array([float(v) for v in g["mask_value"]], np.float32)
    np.testing.assert_array_equal(value.view(np.uint32), exp.view(np.uint32))


def test_stretched_offsets_layout_function_and_gather():
    C, R, S, H, W = 4, 3, 5, 9, 11
    cols = np.arange(C * R * S, dtype=np.int32)
    off = oracle.stretch(cols, C, R, S, H, W).astype(np.int64)
    f = off.reshape(C, R, S)
    # additivity of the layout function: f(c, r, s) = f(c, 0, 0) + f(0, r, s), f(c,0,0) = c*H*W
    np.testing.assert_array_equal(f, f[:, :1, :1] + f[:1, :, :])
    np.testing.assert_array_equal(f[:, 0, 0], np.arange(C) * H * W)
    # gather: base of an output position plus the offset addresses the input element
    rng = np.random.default_rng(0)
    N, stride, pad = 2, 2, 1
    x = rng.uniform(-1, 1, (N, C, H, W)).astype(np.float32)
    flat = x.reshape(-1)
    E = (H + 2 * pad - R) // stride + 1
    F = (W + 2 * pad - S) // stride + 1
    for n in range(N):
        for e in range(E):
            for fo in range(F):
                for c in range(C):
                    for r in range(R):
                        for s in range(S):
                            iy, ix = e * stride - pad + r, fo * stride - pad + s
                            if 0 <= iy < H and 0 <= ix < W:
                                idx = n * C * H * W + f[c, r, s] + (e * stride - pad) * W + (fo * stride - pad)
                                assert flat[idx] == x[n, c, iy, ix]


def test_out_size_matches_torch_shapes_and_first_layer():
    rng = np.random.default_rng(5)
    for _ in range(50):
        k, stride, pad = int(rng.integers(1, 8)), int(rng.integers(1, 5)), int(rng.integers(0, 4))
        n_in = int(rng.integers(max(1, k - 2 * pad), 40))
        t = torch.nn.functional.conv2d(torch.zeros(1, 1, n_in, 3), torch.zeros(1, 1, k, 1),
                                       stride=(stride, 1), padding=(pad, 0))
        assert oracle.out_size(n_in, pad, k, stride) == t.shape[2]
    assert oracle.out_size(227, 0, 11, 4) == 55
    assert oracle.out_size(2, 0, 3, 1) == 0


def test_conv_csr_planes_equals_full_convolution():
    """The per-plane form used on full-size layers: any selection of (n, m) planes, in any
    order and with repeats, equals the corresponding planes of the full list form bit for bit
    ([T] Sec. 3 Eq. (3) summed per output plane; plane id n*M + m)."""
    rng = np.random.default_rng(17)
    for i, (N, C, H, W, M, R, S, st, p) in enumerate([(3, 4, 9, 8, 5, 3, 2, 2, 1), (2, 3, 11, 13, 7, 1, 3, 1, 0),
                                                       (4, 2, 6, 6, 3, 3, 3, 1, 2)]):
        d = workloads.make_custom(N, C, H, W, M, R, S, st, p, 0.5, 7100 + i)
        rowptr, colidx, value = oracle.csr_from_dense(d["w"], d["mask"])
        y64, mag = oracle.conv_csr(d["x"], rowptr, colidx, value, M, R, S, st, p)
        planes = np.concatenate([rng.permutation(N * M), rng.integers(0, N * M, 5)])
        yp, mp = oracle.conv_csr_planes(d["x"], rowptr, colidx, value, M, R, S, st, p, planes)
        E, F = y64.shape[2:]
        np.testing.assert_array_equal(yp, y64.reshape(N * M, E, F)[planes])
        np.testing.assert_array_equal(mp, mag.reshape(N * M, E, F)[planes])


def tolerance_pins_pass(fn) -> bool:
    """Hand-built cases of the parity bar |y - y_ref| <= rel * MAG (MAG = sum |w*x|), with
    MAG = 0 requiring y == 0 exactly; the comparison in double precision."""
    rel = 1e-5
    mag = np.array([1.0, 1.0, 1.0, 0.0, 0.0, 2.0, 1e6, 1.0, 3.0], np.float64)
    ref = np.array([0.5, 0.5, 0.5, 0.0, 0.0, -1.0, 1e6 - 3.0, 0.25, 1.0], np.float64)
    d_at = rel * mag  # the bound, reached exactly by representable differences below
    y = np.array([0.5,                    # exact
                  0.5 + 2.0 ** -17,       # |d| = 7.6e-6 < 1e-5: inside
                  0.5 + 2.0 ** -16,       # |d| = 1.5e-5 > 1e-5: outside
                  0.0,                    # MAG = 0 and y = 0: passes
                  1e-35,                  # MAG = 0 and y != 0 (however small): fails
                  -1.0 + 2.0 ** -17,      # |d| = 7.6e-6 <= 2e-5: inside
                  1e6 - 3.0 + 8.0,        # |d| = 8 <= 10: inside (relative, not absolute)
                  np.nan,                 # NaN: fails
                  1.0 + 2.0 ** -23],      # |d| = 1.2e-7: inside; in fp32 arithmetic also fine
                 np.float64).astype(np.float32)
    want = np.array([True, True, False, True, False, True, True, False, True])
    if not np.array_equal(fn(y, ref, mag, rel), want):
        return False
    # a difference exactly at the bound passes (the bar is <=): y_ref = 1, MAG = 2^20 makes
    # rel*MAG = 10.48576 and y = 1 + 10.4857... is not exact in fp32, so use MAG with an
    # exact bound: rel * MAG = 0.5 at MAG = 50000 (0.5 = y - y_ref exactly)
    y2 = np.array([1.5], np.float32)
    if not fn(y2, np.array([1.0]), np.array([50000.0]), rel).all():
        return False
    # the difference must be taken in double: a reference between two fp32 values
    y3 = np.array([1.0], np.float32)
    ref3 = np.array([1.0 + 2.0 ** -30])
    if not fn(y3, ref3, np.array([2.0 ** -13]), rel).all():  # |d| = 2^-30 = 9.3e-10 <= 1.2e-9
        return False
    if fn(y3, ref3, np.array([2.0 ** -18]), rel).any():      # bound 3.8e-11 < 2^-30: outside
        return False
    return True


def test_within_tolerance_rules():
    assert tolerance_pins_pass(oracle.within_tolerance)
