"""GPU parity of the quad plans (four consecutive positions per lane, 16-byte LDS reads, the
shifted words of a non-zero taken from the next lane by a DPP FMA) against the oracle.

A non-zero's class is its LDS offset mod 4, so every (r, s) tap class and every slot
count the quad kernels exist for (3, 5, 9) is exercised, with stride 1, 2 and 4, the wide
and the padded staging layouts, split rows, class runs longer than the 128-entry ring that
holds a consumer's entries, and batch sizes that leave ragged last tiles.  Same bar as the
other parity tests; one non-zero per output is bit-exact."""
import numpy as np
import pytest

import oracle
import sparse_weight_direct_amd as sc
import workloads
from gpu_util import assert_layer_parity, assert_parity, gpu_sparse

pytestmark = pytest.mark.gpu

QUAD_TILE = 504


def _quad(monkeypatch, extra=""):
    monkeypatch.setenv("SPARSECONV_PLAN", "QUAD=1" + ("," + extra if extra else ""))


def _check(d, stride, pad, what, mask=None):
    m = d["mask"] if mask is None else mask
    r = oracle.reference(d["x"], d["w"], m, stride, pad)
    y, h = gpu_sparse(d["x"], d["w"], m, stride, pad)
    assert h.info()["tile_pixels"] == QUAD_TILE, h.info()
    assert_parity(y, r["y64"], r["mag"], what)
    return y, h


@pytest.mark.parametrize("name", ["tiny", "mid", "late", "first11", "pw1x1"])
def test_layer_full_parity_quad(name, monkeypatch):
    _quad(monkeypatch)
    d = workloads.make(name)
    L = d["layer"]
    _check(d, L.stride, L.pad, "quad " + name)


@pytest.mark.parametrize("name", ["imb80", "imb90", "imb95", "imb99"])
def test_full_size_quad(name, monkeypatch):
    """The timed workload family at full size through the quad plan, against the oracle on
    every output."""
    _quad(monkeypatch)
    d = workloads.make(name)
    L = d["layer"]
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad)
    assert h.info()["tile_pixels"] == QUAD_TILE
    assert_layer_parity(name, y, "quad " + name)


@pytest.mark.parametrize("plan", ["OCW=9", "OCW=5", "OCW=3", "OCW=9,D=2", "OCW=5,CC=3", "OCW=3,D=4,CC=1",
                                  "OCW=9,NARROW"])
@pytest.mark.parametrize("pad", [0, 1, 2])
def test_every_quad_plan_shape(plan, pad, monkeypatch):
    """Slot counts, ring depths, chunk sizes (a ragged last chunk with CC=3) and both staging
    layouts (W % 4 == 0: wide unless NARROW)."""
    _quad(monkeypatch, plan)
    d = workloads.make_custom(3, 20, 23, 36, 50, 3, 3, 1, pad, 0.15, 90 + pad)
    _check(d, 1, pad, f"{plan} pad {pad}")


def _cases(count, seed0):
    rng = np.random.default_rng(seed0)
    keeps = [0.9, 0.5, 0.1, 0.0, 1.0]
    out = []
    for i in range(count):
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        stride, pad = int(rng.integers(1, 5)), int(rng.integers(0, 3))
        H = int(rng.integers(max(1, R - 2 * pad), 40))
        W = int(rng.integers(max(1, S - 2 * pad), 40))
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 40)), H, W, int(rng.integers(1, 70)), R, S, stride,
                    pad, keeps[i % 5], 7000 + i))
    return out


@pytest.mark.parametrize("c", _cases(30, 17), ids=lambda c: "N{}C{}H{}W{}M{}R{}S{}st{}p{}k{}".format(*c[:10]))
def test_random_shapes_quad(c, monkeypatch):
    _quad(monkeypatch)
    N, C, H, W, M, R, S, st, pad, keep, seed = c
    d = workloads.make_custom(N, C, H, W, M, R, S, st, pad, keep, seed)
    _check(d, st, pad, str(c))


@pytest.mark.parametrize("R,S,stride,pad,H,W", [(3, 3, 1, 1, 30, 41), (11, 11, 4, 0, 67, 59), (5, 3, 2, 2, 17, 23),
                                                (1, 1, 1, 0, 7, 7), (4, 4, 1, 0, 20, 24)])
def test_single_nonzero_every_class_bit_exact(R, S, stride, pad, H, W, monkeypatch):
    """One non-zero per output channel, at every tap of the filter in turn across the output
    channels (so every class 0..3 of the LDS offset occurs): each output is one fp32 product,
    identical to the oracle's rounded value bit for bit."""
    _quad(monkeypatch)
    rng = np.random.default_rng(R * 131 + W)
    N, C = 2, 3
    M = R * S
    x = rng.uniform(-1, 1, (N, C, H, W)).astype(np.float32)
    w = np.zeros((M, C, R, S), np.float32)
    for m in range(M):
        w[m, m % C, m // S, m % S] = np.float32(rng.uniform(0.5, 1.5))
    r = oracle.reference(x, w, None, stride, pad)
    y, h = gpu_sparse(x, w, None, stride, pad)
    assert h.info()["tile_pixels"] == QUAD_TILE
    np.testing.assert_array_equal(y.view(np.uint32), r["y"].view(np.uint32))


def test_class_runs_longer_than_the_entry_ring(monkeypatch):
    """Dense 7x7 rows, one row per wavefront (15 equal rows are not split).  The padded pitch
    is 15 words, so tap (r, s) has class (15 r + s) mod 4 and every class holds at least 12
    of the 49 taps: with at least 11 channels in a chunk, a slot's run of one class in one
    chunk exceeds the 128 entries of the ring, which is then refilled inside the run."""
    _quad(monkeypatch, "OCW=3,D=2")
    d = workloads.make_custom(2, 32, 9, 9, 15, 7, 7, 1, 3, 1.0, 99)
    y, h = _check(d, 1, 3, "long runs")
    info = h.info()
    per_class = [sum(1 for r in range(7) for s in range(7) if (15 * r + s) % 4 == k) for k in range(4)]
    assert min(per_class) >= 12
    assert info["chunk_channels"] * min(per_class) > 128 and info["split_pieces"] == 0, info


def test_split_rows_quad(monkeypatch):
    """Dense channels split over several wavefronts (partial sums in LDS buffers, combined in
    piece order), with many work units per workgroup; twice, bit-identical."""
    _quad(monkeypatch, "OCW=3")
    d = workloads.make_custom(6, 24, 40, 40, 36, 3, 3, 1, 1, 0.03, 41)
    mask = d["mask"].copy()
    mask[3] = 1
    mask[20] = 1
    y, h = _check(d, 1, 1, "split quad", mask=mask)
    assert h.info()["split_pieces"] > 0
    y2, _ = gpu_sparse(d["x"], d["w"], mask, 1, 1, handle=h)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_empty_rows_and_all_zero_weights_quad(monkeypatch):
    _quad(monkeypatch)
    d = workloads.make_custom(2, 8, 12, 12, 40, 3, 3, 1, 1, 0.2, 21)
    mask = d["mask"].copy()
    mask[::3] = 0
    y, _ = gpu_sparse(d["x"], d["w"], mask, 1, 1)
    assert np.all(y[:, ::3] == 0) and not np.signbit(y[:, ::3]).any()
    y0, _ = gpu_sparse(d["x"], d["w"], np.zeros_like(mask), 1, 1)
    assert np.all(y0 == 0) and not np.signbit(y0).any()


def test_batch_sizes_share_one_quad_handle(monkeypatch):
    """N is a forward-time argument: ragged last tiles at several batch sizes."""
    _quad(monkeypatch)
    d = workloads.make("late")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"])
    assert h.info()["tile_pixels"] == QUAD_TILE
    for n in (1, 3, 7):
        x = d["x"][:n]
        r = oracle.reference(x, d["w"], d["mask"], L.stride, L.pad)
        y, _ = gpu_sparse(x, d["w"], d["mask"], L.stride, L.pad, handle=h)
        assert_parity(y, r["y64"], r["mag"], f"late N={n}")


def test_default_handles_offer_a_quad_variant():
    """Handles with 8-byte entries carry a quad plan among their variants; the forward's
    cost model picks between them (parity of whichever it picks is covered by every other
    test file)."""
    d = workloads.make("imb95", n_override=1)
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"])
    assert h.info()["plan_variants"] >= 2
    h16 = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                    flags=sc.SC_PACK_FP16_WORD)
    assert h16.info()["tile_pixels"] != QUAD_TILE
