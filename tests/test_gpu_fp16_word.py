"""GPU parity of the 32-bit packed-word form (SC_PACK_FP16_WORD) against the oracle.

The oracle encodes the non-zeros as the words of Tuteja et al., "Theoretical and Empirical
Analysis of Sparse Convolution", Sec. 5.3 / Fig. 4, decodes them, and convolves with the
decoded fp16 weights in double precision; the kernel widens the same fp16 weights to fp32
and accumulates in fp32.  Same bar as the fp32 path: |gpu - oracle| <= 1e-5 * sum|w16*x|."""
import numpy as np
import pytest
import torch

import oracle
import sparse_weight_direct_amd as sc
import workloads
from gpu_util import assert_parity, gpu_sparse

pytestmark = pytest.mark.gpu


def _handle16(w, mask, H, W, stride, pad):
    M, C, R, S = w.shape
    return sc.Handle(M, C, R, S, H, W, stride, pad, values=w, mask=mask, flags=sc.SC_PACK_FP16_WORD)


@pytest.mark.parametrize("name", ["tiny", "mid", "late", "first11"])
def test_layer_full_parity_fp16_word(name):
    d = workloads.make(name)
    L = d["layer"]
    r = oracle.reference_fp16(d["x"], d["w"], d["mask"], L.stride, L.pad)
    h = _handle16(d["w"], d["mask"], L.H, L.W, L.stride, L.pad)
    assert h.info()["entry_bytes"] == 4
    y, _ = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad, handle=h)
    assert_parity(y, r["y64"], r["mag"], name + " fp16 word")
    rowptr, words = h.export_words()
    np.testing.assert_array_equal(rowptr, r["rowptr"])
    np.testing.assert_array_equal(words, r["words"])


@pytest.mark.parametrize("name", ["imb80", "imb90", "imb95", "imb99"])
def test_full_size_sampled_planes_fp16_word(name):
    """The 112x112 batch-8 layers in the benchmark's launch configuration: 64 sampled planes
    (the densest and emptiest channels, random ones; first, last and random images) against
    the oracle on the fp16-rounded weights."""
    d = workloads.make(name)
    L = d["layer"]
    h = _handle16(d["w"], d["mask"], L.H, L.W, L.stride, L.pad)
    y, _ = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad, handle=h)
    assert np.isfinite(y).all()
    rowptr, colidx, value = oracle.csr_from_dense(d["w"], d["mask"])
    col16, val16 = oracle.csr_from_words(oracle.words_from_csr(colidx, value, L.C, L.R, L.S), L.R, L.S)
    rows = np.diff(rowptr)
    rng = np.random.default_rng(L.seed + 16)
    ms = {int(rows.argmax()), int(rows.argmin())} | set(int(m) for m in rng.choice(L.M, 14, replace=False))
    planes = sorted({n * L.M + m for n in (0, L.N - 1, int(rng.integers(1, L.N - 1)), int(rng.integers(1, L.N - 1)))
                     for m in ms})[:64]
    y64, mag = oracle.conv_csr_planes(d["x"], rowptr, col16, val16, L.M, L.R, L.S, L.stride, L.pad, planes)
    got = np.stack([y[p // L.M, p % L.M] for p in planes])
    assert_parity(got, y64, mag, name + " fp16 word")


@pytest.mark.parametrize("plan", ["K=1,OCW=1", "K=2,OCW=5", "K=4,OCW=2,CC=3", "K=8,OCW=5,D=2", "K=16,OCW=3",
                                  "K=7,OCW=9,D=4", "K=6,OCW=1,NARROW"])
def test_every_plan_shape_fp16_word(plan, monkeypatch):
    monkeypatch.setenv("SPARSECONV_PLAN", plan)
    d = workloads.make_custom(2, 20, 33, 37, 24, 3, 3, 1, 1, 0.3, 616)
    r = oracle.reference_fp16(d["x"], d["w"], d["mask"], 1, 1)
    h = _handle16(d["w"], d["mask"], 33, 37, 1, 1)
    y, _ = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1, handle=h)
    assert_parity(y, r["y64"], r["mag"], "fp16 word " + plan)


def test_split_rows_fp16_word():
    d = workloads.make_custom(6, 24, 40, 40, 36, 3, 3, 1, 1, 0.03, 41)
    mask = d["mask"].copy()
    mask[3] = 1
    mask[20] = 1
    r = oracle.reference_fp16(d["x"], d["w"], mask, 1, 1)
    h = _handle16(d["w"], mask, 40, 40, 1, 1)
    y, _ = gpu_sparse(d["x"], d["w"], mask, 1, 1, handle=h)
    assert h.info()["split_pieces"] > 0
    assert_parity(y, r["y64"], r["mag"], "fp16 word split")


@pytest.mark.parametrize("R,S,stride,pad,H,W", [(3, 3, 1, 1, 30, 41), (11, 11, 4, 0, 67, 59), (5, 3, 2, 2, 17, 23)])
def test_single_nonzero_bit_exact_fp16_word(R, S, stride, pad, H, W):
    """One non-zero per output channel: every output is one fp32 product of the widened fp16
    weight and an input, the same value as the oracle's double product rounded once."""
    rng = np.random.default_rng(R * 100 + S)
    C, M = 5, 7
    x = rng.uniform(-1, 1, (2, C, H, W)).astype(np.float32)
    w = np.zeros((M, C, R, S), np.float32)
    for m in range(M):
        w[m, rng.integers(C), rng.integers(R), rng.integers(S)] = rng.uniform(-2, 2)
    r = oracle.reference_fp16(x, w, None, stride, pad)
    y, _ = gpu_sparse(x, w, None, stride, pad, handle=_handle16(w, None, H, W, stride, pad))
    np.testing.assert_array_equal(y.view(np.uint32), r["y"].view(np.uint32))


def test_fp16_and_fp32_handles_agree_on_fp16_exact_weights():
    """Weights that fp16 holds exactly: the two entry formats of the LDS-tile kernel compute
    the same products in the same order, so their outputs are identical bit for bit."""
    d = workloads.make("mid")
    L = d["layer"]
    w16 = d["w"].astype(np.float16).astype(np.float32)
    y32, _ = gpu_sparse(d["x"], w16, d["mask"], L.stride, L.pad, flags=sc.SC_PACK_LDS_TILE)
    y16, _ = gpu_sparse(d["x"], w16, d["mask"], L.stride, L.pad,
                        handle=_handle16(w16, d["mask"], L.H, L.W, L.stride, L.pad))
    np.testing.assert_array_equal(y16.view(np.uint32), y32.view(np.uint32))


def _cases(count, seed0):
    rng = np.random.default_rng(seed0)
    out = []
    for i in range(count):
        R, S = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        st, p = int(rng.integers(1, 5)), int(rng.integers(0, 3))
        H = int(rng.integers(max(1, R - 2 * p), 48))
        W = int(rng.integers(max(1, S - 2 * p), 48))
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 40)), H, W, int(rng.integers(1, 70)), R, S, st, p,
                    [0.9, 0.5, 0.1, 0.0, 1.0, 0.03][i % 6], 7000 + i))
    return out


@pytest.mark.parametrize("c", _cases(24, 5), ids=lambda c: "N{}C{}H{}W{}M{}R{}S{}st{}p{}k{}".format(*c[:10]))
def test_random_shapes_fp16_word(c):
    N, C, H, W, M, R, S, st, p, keep, seed = c
    d = workloads.make_custom(N, C, H, W, M, R, S, st, p, keep, seed)
    r = oracle.reference_fp16(d["x"], d["w"], d["mask"], st, p)
    h = _handle16(d["w"], d["mask"], H, W, st, p)
    y, _ = gpu_sparse(d["x"], d["w"], d["mask"], st, p, handle=h)
    assert_parity(y, r["y64"], r["mag"], "fp16 word random")


def test_batch_sizes_share_one_fp16_word_handle():
    """N is a forward-time argument, and the forward picks a plan variant per N."""
    d = workloads.make("late")
    L = d["layer"]
    h = _handle16(d["w"], d["mask"], L.H, L.W, L.stride, L.pad)
    for n in (1, 5, 32):
        x = d["x"][:n]
        r = oracle.reference_fp16(x, d["w"], d["mask"], L.stride, L.pad)
        y, _ = gpu_sparse(x, d["w"], d["mask"], L.stride, L.pad, handle=h)
        assert_parity(y, r["y64"], r["mag"], f"late fp16 word N={n}")
