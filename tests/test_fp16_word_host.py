"""The 32-bit packed-word form (SC_PACK_FP16_WORD) on the host (CPU only, no GPU calls).

Tuteja et al., "Theoretical and Empirical Analysis of Sparse Convolution", Sec. 5.3 and
Fig. 4: one u32 per non-zero with the fp16 weight, the input channel and the kernel column
and row offsets.  The library's words and fp16-rounded values are compared bit for bit with
the oracle's encoder, and its fp16 rounding with numpy's float16 cast."""
import numpy as np
import pytest

import oracle
import sparse_weight_direct_amd as sc
import workloads


def _status(fn):
    try:
        fn()
        return sc.SC_OK, ""
    except sc.SparseConvError as e:
        return e.status, str(e)


def _pack16(d, L, flags=0):
    return sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                     flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_FP16_WORD | flags)


@pytest.mark.parametrize("name", ["tiny", "mid", "late", "imb95", "first11"])
def test_words_bit_exact_vs_oracle(name):
    d = workloads.make(name, n_override=1)
    L = d["layer"]
    h = _pack16(d, L)
    rowptr, words = h.export_words()
    o_rowptr, o_col, o_val = oracle.csr_from_dense(d["w"], d["mask"])
    o_words = oracle.words_from_csr(o_col, o_val, L.C, L.R, L.S)
    np.testing.assert_array_equal(rowptr, o_rowptr)
    np.testing.assert_array_equal(words, o_words)
    # the canonical export holds the fp16-rounded weights and the same offsets
    rp2, off, val = h.export()
    col16, val16 = oracle.csr_from_words(o_words, L.R, L.S)
    np.testing.assert_array_equal(val.view(np.uint32), val16.view(np.uint32))
    np.testing.assert_array_equal(off, oracle.stretch(col16, L.C, L.R, L.S, L.H, L.W))
    info = h.info()
    assert info["entry_bytes"] == 4
    assert info["packed_bytes"] == (info["nnz"] + L.M + 1) * 4


def test_fp16_rounding_matches_numpy_cast():
    """Many values over every binade (subnormal halves, ties, the overflow edge) in one CSR
    row: the high half of each word is numpy's float16 bits."""
    rng = np.random.default_rng(5)
    e = rng.uniform(-27, 15.99, 4000)
    v = (np.sign(rng.uniform(-1, 1, e.size)) * np.exp2(e)).astype(np.float32)
    h = np.arange(0, 0x7BFF, 31, dtype=np.uint16)
    mids = ((h.view(np.float16).astype(np.float64) + (h + 1).view(np.float16).astype(np.float64)) / 2)
    v = np.concatenate([v, mids.astype(np.float32), -mids.astype(np.float32),
                        np.float32([65504, 65519.996, -65519.996, 2 ** -24, 2 ** -25, 3 * 2 ** -25])])
    v = v[v != 0]
    C, R, S = 256, 16, 16
    nnz = min(v.size, C * R * S)
    v = v[:nnz]
    colidx = np.arange(nnz, dtype=np.int32)
    rowptr = np.array([0, nnz], np.int32)
    ptr = sc.sparseconv_pack(1, C, R, S, 20, 20, 1, 0, values=v, colidx=colidx, rowptr=rowptr,
                             flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_FP16_WORD)
    try:
        _, words = sc.sparseconv_export_words(ptr)
        _, _, val = sc.sparseconv_export_packed(ptr)
    finally:
        sc.sparseconv_destroy(ptr)
    want = v.astype(np.float16)
    np.testing.assert_array_equal((words >> 16).astype(np.uint16), want.view(np.uint16))
    np.testing.assert_array_equal(val, want.astype(np.float32))
    # the low half: channel, column, row of column index c*R*S + r*S + s
    c, r, s = colidx // (R * S), (colidx // S) % R, colidx % S
    np.testing.assert_array_equal(words & 0xFFFF, (c << 8) | (s << 4) | r)


def test_word_limits_and_errors():
    # the 512-channel pointwise layer does not fit the word's 8-bit channel field
    d = workloads.make("pw1x1", n_override=1)
    st, msg = _status(lambda: _pack16(d, d["layer"]))
    assert st == sc.SC_EUNSUPPORTED and "C <= 256" in msg
    w = np.ones((2, 257, 1, 1), np.float32)
    st, msg = _status(lambda: sc.sparseconv_pack(2, 257, 1, 1, 5, 5, 1, 0, values=w,
                                                 flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_FP16_WORD))
    assert st == sc.SC_EUNSUPPORTED and "C <= 256" in msg
    w = np.ones((1, 1, 17, 3), np.float32)
    st, _ = _status(lambda: sc.sparseconv_pack(1, 1, 17, 3, 20, 20, 1, 0, values=w,
                                               flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_FP16_WORD))
    assert st == sc.SC_EUNSUPPORTED
    # 256 channels and 16x16 filters are inside the word's fields
    w = np.zeros((1, 256, 16, 16), np.float32)
    w[0, 255, 15, 15] = 1.0
    h = sc.Handle.from_dense(w, 20, 20, 1, 0, flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_FP16_WORD)
    assert h.export_words()[1].tolist() == [0x3C00FFFF]
    # a finite weight that rounds to infinity is rejected; 65519 rounds to 65504
    for big, ok in ((65520.0, False), (1e6, False), (65519.0, True)):
        w = np.full((1, 1, 3, 3), big, np.float32)
        st, msg = _status(lambda: sc.Handle.from_dense(w, 5, 5, 1, 1, flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_FP16_WORD))
        assert (st == sc.SC_OK) == ok, (big, msg)
        if not ok:
            assert st == sc.SC_EINVAL and "overflows fp16" in msg
    # words of a handle packed without the flag
    w = np.ones((1, 1, 3, 3), np.float32)
    h = sc.Handle.from_dense(w, 5, 5, 1, 1, flags=sc.SC_PACK_HOST_ONLY)
    assert h.info()["entry_bytes"] == 8
    st, msg = _status(lambda: h.export_words())
    assert st == sc.SC_EINVAL and "SC_PACK_FP16_WORD" in msg


def test_all_taps_with_words():
    d = workloads.make("tiny")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w_masked"],
                  flags=sc.SC_PACK_HOST_ONLY | sc.SC_PACK_ALL_TAPS | sc.SC_PACK_FP16_WORD)
    _, words = h.export_words()
    crs = L.C * L.R * L.S
    col = np.tile(np.arange(crs, dtype=np.int32), L.M)
    np.testing.assert_array_equal(words, oracle.words_from_csr(col, d["w_masked"].reshape(-1), L.C, L.R, L.S))
