"""Pins of the oracle's packed-word form (CPU only).

The packed word of Tuteja et al., "Theoretical and Empirical Analysis of Sparse
Convolution", Sec. 5.3 and Fig. 4, holds one non-zero in 32 bits: the fp16 weight in bits
31-16, the input channel ic in bits 15-8, the kernel column offset px in bits 7-4 and the
kernel row offset py in bits 3-0.  The oracle's fp16 rounding is pinned to
  * IEEE 754 binary16 values that follow from the format's definition (1.0 = 0x3C00, the
    largest finite 65504 = 0x7BFF, the smallest subnormal 2^-24 = 0x0001, ties to even);
  * numpy's float16 cast (a library routine the oracle does not use), bit for bit, on every
    binade and on all 65536 half values;
and the word layout to literal words read off the figure's bit positions.  The convolution
over decoded words is pinned to the definitional form on numpy-rounded weights.
"""
import numpy as np
import pytest

import oracle
import workloads

# value -> binary16 bits, each from the format's definition:
# sign | biased exponent (bias 15) << 10 | 10-bit fraction; subnormals n * 2^-24.
TEXTBOOK = [
    (1.0, 0x3C00), (-2.0, 0xC000), (0.5, 0x3800), (1.5, 0x3E00), (-0.5, 0xB800),
    (65504.0, 0x7BFF),                 # largest finite half
    (65520.0, 0x7C00),                 # halfway to 2^16 rounds to even: overflow to +inf
    (-65520.0, 0xFC00),
    (2.0 ** -14, 0x0400),              # smallest normal
    (2.0 ** -24, 0x0001),              # smallest subnormal
    (2.0 ** -25, 0x0000),              # halfway between 0 and 2^-24: ties to even (0)
    (3 * 2.0 ** -25, 0x0002),          # halfway between 1 and 2 quanta: ties to even (2)
    (1.0 + 2.0 ** -11, 0x3C00),        # halfway between 1 and 1 + 2^-10: even is 1
    (1.0 + 3 * 2.0 ** -11, 0x3C02),    # halfway between 1 + 2^-10 and 1 + 2^-9: even is +2
    (2047.5, 0x6800),                  # 2047.5 -> 2048 (tie to the even significand, next binade)
    (0.0, 0x0000), (-0.0, 0x8000),
    (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
]


@pytest.mark.parametrize("v,bits", TEXTBOOK, ids=[f"{v!r}" for v, _ in TEXTBOOK])
def test_fp16_textbook_values(v, bits):
    assert oracle.fp16_bits(v) == bits
    back = oracle.fp16_value(bits)
    if bits & 0x7C00 != 0x7C00:
        assert back == np.float64(np.float16(v)) or (v == 0.0 and back == 0.0)


def test_fp16_nan_stays_nan():
    h = oracle.fp16_bits(float("nan"))
    assert (h & 0x7C00) == 0x7C00 and (h & 0x3FF) != 0
    assert np.isnan(oracle.fp16_value(h))


def test_fp16_matches_numpy_cast_on_every_binade():
    """Bit-for-bit agreement with numpy's float16 cast (round to nearest even) on random fp32
    values from 2^-30 to 2^17, both signs, plus the exact halfway points of every binade."""
    rng = np.random.default_rng(16)
    e = rng.uniform(-30, 17, 20000)
    v = (np.sign(rng.uniform(-1, 1, e.size)) * np.exp2(e)).astype(np.float32)
    # halfway points between adjacent halves (exactly representable in fp32)
    h = np.arange(0, 0x7BFF, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    h1 = (np.arange(0, 0x7BFF, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    mids = ((h + h1) / 2).astype(np.float32)
    allv = np.concatenate([v, mids, -mids])
    with np.errstate(over="ignore"):
        want = allv.astype(np.float16).view(np.uint16)
    got = np.array([oracle.fp16_bits(float(x)) for x in allv], np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(allv[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_fp16_value_of_every_half_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32)
    want = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_value(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # and every finite half round-trips through the encoder
    fin = ~nan & ~np.isinf(want)
    rt = np.array([oracle.fp16_bits(float(x)) for x in want[fin]], np.uint32)
    assert np.array_equal(rt, bits[fin])


# literal words read off the figure's bit positions: value | ic | px | py as hex nibbles
WORDS = [
    ((1.0, 0xAB, 0xC, 0xD), 0x3C00ABCD),
    ((-0.5, 0x01, 0x2, 0x3), 0xB8000123),
    ((1.5, 0xFF, 0xF, 0xF), 0x3E00FFFF),
    ((0.0, 0x00, 0x0, 0x0), 0x00000000),
    ((65504.0, 0x80, 0x1, 0x0), 0x7BFF8010),
]


@pytest.mark.parametrize("fields,word", WORDS, ids=[hex(w) for _, w in WORDS])
def test_word_layout_literals(fields, word):
    assert oracle.pack_word(*fields) == word
    v, ic, px, py = oracle.unpack_word(word)
    assert (v, ic, px, py) == (float(np.float16(fields[0])), fields[1], fields[2], fields[3])


def test_word_field_ranges_are_enforced():
    with pytest.raises(ValueError):
        oracle.pack_word(1.0, 256, 0, 0)
    with pytest.raises(ValueError):
        oracle.pack_word(1.0, 0, 16, 0)
    with pytest.raises(ValueError):
        oracle.words_from_csr(np.zeros(1, np.int32), np.ones(1, np.float32), 257, 3, 3)
    with pytest.raises(ValueError):
        oracle.words_from_csr(np.zeros(1, np.int32), np.ones(1, np.float32), 8, 17, 3)


def test_words_from_csr_place_row_and_column():
    """One non-zero at input channel 2, filter row 1, column 0 of a 3x3 filter: px = 0 (the
    column) and py = 1 (the row); value 1.5 = 0x3E00."""
    w = np.zeros((1, 3, 3, 3), np.float32)
    w[0, 2, 1, 0] = 1.5
    rowptr, colidx, value = oracle.csr_from_dense(w)
    words = oracle.words_from_csr(colidx, value, 3, 3, 3)
    assert words.tolist() == [0x3E000201]
    # a 2x5 filter: row 1, column 4 of channel 7 -> py = 1, px = 4
    w = np.zeros((1, 8, 2, 5), np.float32)
    w[0, 7, 1, 4] = -2.0
    _, colidx, value = oracle.csr_from_dense(w)
    assert oracle.words_from_csr(colidx, value, 8, 2, 5).tolist() == [0xC0000741]
    col2, val2 = oracle.csr_from_words(np.array([0xC0000741], np.uint32), 2, 5)
    assert col2.tolist() == colidx.tolist() and val2.tolist() == [-2.0]


@pytest.mark.parametrize("shape", [(2, 3, 9, 7, 4, 2, 3, 2, 1), (1, 5, 8, 11, 3, 4, 2, 1, 2),
                                   (1, 4, 12, 12, 6, 3, 3, 1, 1)])
def test_reference_fp16_is_conv_of_numpy_rounded_weights(shape):
    """The packed-word oracle equals the definitional convolution applied to the weights
    rounded by numpy's float16 cast (R != S shapes catch a px/py swap)."""
    N, C, H, W, M, R, S, st, p = shape
    d = workloads.make_custom(N, C, H, W, M, R, S, st, p, 0.6, 4242 + C)
    r16 = oracle.reference_fp16(d["x"], d["w"], d["mask"], st, p)
    w16 = d["w"].astype(np.float16).astype(np.float32)
    y, mag = oracle.conv_def(d["x"], w16, d["mask"], st, p)
    assert np.array_equal(r16["y64"], y) or np.all(np.abs(r16["y64"] - y) <= 1e-12 * mag)
    assert np.array_equal(r16["values"], w16.reshape(M, -1)[d["mask"].reshape(M, -1) != 0])
    # weights already fp16-exact: identical to the fp32 oracle
    d["w"] = w16
    r32 = oracle.reference(d["x"], w16, d["mask"], st, p)
    r16b = oracle.reference_fp16(d["x"], w16, d["mask"], st, p)
    assert np.array_equal(r32["y64"], r16b["y64"])
