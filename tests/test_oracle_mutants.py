"""Planted mistakes in the oracle (CPU only): each mutant is a copy of oracle.c with one
plausible error (a wrong sign, a transposed index, an off-by-one bound, swapped dims).  The
pins must reject every mutant, which shows they are sharp enough to trust the oracle."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "pad_sign": ("int64_t iy = e * stride - pad + r;\n            if (iy < 0 || iy >= H) continue;",
                 "int64_t iy = e * stride + pad + r;\n            if (iy < 0 || iy >= H) continue;"),
    "r_s_transposed": ("int64_t r = (col / S) % R;\n        int64_t s = col % S;\n        double v",
                       "int64_t r = col % R;\n        int64_t s = (col / R) % S;\n        double v"),
    "row_bound_off_by_one": ("if (iy < 0 || iy >= H) continue;\n            for",
                             "if (iy < 0 || iy >= H - 1) continue;\n            for"),
    "stride_dropped_x": ("int64_t ix = f * stride - pad + s;\n                if (ix < 0 || ix >= W) continue;\n                double prod = v",
                         "int64_t ix = f - pad + s;\n                if (ix < 0 || ix >= W) continue;\n                double prod = v"),
    "stretch_h_w_swapped": ("off[j] = (uint32_t)(((int64_t)c * H + r) * W + s);",
                            "off[j] = (uint32_t)(((int64_t)c * W + r) * H + s);"),
    "value_sign": ("double v = (double)value[j];", "double v = -(double)value[j];"),
    "output_transposed": ("yp[e * F + f] += prod;", "yp[f * E + e] += prod;"),
    # packed-word form ([T] Sec. 5.3 / Fig. 4)
    "fp16_truncates": ("double n = rint(a / ldexp(1.0, e - 10));", "double n = floor(a / ldexp(1.0, e - 10));"),
    "fp16_ties_away": ("double n = rint(a / ldexp(1.0, e - 10));", "double n = round(a / ldexp(1.0, e - 10));"),
    "fp16_subnormal_quantum": ("double n = rint(a / ldexp(1.0, -24));", "double n = rint(a / ldexp(1.0, -23));"),
    "fp16_exponent_bias": ("(uint16_t)((e + 15) << 10)", "(uint16_t)((e + 14) << 10)"),
    "word_px_py_swapped": ("words[j] = oracle_pack_word(value[j], c, s, r);",
                           "words[j] = oracle_pack_word(value[j], c, r, s);"),
    "word_ic_shift": ("((uint32_t)ic << 8)", "((uint32_t)ic << 9)"),
    "word_decode_col_order": ("colidx[j] = (ic * R + py) * S + px;", "colidx[j] = (ic * S + px) * R + py;"),
    # the per-plane form that checks full-size layers plane by plane
    "planes_n_m_swapped": ("conv_plane_csr(planes_sel[q] / M, planes_sel[q] % M,",
                           "conv_plane_csr(planes_sel[q] % M, planes_sel[q] / M,"),
    "planes_split_by_images": ("conv_plane_csr(planes_sel[q] / M, planes_sel[q] % M,",
                               "conv_plane_csr(planes_sel[q] / N, planes_sel[q] % N,"),
}


def _word_pins_pass():
    """Compact packed-word pins: binary16 values from the format's definition (with ties),
    numpy's float16 cast, a literal word, and the packed-word oracle against the
    definitional form on numpy-rounded weights (R != S)."""
    for v, bits in [(1.0, 0x3C00), (65504.0, 0x7BFF), (2.0 ** -24, 0x0001), (1.0 + 3 * 2.0 ** -11, 0x3C02),
                    (1.0 + 2.0 ** -11, 0x3C00),
                    (2047.5, 0x6800), (3 * 2.0 ** -25, 0x0002)]:
        if oracle.fp16_bits(v) != bits:
            return False
    rng = np.random.default_rng(3)
    vals = (rng.standard_normal(2000) * np.exp2(rng.integers(-26, 15, 2000))).astype(np.float32)
    if any(oracle.fp16_bits(float(v)) != int(np.float16(v).view(np.uint16)) for v in vals):
        return False
    if oracle.pack_word(1.0, 0xAB, 0xC, 0xD) != 0x3C00ABCD:
        return False
    d = workloads.make_custom(1, 3, 7, 9, 3, 2, 3, 1, 1, 0.6, 77)
    r16 = oracle.reference_fp16(d["x"], d["w"], d["mask"], 1, 1)
    y, mag = oracle.conv_def(d["x"], d["w"].astype(np.float16).astype(np.float32), d["mask"], 1, 1)
    return bool(np.all(np.abs(r16["y64"] - y) <= 1e-12 * mag + 1e-300))


def _pins_pass():
    """A compact run of the pins: torch float64 conv2d on non-square strided/padded shapes,
    the stretched-offset gather, and the packed-word pins."""
    if not _word_pins_pass():
        return False
    for seed, (N, C, H, W, M, R, S, st, p) in enumerate([(2, 3, 9, 7, 4, 3, 2, 2, 1),
                                                          (1, 2, 8, 11, 3, 2, 4, 1, 2),
                                                          (1, 2, 12, 12, 2, 3, 3, 1, 1)]):
        d = workloads.make_custom(N, C, H, W, M, R, S, st, p, 0.7, 900 + seed)
        r = oracle.reference(d["x"], d["w"], d["mask"], st, p)
        t = torch.nn.functional.conv2d(torch.from_numpy(d["x"]).double(),
                                       torch.from_numpy(d["w_masked"]).double(), stride=st, padding=p).numpy()
        if t.shape != r["y64"].shape or not np.all(np.abs(t - r["y64"]) <= 1e-12 * r["mag"] + 1e-300):
            return False
    # the per-plane form: every (n, m) plane, in a shuffled order, equals the full form
    d = workloads.make_custom(3, 4, 9, 8, 5, 3, 2, 2, 1, 0.6, 950)
    rowptr, colidx, value = oracle.csr_from_dense(d["w"], d["mask"])
    y64, mag = oracle.conv_csr(d["x"], rowptr, colidx, value, 5, 3, 2, 2, 1)
    planes = np.random.default_rng(1).permutation(15)
    yp, mp = oracle.conv_csr_planes(d["x"], rowptr, colidx, value, 5, 3, 2, 2, 1, planes)
    if not (np.array_equal(yp, y64.reshape(15, *y64.shape[2:])[planes]) and
            np.array_equal(mp, mag.reshape(15, *mag.shape[2:])[planes])):
        return False
    C, R, S, H, W = 3, 2, 3, 5, 7
    off = oracle.stretch(np.arange(C * R * S, dtype=np.int32), C, R, S, H, W).reshape(C, R, S)
    x = np.arange(C * H * W, dtype=np.float32).reshape(C, H, W)
    for c in range(C):
        for r_ in range(R):
            for s in range(S):
                if x.reshape(-1)[off[c, r_, s]] != x[c, r_, s]:
                    return False
    return True


def test_unmutated_oracle_passes_compact_pins():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_rejected(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-o", str(so_path), str(c_path), "-lm"])
    saved = oracle._lib
    try:
        oracle._lib = oracle._bind(str(so_path))
        assert not _pins_pass(), f"mutant {name} survived the pins"
    finally:
        oracle._lib = saved


# Planted mistakes in the comparator (oracle.within_tolerance), each a plausible slip.
def _tol_exact(y_gpu, y_ref64, mag, rel=1e-5):  # the comparator as written
    return oracle.within_tolerance(y_gpu, y_ref64, mag, rel)


def _tol_strict(y_gpu, y_ref64, mag, rel=1e-5):  # "<" where the bar is "<="
    d = np.abs(y_gpu.astype(np.float64) - y_ref64)
    ok = d < rel * mag
    zero = mag == 0
    ok[zero] = y_gpu[zero] == 0
    return ok


def _tol_absolute(y_gpu, y_ref64, mag, rel=1e-5):  # absolute instead of relative bound
    d = np.abs(y_gpu.astype(np.float64) - y_ref64)
    ok = d <= rel
    zero = mag == 0
    ok[zero] = y_gpu[zero] == 0
    return ok


def _tol_no_zero_rule(y_gpu, y_ref64, mag, rel=1e-5):  # forgets "mag == 0 => exactly 0"
    d = np.abs(y_gpu.astype(np.float64) - y_ref64)
    return d <= rel * mag + 1e-30


def _tol_nan_passes(y_gpu, y_ref64, mag, rel=1e-5):  # NaN compares as "not outside"
    d = np.abs(y_gpu.astype(np.float64) - y_ref64)
    ok = ~(d > rel * mag)
    zero = mag == 0
    ok[zero] = y_gpu[zero] == 0
    return ok


def _tol_fp32_diff(y_gpu, y_ref64, mag, rel=1e-5):  # difference taken in fp32
    d = np.abs(y_gpu - y_ref64.astype(np.float32)).astype(np.float64)
    ok = d <= rel * mag
    zero = mag == 0
    ok[zero] = y_gpu[zero] == 0
    return ok


TOL_MUTANTS = {"strict": _tol_strict, "absolute": _tol_absolute, "no_zero_rule": _tol_no_zero_rule,
               "nan_passes": _tol_nan_passes, "fp32_diff": _tol_fp32_diff}


def test_comparator_pins_accept_the_comparator():
    from test_oracle_pins import tolerance_pins_pass
    assert tolerance_pins_pass(_tol_exact)


@pytest.mark.parametrize("name", sorted(TOL_MUTANTS))
def test_comparator_mutant_is_rejected(name):
    from test_oracle_pins import tolerance_pins_pass
    assert not tolerance_pins_pass(TOL_MUTANTS[name]), f"comparator mutant {name} survived the pins"
