"""Roofline arithmetic against the numbers the page prints (CPU only).

Tuteja et al., Sec. 4.1 Table 1 (AI vs sparsity, one decimal), the dense AI of about 96
(same section) and the four FP32 ridge points of Sec. 4; fixture tests/golden/table1_ai.txt."""
import os

import pytest

from sparse_weight_direct_amd import roofline

GOLD = os.path.join(os.path.dirname(__file__), "golden", "table1_ai.txt")


def _rows():
    out = []
    for line in open(GOLD):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


def test_table1_arithmetic_intensity():
    rows = [r for r in _rows() if r[0][0] == "0"]
    assert len(rows) == 9
    for s, ai in rows:
        # the page's 94% entry prints 5.7 where the formula gives 5.76: within 0.1 everywhere
        assert abs(roofline.ai_table1(float(s)) - float(ai)) < 0.1, (s, ai, roofline.ai_table1(float(s)))


def test_dense_ai_about_96():
    (row,) = [r for r in _rows() if r[0] == "dense"]
    assert abs(roofline.ai_dense() - float(row[1])) < 0.5


def test_ridge_points():
    for _, name, peak, bw, exp in [r for r in _rows() if r[0] == "ridge"]:
        assert abs(roofline.ridge(float(peak), float(bw)) - float(exp)) < 0.01, name


def test_algorithmic_bytes_and_flops_of_a_layer():
    # 112x112 layer, batch 8, C = M = 128, nnz = 1000
    b = roofline.algorithmic_bytes(8, 128, 112, 112, 128, 112, 112, 1000)
    assert b == 4 * 8 * 128 * 112 * 112 * 2 + 4 * (2000 + 129)
    assert roofline.effective_flops(1000, 8, 112, 112) == 2 * 1000 * 8 * 112 * 112


WINO = os.path.join(os.path.dirname(__file__), "golden", "winograd_tables.txt")


def _wino_tables():
    tabs = {}
    for line in open(WINO):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "ic":
            tabs[f[1]] = {"ic": [int(v) for v in f[2:]], "rows": []}
        else:
            tabs[f[0]]["rows"].append((int(f[1]), [float(v) for v in f[2:]]))
    return tabs


def test_table2_winograd_speedup_a100():
    """All 25 printed cells of Table 2 (A100, N=32, 256x256) to one decimal, with the roofline
    times max(T_comp, T_comm) of Sec. 4.2 at 19.5 TFLOP/s and 1.5 TB/s and a Winograd
    operation reduction of 2 (the text says 1.5x and quotes 2 TB/s for the ridge point;
    neither reproduces the printed table)."""
    t = _wino_tables()["T2"]
    for oc, vals in t["rows"]:
        for ic, v in zip(t["ic"], vals):
            got = roofline.winograd_speedup(oc, ic, 19.5, 1.5, N=32, H=256, reduction=2.0)
            assert round(got, 1) == v, (oc, ic, got, v)


def test_table3_winograd_speedup_jetson_nano():
    """Table 3 (Tegra X1 at 0.236 TFLOP/s and 25.6 GB/s, N=8, 128x128): 22 of 25 cells to one
    decimal; three print 0.07-0.1 above the model (listed), no bandwidth reproduces all."""
    t = _wino_tables()["T3"]
    off = {(24, 24), (32, 32), (48, 24)}
    for oc, vals in t["rows"]:
        for ic, v in zip(t["ic"], vals):
            got = roofline.winograd_speedup(oc, ic, 0.236, 0.0256, N=8, H=128, reduction=2.0)
            if (oc, ic) in off:
                assert 0.0 < v - got <= 0.1 + 1e-9, (oc, ic, got, v)
            else:
                assert round(got, 1) == v, (oc, ic, got, v)


def test_winograd_speedup_limits():
    """IC = 1: both memory-bound on the same activation bytes (speedup 1.0); large channels:
    both compute-bound, speedup = 1 / (reduction * (1 - S))."""
    assert abs(roofline.winograd_speedup(64, 1, 19.5, 1.5) - 1.0) < 0.02
    assert abs(roofline.winograd_speedup(4096, 4096, 19.5, 1.5) - 1.0 / (2.0 * 0.1)) < 1e-9
    assert abs(roofline.winograd_speedup(4096, 4096, 19.5, 1.5, sparsity=0.95, reduction=1.5) - 1.0 / (1.5 * 0.05)) < 1e-9


def test_report_runs():
    text = roofline.report()
    assert "Table 2" in text and "9.75" in text and "MI355X" in text
