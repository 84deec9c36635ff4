"""The seeded generators: reproducible, and realizing the stated sparsity recipes (CPU)."""
import numpy as np
import pytest

import workloads


@pytest.mark.parametrize("name", ["tiny", "mid", "first11", "pw1x1"])
def test_reproducible_and_shapes(name):
    a = workloads.make(name)
    b = workloads.make(name)
    L = a["layer"]
    assert a["x"].shape == (L.N, L.C, L.H, L.W) and a["x"].dtype == np.float32
    assert a["w"].shape == (L.M, L.C, L.R, L.S) and a["mask"].dtype == np.uint8
    for k in ("x", "w", "mask"):
        np.testing.assert_array_equal(a[k], b[k])
    assert np.all(a["w_masked"][a["mask"] == 0] == 0)


def test_exact_keep_counts():
    for name in ["mid", "first11", "pw1x1"]:
        L = workloads.LAYERS[name]
        d = workloads.make(name)
        assert int(d["mask"].sum()) == round(L.keep * L.M * L.C * L.R * L.S)


def test_late_layer_is_large_and_relu():
    L = workloads.LAYERS["late"]
    d = workloads.make("late")
    assert int(d["mask"].sum()) == round(0.01 * L.M * L.C * 9)
    assert d["x"].min() == 0.0
    frac0 = float((d["x"] == 0).mean())
    assert 0.45 < frac0 < 0.55


@pytest.mark.parametrize("name,keep", [("imb80", 0.2), ("imb90", 0.1), ("imb95", 0.05), ("imb99", 0.01)])
def test_beta_rows_mean_density(name, keep):
    d = workloads.make(name, n_override=1)
    L = d["layer"]
    crs = L.C * L.R * L.S
    rows = d["mask"].reshape(L.M, crs).sum(1)
    # 128 rows of Beta(0.5, b): mean density within a few standard errors of keep
    sd = np.sqrt(keep * (1 - keep) / (0.5 + 0.5 * (1 - keep) / keep + 1)) / np.sqrt(L.M)
    assert abs(rows.mean() / crs - keep) < 5 * sd
    assert rows.min() >= 0 and rows.max() <= crs


def test_tiny_bernoulli_near_ten_percent():
    d = workloads.make("tiny")
    assert 0.08 < d["mask"].mean() < 0.12
