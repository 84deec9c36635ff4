"""Seeded synthetic layer inputs for sparse direct convolution.

This module only draws random numbers: dense NCHW activations, a dense M x C x R x S
weight tensor and a u8 keep-mask over it.  It computes nothing of the convolution and
nothing of the weight packing, so that both the CPU oracle and the GPU path can be fed
from it without sharing any of the method's arithmetic.

The layer shapes are the synthetic stand-ins for pruned CNN layers (an early 3x3 stage,
a batched late 3x3 stage, a 112x112 stage with per-channel density skew, an 11x11/stride-4
first layer and a 1x1 bottleneck).  No dataset is involved: the pages themselves draw
their weights at random (Tuteja et al., "Theoretical and Empirical Analysis of Sparse
Convolution", Sec. 6 and the artifact appendix).

Sampling recipe (numpy ``Generator(PCG64(seed))``, float64 draws rounded once to fp32):
  1. activations X, 2. weight values, 3. keep-mask.
Mask kinds:
  * ``bernoulli`` -- each position kept independently with probability ``keep``;
  * ``exact``     -- exactly ``round(keep * M*C*R*S)`` positions, uniform without replacement
                     over the whole M x CRS matrix;
  * ``beta_rows`` -- each output channel's density p_m ~ Beta(0.5, b) with
                     b = 0.5 * (1 - keep) / keep (so E[p_m] = keep); the row keeps
                     round(p_m * CRS) positions, uniform without replacement within the row.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Layer", "LAYERS", "BENCH_LAYER", "CHAINS", "make", "make_custom", "make_chain", "layer_seed"]


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    N: int
    C: int
    H: int
    W: int
    M: int
    R: int
    S: int
    stride: int
    pad: int
    keep: float          # mean fraction of weights kept (1 - sparsity)
    x_dist: str          # "u11" | "relu_n01"
    w_dist: str          # "u11" | "n0.05" | "n0.02"
    mask_kind: str       # "bernoulli" | "exact" | "beta_rows"
    seed: int

    @property
    def E(self) -> int:
        return (self.H + 2 * self.pad - self.R) // self.stride + 1

    @property
    def F(self) -> int:
        return (self.W + 2 * self.pad - self.S) // self.stride + 1

    @property
    def sparsity(self) -> float:
        return 1.0 - self.keep


def layer_seed(k: int, j: int = 0) -> int:
    """Seed for layer family k, sweep point j."""
    return 1000 * k + j


def _L(name, k, j, N, C, H, W, M, R, S, stride, pad, keep, x, w, mask):
    return Layer(name, N, C, H, W, M, R, S, stride, pad, keep, x, w, mask, layer_seed(k, j))


LAYERS: dict[str, Layer] = {
    # 16x16 early layer, i.i.d. 10% keep
    "tiny": _L("tiny", 1, 0, 1, 16, 16, 16, 32, 3, 3, 1, 1, 0.10, "u11", "u11", "bernoulli"),
    # 56x56 mid-stage 3x3, exactly 5% kept, weights N(0, 0.05)
    "mid": _L("mid", 2, 0, 1, 64, 56, 56, 64, 3, 3, 1, 1, 0.05, "u11", "n0.05", "exact"),
    # 14x14 late stage, batch 32, ReLU'd activations, exactly 1% kept
    "late": _L("late", 3, 0, 32, 256, 14, 14, 256, 3, 3, 1, 1, 0.01, "relu_n01", "n0.02", "exact"),
    # 112x112 stage, batch 8, per-channel density ~ Beta(0.5, b): mean sparsity 80/90/95/99%
    "imb80": _L("imb80", 4, 0, 8, 128, 112, 112, 128, 3, 3, 1, 1, 0.20, "u11", "u11", "beta_rows"),
    "imb90": _L("imb90", 4, 1, 8, 128, 112, 112, 128, 3, 3, 1, 1, 0.10, "u11", "u11", "beta_rows"),
    "imb95": _L("imb95", 4, 2, 8, 128, 112, 112, 128, 3, 3, 1, 1, 0.05, "u11", "u11", "beta_rows"),
    "imb99": _L("imb99", 4, 3, 8, 128, 112, 112, 128, 3, 3, 1, 1, 0.01, "u11", "u11", "beta_rows"),
    # 227x227 first layer, 11x11 stride 4, exactly 10% kept
    "first11": _L("first11", 5, 0, 16, 3, 227, 227, 96, 11, 11, 4, 0, 0.10, "u11", "u11", "exact"),
    # 7x7 1x1 bottleneck, batch 64, exactly 2% kept
    "pw1x1": _L("pw1x1", 5, 1, 64, 512, 7, 7, 512, 1, 1, 1, 0, 0.02, "u11", "u11", "exact"),
}

# the layer the throughput benchmark runs (112x112, batch 8, mean sparsity 95%)
BENCH_LAYER = "imb95"


def _draw(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "u11":
        v = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "relu_n01":
        v = np.maximum(rng.normal(0.0, 1.0, size=shape), 0.0)
    elif dist.startswith("n"):
        v = rng.normal(0.0, float(dist[1:]), size=shape)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return v.astype(np.float32)


def _mask(rng: np.random.Generator, kind: str, keep: float, M: int, crs: int) -> np.ndarray:
    if kind == "bernoulli":
        return (rng.random((M, crs)) < keep).astype(np.uint8)
    mask = np.zeros((M, crs), dtype=np.uint8)
    if kind == "exact":
        k = int(round(keep * M * crs))
        pos = rng.choice(M * crs, size=k, replace=False)
        mask.reshape(-1)[pos] = 1
        return mask
    if kind == "beta_rows":
        b = 0.5 * (1.0 - keep) / keep
        dens = rng.beta(0.5, b, size=M)
        for m in range(M):
            k = int(round(dens[m] * crs))
            if k:
                mask[m, rng.choice(crs, size=k, replace=False)] = 1
        return mask
    raise ValueError(f"unknown mask kind {kind!r}")


def make_custom(N, C, H, W, M, R, S, stride, pad, keep, seed, x_dist="u11", w_dist="u11",
                mask_kind="bernoulli", n_override=None):
    """Draw (x, w, mask) for an arbitrary layer shape.

    Returns a dict with ``x`` (N,C,H,W fp32), ``w`` (M,C,R,S fp32, every position drawn),
    ``mask`` (M,C,R,S u8) and ``w_masked`` (w with the dropped positions set to +0.0).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n = N if n_override is None else n_override
    x = _draw(rng, x_dist, (n, C, H, W))
    w = _draw(rng, w_dist, (M, C, R, S))
    mask = _mask(rng, mask_kind, keep, M, C * R * S).reshape(M, C, R, S)
    w_masked = np.where(mask != 0, w, np.float32(0.0)).astype(np.float32)
    return {"x": x, "w": w, "mask": mask, "w_masked": w_masked}


def make(name: str, n_override: int | None = None):
    """Draw the inputs of a named layer (see ``LAYERS``); ``n_override`` shrinks the batch
    (the first images are identical to the full draw's only when n_override == N)."""
    L = LAYERS[name]
    d = make_custom(L.N, L.C, L.H, L.W, L.M, L.R, L.S, L.stride, L.pad, L.keep, L.seed,
                    L.x_dist, L.w_dist, L.mask_kind, n_override)
    d["layer"] = L
    return d


# Layer stacks for the chaining measurement: the same shape repeated, each layer with its own
# weights (layer family 9 + the stack's index in CHAINS, sweep point = position in the
# stack); layer i+1 takes layer i's output, so C = M and the 3x3, stride-1, pad-1 layers
# keep H x W.
CHAINS = {
    "tiny4": dict(depth=4, N=1, C=16, H=16, W=16, R=3, S=3, stride=1, pad=1, keep=0.10,
                  w_dist="u11", mask_kind="bernoulli"),
    "mid4": dict(depth=4, N=1, C=64, H=56, W=56, R=3, S=3, stride=1, pad=1, keep=0.05,
                 w_dist="n0.05", mask_kind="exact"),
}


def make_chain(name: str):
    """Draw a layer stack: the first layer's activations and every layer's (w, mask).
    Returns a list of per-layer dicts (as make_custom, with ``geom``); only the first holds
    a meaningful ``x``."""
    c = CHAINS[name]
    out = []
    for j in range(c["depth"]):
        d = make_custom(c["N"], c["C"], c["H"], c["W"], c["C"], c["R"], c["S"], c["stride"], c["pad"],
                        c["keep"], layer_seed(9 + list(CHAINS).index(name), j), "u11", c["w_dist"],
                        c["mask_kind"], n_override=c["N"] if j == 0 else 1)
        d["geom"] = dict(M=c["C"], C=c["C"], R=c["R"], S=c["S"], H=c["H"], W=c["W"],
                         stride=c["stride"], pad=c["pad"])
        out.append(d)
    return out
