"""GPU parity of the weights-in-code kernels (the default mapping for fp32 weights) beyond the
per-layer tests in test_gpu_parity.py: forced plan options, the choice between a handle's
kernels by batch size, channel splits on random shapes, and graph replay.

Bar: |gpu - oracle| <= 1e-5 * sum|w*x| per output element, exact +0 where no term
contributes.  Plans that differ only in groups, load depth, lane shifts or units per
workgroup keep every output's summation order (channels, then filter rows and columns, in
order), so their outputs must agree bit for bit; channel splits add partial sums of channel
ranges in a fixed order, so repeated launches must agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import sparse_weight_direct_amd as sc
import workloads
from gpu_util import assert_layer_parity, assert_parity, gpu_sparse

pytestmark = pytest.mark.gpu

LAYER = (3, 20, 23, 37, 50, 3, 3, 1, 1, 0.15, 77)  # N, C, H, W, M, R, S, stride, pad, keep, seed


def _layer():
    d = workloads.make_custom(*LAYER)
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, 1)
    return d, r


@pytest.mark.parametrize("env", ["G=1,Q=1,T=4", "G=2,Q=1,T=4", "G=5,Q=1,T=1", "G=1,Q=1,T=4,D=1",
                                 "G=1,Q=1,T=4,DPP=0", "G=3,Q=1,T=2,D=7,DPP=0", "G=50,Q=1,T=4"])
def test_plans_keep_the_summation_order(env, monkeypatch):
    d, r = _layer()
    monkeypatch.setenv("SPARSECONV_BAKE", "G=1,Q=1,T=4")
    base, _ = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1)
    monkeypatch.setenv("SPARSECONV_BAKE", env)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1)
    assert h.info()["mapping"] == sc.MAPPING_BAKED and h.info()["bake_variants"] == 1
    assert_parity(y, r["y64"], r["mag"], env)
    np.testing.assert_array_equal(y.view(np.uint32), base.view(np.uint32))


@pytest.mark.parametrize("env", ["G=1,Q=2,T=1", "G=1,Q=2,T=4", "G=1,Q=4,T=1", "G=2,Q=8,T=2", "G=4,Q=2,T=3,D=2",
                                 "G=1,Q=2,T=1,DPP=0"])
def test_channel_splits(env, monkeypatch):
    d, r = _layer()
    monkeypatch.setenv("SPARSECONV_BAKE", env)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1)
    info = h.info()
    assert info["bake_splits"] > 1 and info["bake_lds_bytes"] > 0
    assert_parity(y, r["y64"], r["mag"], env)
    y2, _ = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1, handle=h)
    np.testing.assert_array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_batch_size_picks_among_the_handles_kernels():
    """One handle, several batch sizes: the forward launches the kernel its estimate picks
    for N (the staged kernel once it gives every SIMD a wavefront), and every launch matches
    the oracle."""
    d = workloads.make("imb95")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"])
    assert h.info()["bake_variants"] >= 2
    big = h.launch_info(L.N)
    assert big["mapping"] == sc.MAPPING_BAKED and big["stage"] == 1
    assert big["waves"] >= 4 * torch.cuda.get_device_properties(0).multi_processor_count
    seen = set()
    for n in (1, 2, 5, 8):
        li = h.launch_info(n)
        seen.add(li["variant"])
        x = d["x"][:n]
        r = oracle.reference(x, d["w"], d["mask"], L.stride, L.pad)
        y, _ = gpu_sparse(x, d["w"], d["mask"], L.stride, L.pad, handle=h)
        assert_parity(y, r["y64"], r["mag"], f"imb95 N={n} variant {li['variant']}")
    assert seen, "no launch"


def test_many_output_channels_several_groups():
    """M = 300 output channels do not fit one wavefront's registers: the base plan has
    several groups, each a code section of its own, selected by a long jump."""
    d = workloads.make_custom(2, 24, 19, 21, 300, 3, 3, 1, 1, 0.08, 93)
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, 1)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1)
    assert h.info()["bake_groups"] >= 2
    assert_parity(y, r["y64"], r["mag"], "M=300")


def _cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        R = int(rng.choice([1, 2, 3, 3, 5, 7]))
        S = int(rng.choice([1, 2, 3, 3, 5, 7]))
        st, pad = int(rng.integers(1, 4)), int(rng.integers(0, 3))
        H = int(rng.integers(max(1, R - 2 * pad), 30))
        W = int(rng.integers(max(1, S - 2 * pad), 30))
        N, C, M = int(rng.integers(1, 5)), int(rng.choice([1, 5, 17, 60])), int(rng.choice([1, 9, 40, 130]))
        keep = float(rng.choice([0.0, 0.03, 0.2, 1.0]))
        E, F = (H + 2 * pad - R) // st + 1, (W + 2 * pad - S) // st + 1
        if C * M * R * S > 200_000 or (keep * C * M * R * S + C * R * S) * N * E * F > 2e7:
            continue
        out.append((N, C, H, W, M, R, S, st, pad, keep, seed * 1000 + len(out)))
    return out


@pytest.mark.parametrize("env", ["G=1,Q=2,T=2", "Q=4,T=1"])
def test_random_shapes_with_channel_splits(env, monkeypatch):
    """60 seeded shapes (filters to 7x7, stride to 3, pad to 2, dense and empty filters)
    through forced channel splits, failures listed together."""
    monkeypatch.setenv("SPARSECONV_BAKE", env)
    failures = []
    for c in _cases(60, 5150):
        d = workloads.make_custom(*c)
        y, h = gpu_sparse(d["x"], d["w"], d["mask"], c[7], c[8])
        r = oracle.reference(d["x"], d["w"], d["mask"], c[7], c[8])
        ok = oracle.within_tolerance(y, r["y64"], r["mag"], 1e-5)
        if not ok.all():
            failures.append((c, int((~ok).sum())))
    assert not failures, failures[:5]


def test_graph_replay_equals_eager():
    """The forward allocates nothing and records one kernel launch, so it can be captured in
    a HIP graph; replays (with other work between them) equal the eager result bit for bit."""
    d = workloads.make("mid")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"])
    x = torch.from_numpy(d["x"]).cuda()
    y = torch.empty((L.N, L.M, L.E, L.F), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        h.forward(x, y, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = y.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.forward(x, y)
    for _ in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), eager.view(np.uint32))
        torch.ones(1000, device="cuda").sum()  # other work between replays


@pytest.mark.parametrize("name,flags", [("late", 0), ("mid", 0), ("mid", sc.SC_PACK_LDS_TILE)])
def test_tune_pins_the_fastest_kernel(name, flags):
    """sparseconv_tune times the handle's kernels for the batch, pins the fastest for that N
    (launch_info reports it), leaves its result in the output, and later forwards use it; every
    result matches the oracle."""
    d = workloads.make(name)
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"], flags=flags)
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    x = torch.from_numpy(d["x"]).cuda()
    y = torch.full((L.N, L.M, L.E, L.F), float("nan"), device="cuda")
    chosen = h.tune(x, y, reps=3)
    torch.cuda.synchronize()
    assert chosen >= 0 and h.launch_info(L.N)["variant"] == chosen
    assert_parity(y.cpu().numpy(), r["y64"], r["mag"], f"{name} tuned output")
    y2, _ = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad, handle=h)
    assert_parity(y2, r["y64"], r["mag"], f"{name} forward after tuning")
    if L.N > 1:  # another batch size keeps the estimate's choice
        assert h.launch_info(1)["variant"] == sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"],
                                                        mask=d["mask"], flags=flags).launch_info(1)["variant"]


def test_tune_on_an_escoin_handle_chooses_its_only_kernel():
    d = workloads.make("tiny")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                  flags=sc.SC_PACK_ESCOIN_MAP)
    x = torch.from_numpy(d["x"]).cuda()
    assert h.tune(x) == 0


WIDE_LAYER = (3, 21, 23, 36, 50, 3, 3, 1, 1, 0.15, 78)  # W % 4 == 0: 16-byte DMA


@pytest.mark.parametrize("layer", [LAYER, WIDE_LAYER], ids=["narrow", "wide"])
@pytest.mark.parametrize("env", ["STAGE=1", "STAGE=1,T=1", "STAGE=1,T=2", "STAGE=1,G=3,T=3", "STAGE=1,G=50,T=4",
                                 "NB=3,RA=2", "NB=4,CC=3,RA=4,T=2,CB=0", "CB=0", "CB=1,RA=2,T=2", "SEQ=1,G=2",
                                 "SEQ=1,G=3,T=2,NB=3", "SEQ=1,G=4,CB=0", "GW=1,G=2", "GW=1,G=5,T=3,CC=3",
                                 "GW=1,G=4,CB=0,NB=3"])
def test_staged_plans(layer, env, monkeypatch):
    """Staged kernels (input windows copied into LDS by LDS DMA per chunk of channels, taps read
    from LDS): the same FMAs in the same order as the default plan, so the outputs agree with it
    bit for bit, and with the oracle."""
    d = workloads.make_custom(*layer)
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, 1)
    monkeypatch.setenv("SPARSECONV_BAKE", "G=1,Q=1,T=4")
    base, _ = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1)
    monkeypatch.setenv("SPARSECONV_BAKE", env)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1)
    info = h.info()
    assert info["bake_stage"] == 1 and info["bake_lds_bytes"] > 0
    assert_parity(y, r["y64"], r["mag"], env)
    np.testing.assert_array_equal(y.view(np.uint32), base.view(np.uint32))


@pytest.mark.parametrize("layer", [LAYER, WIDE_LAYER], ids=["narrow", "wide"])
@pytest.mark.parametrize("env", ["C0=1", "C0=2,CC=5,NB=3", "ES=-1,ORD=1", "ES=2,ESNT=1,CC=3,ORD=1",
                                 "ES=-1,ORD=1,ESNT=2,CC=4", "GW=1,G=2,ES=-1,ORD=1,CC=3", "SEQ=1,G=2,ES=1,CC=4",
                                 "CB=2", "GW=1,G=2,CB=2", "CB=2,ES=-1,ORD=1,C0=1", "PB=1", "PB=1,GW=1,G=2,NB=3"])
def test_staged_options(layer, env, monkeypatch):
    """Staged-kernel options: a smaller first chunk (C0), the walk's channel order that completes
    output channels early (ORD=1, which every plan of the handle takes) with stores issued during
    the walk (ES, with a cache policy ESNT; the chunk waits then count those stores, relying on
    vector memory operations completing in issue order), and channel-pair tap batches (CB=2).
    The same FMAs in the same order as the default plan of the same channel order: bit for bit
    equal to it, and within tolerance of the oracle."""
    d = workloads.make_custom(*layer)
    r = oracle.reference(d["x"], d["w"], d["mask"], 1, 1)
    monkeypatch.setenv("SPARSECONV_BAKE", "G=1,Q=1,T=4" + (",ORD=1" if "ORD=1" in env else ""))
    base, _ = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1)
    monkeypatch.setenv("SPARSECONV_BAKE", env)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], 1, 1)
    assert h.info()["bake_stage"] == 1
    assert_parity(y, r["y64"], r["mag"], env)
    np.testing.assert_array_equal(y.view(np.uint32), base.view(np.uint32))


@pytest.mark.parametrize("env", ["STAGE=1,ES=-1,ORD=1", "STAGE=1,ES=1,ESNT=1", "STAGE=1,CB=2,C0=4",
                                 "GW=1,G=2,ES=-1,ORD=1", "STAGE=1,PB=1"])
def test_staged_options_full_size(env, monkeypatch):
    """Early stores (their waits count the stores in flight), pair batches and a small first
    chunk on the full-size 112x112 layer at 95% sparsity: every output against the oracle."""
    d = workloads.make("imb95")
    L = d["layer"]
    monkeypatch.setenv("SPARSECONV_BAKE", env)
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad)
    assert h.info()["bake_stage"] == 1 and h.launch_info(L.N)["mapping"] == sc.MAPPING_BAKED
    assert_layer_parity("imb95", y, f"imb95 {env}")


@pytest.mark.parametrize("name", ["imb95", "imb99", "late", "pw1x1"])
def test_staged_full_size(name, monkeypatch):
    """A staged kernel on the full-size layers, every output against the oracle."""
    d = workloads.make(name)
    L = d["layer"]
    monkeypatch.setenv("SPARSECONV_BAKE", "STAGE=1")
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad)
    assert h.info()["bake_stage"] == 1 and h.launch_info(L.N)["mapping"] == sc.MAPPING_BAKED
    assert_layer_parity(name, y, f"{name} staged")


@pytest.mark.parametrize("n", [1, 3, 7])
def test_staged_kernel_smaller_batches(n, monkeypatch):
    """One staged handle of the 112x112 layer at 95% sparsity launched on batches of 1, 3 and 7
    images (52, 155 and 362 workgroups, the last one partly past the batch's positions; the grid
    rounded up to a multiple of the 8 XCDs): every output against the oracle."""
    d = workloads.make("imb95", n_override=n)
    L = d["layer"]
    monkeypatch.setenv("SPARSECONV_BAKE", "STAGE=1")
    y, h = gpu_sparse(d["x"], d["w"], d["mask"], L.stride, L.pad)
    assert h.launch_info(n)["stage"] == 1
    r = oracle.reference(d["x"], d["w"], d["mask"], L.stride, L.pad)
    assert_parity(y, r["y64"], r["mag"], f"imb95 staged N={n}")


def test_staged_kernel_input_not_16_byte_aligned():
    """The staged kernel copies 16 bytes a lane and needs a 16-byte aligned input; an input 4 bytes
    off falls back to the first kernel that reads rows directly, with the same result."""
    d = workloads.make("imb99")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"])
    assert h.launch_info(L.N)["stage"] == 1
    x = torch.from_numpy(d["x"]).cuda()
    xa = torch.empty(x.numel() + 4, device="cuda")[1:1 + x.numel()].view(x.shape)
    xa.copy_(x)
    assert xa.data_ptr() % 16 == 4
    ya = torch.full((L.N, L.M, L.E, L.F), float("nan"), device="cuda")
    y = torch.full_like(ya, float("nan"))
    h.forward(x, y)
    h.forward(xa, ya)
    torch.cuda.synchronize()
    assert_layer_parity("imb99", ya.cpu().numpy(), "imb99 unaligned input")
    assert_layer_parity("imb99", y.cpu().numpy(), "imb99 aligned input")
