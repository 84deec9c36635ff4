"""The weights-in-code kernels on the CPU: pack a layer on the host (SC_PACK_HOST_ONLY
generates and assembles the kernel without a device), run its generated gfx950 code in the
instruction emulator (tests/gcn_emu.py), and compare every output element with the oracle.

The emulator also checks what the hardware leaves to the code: the wait states gfx950 needs
between dependent instructions, loads retired before their registers are read, VGPRs within
the declared count, and each output element stored exactly once (junk lanes and padding
positions never stored, no position stored twice)."""
import numpy as np
import pytest

import gcn_emu
import oracle
import sparse_weight_direct_amd as sc
import workloads


def _emulate(d, stride, pad, env=None, monkeypatch=None):
    if env is not None:
        monkeypatch.setenv("SPARSECONV_BAKE", env)
    x, w, mask = d["x"], d["w"], d["mask"]
    M, C, R, S = w.shape
    N, _, H, W = x.shape
    h = sc.Handle(M, C, R, S, H, W, stride, pad, values=w, mask=mask, flags=sc.SC_PACK_HOST_ONLY)
    info = h.info()
    assert info["mapping"] == sc.MAPPING_BAKED, info
    y, written = gcn_emu.run_baked(h.kernel_source(), info, x, M, h.E, h.F)
    return y, written, info


def _check(d, stride, pad, what, env=None, monkeypatch=None):
    y, written, info = _emulate(d, stride, pad, env, monkeypatch)
    assert (written == 1).all(), f"{what}: {int((written != 1).sum())} outputs not stored exactly once"
    r = oracle.reference(d["x"], d["w"], d["mask"], stride, pad)
    ok = oracle.within_tolerance(y, r["y64"], r["mag"], 1e-5)
    assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance"
    return y, info


def test_tiny_layer():
    d = workloads.make("tiny")
    L = d["layer"]
    _check(d, L.stride, L.pad, "tiny")


CASES = [  # N, C, H, W, M, R, S, stride, pad, keep, seed
    (2, 5, 13, 11, 9, 3, 3, 1, 1, 0.3, 5),
    (2, 3, 27, 23, 7, 5, 5, 2, 2, 0.4, 6),
    (3, 4, 9, 9, 6, 1, 1, 1, 0, 0.5, 7),
    (2, 3, 40, 37, 5, 11, 11, 4, 0, 0.2, 8),
    (1, 3, 10, 12, 150, 3, 3, 1, 1, 0.2, 9),
    (1, 2, 6, 70, 9, 3, 7, 1, 3, 0.5, 10),
    (4, 2, 5, 3, 11, 2, 3, 3, 2, 0.7, 11),   # several images per wavefront, stride 3
    (1, 6, 1, 90, 5, 1, 4, 1, 1, 0.6, 12),   # one input row
    (2, 7, 17, 19, 13, 3, 3, 1, 1, 0.0, 13),  # no non-zero at all: exact +0 everywhere
    (2, 4, 15, 15, 12, 3, 3, 1, 1, 1.0, 14),  # dense filters
]


@pytest.mark.parametrize("c", CASES, ids=lambda c: "N{}C{}H{}W{}M{}R{}S{}st{}p{}k{}".format(*c[:10]))
def test_random_shapes(c):
    d = workloads.make_custom(*c)
    y, info = _check(d, c[7], c[8], str(c))
    if c[9] == 0.0:
        assert np.all(y == 0) and not np.signbit(y).any()


@pytest.mark.parametrize("env", ["G=3", "DPP=0", "G=2,DPP=0,D=3", "T=1", "D=1", "G=5,T=2,D=2", "Q=2,T=1",
                                 "Q=4,T=1", "Q=8,T=2", "G=3,Q=2,T=3,D=3", "Q=2,DPP=0,D=4", "PERM=0",
                                 "PERM=0,G=2,D=3", "PERM=1,D=2", "PERM=0,Q=2,T=1", "Q=3,T=1", "Q=5,T=2",
                                 "Q=6,T=1,D=3", "G=2,Q=3,T=2"])
def test_plan_options(env, monkeypatch):
    """Groups, lane shifts off, load depth and units per workgroup change the code but not
    the per-channel summation order: the outputs must equal the default plan's bit for bit,
    and the oracle's within tolerance.  Channel splits (Q) add partial sums of channel
    ranges in LDS: the order changes, the result stays within tolerance, and repeating the
    launch gives the same bits."""
    c = (2, 7, 27, 23, 17, 5, 5, 2, 2, 0.4, 6)
    d = workloads.make_custom(*c)
    base, _ = _check(d, c[7], c[8], "default")
    y, info = _check(d, c[7], c[8], env, env, monkeypatch)
    if "Q=" not in env:
        assert np.array_equal(y.view(np.uint32), base.view(np.uint32))
    else:
        assert info["bake_splits"] > 1 and info["bake_lds_bytes"] > 0
        y2, _, _ = _emulate(d, c[7], c[8])
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_single_nonzero_bit_exact():
    """One non-zero per output channel: the kernel's single rounding fma(w, x, +0) and the
    oracle's rounded double product are the same fp32 value; +0 where the tap lies in the
    padding."""
    rng = np.random.default_rng(3)
    N, C, M, H, W, R, S, st, pad = 2, 5, 6, 30, 41, 3, 3, 1, 1
    x = rng.uniform(-1, 1, (N, C, H, W)).astype(np.float32)
    w = np.zeros((M, C, R, S), np.float32)
    w[2, 4, R - 1, 0] = np.float32(0.8125)
    w[5, 0, 0, S - 1] = np.float32(-1.3)
    d = {"x": x, "w": w, "mask": None}
    y, written, _ = _emulate(d, st, pad)
    r = oracle.reference(x, w, None, st, pad)
    np.testing.assert_array_equal(y.view(np.uint32), r["y"].view(np.uint32))


def test_generated_code_shape():
    """Per non-zero exactly one FMA with the weight as a literal (first use of an accumulator
    as w*x + 0), every FMA's weight is one of the layer's weights, and nothing else in the
    hot loop touches memory but the row-vector loads."""
    d = workloads.make("tiny")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                  flags=sc.SC_PACK_HOST_ONLY)
    src = h.kernel_source()
    code = src.split("\t.section .rodata")[0]
    fmas = [ln for ln in code.splitlines() if "v_fmac_f32" in ln or "v_fmamk_f32" in ln]
    nnz = int(d["mask"].sum())
    assert len(fmas) == nnz
    lits = set()
    for ln in fmas:
        tok = [t.strip() for t in ln.replace("\t", " ").split(",")]
        lits.add(int(tok[1] if "fmac" in ln else tok[2], 0))
    vals = set(int(v) for v in d["w"][d["mask"].astype(bool)].view(np.uint32))
    assert lits <= vals
    ops = set(ln.split()[0] for ln in code.splitlines() if ln.startswith("\t") and not ln.startswith("\t."))
    assert {o for o in ops if o.startswith(("global_", "flat_", "scratch_"))} == set()
    assert {o for o in ops if o.startswith("buffer_")} == {"buffer_load_dword", "buffer_store_dword"}
    # lane shifts go through the LDS crossbar (ds_bpermute), which uses no LDS memory
    assert {o for o in ops if o.startswith("ds_")} == {"ds_bpermute_b32"}
    assert h.info()["bake_lds_bytes"] == 0 and ".amdhsa_group_segment_fixed_size 0" in src


SHIFT_CASES = [  # N, C, H, W, M, R, S, stride, pad, keep, seed: shifts of 1..5 lanes, 1..4 phases
    (2, 5, 13, 11, 9, 3, 3, 1, 1, 0.3, 21),
    (2, 3, 27, 23, 7, 5, 5, 2, 2, 0.4, 22),
    (1, 2, 6, 70, 9, 3, 7, 1, 3, 0.5, 23),
    (2, 3, 40, 37, 5, 11, 11, 4, 0, 0.2, 24),
    (2, 4, 19, 30, 6, 2, 6, 1, 2, 0.6, 25),
    (3, 4, 17, 23, 8, 3, 9, 3, 1, 0.5, 26),
]


@pytest.mark.parametrize("c", SHIFT_CASES, ids=lambda c: "R{}S{}st{}".format(*c[5:8]))
def test_crossbar_shifts_equal_dpp_shifts(c, monkeypatch):
    """Lane shifts through the LDS crossbar (ds_bpermute) and by DPP moves feed the same FMAs
    in the same order: the two kernels' outputs agree bit for bit, and with the oracle."""
    d = workloads.make_custom(*c)
    y1, info1 = _check(d, c[7], c[8], "crossbar", "PERM=1", monkeypatch)
    y0, info0 = _check(d, c[7], c[8], "dpp", "PERM=0", monkeypatch)
    assert np.array_equal(y1.view(np.uint32), y0.view(np.uint32))


@pytest.mark.parametrize("env", ["G=2,Q=4,T=1", "G=2,Q=3,T=2"])
def test_channel_split_reduction_in_rounds(env, monkeypatch):
    """128 accumulators per wavefront and several channel splits: the partial sums go through one
    LDS buffer of 32 channels per split, reused over 4 rounds (two barriers per round), so a unit
    needs Q * 8 KB of LDS however many channels it holds; each split adds the partial sums of its
    own blocks of 4 channels in split order and stores them, so the result equals the oracle's
    within tolerance and repeats bit for bit."""
    d = workloads.make_custom(1, 12, 5, 7, 256, 3, 3, 1, 1, 0.3, 31)
    y, info = _check(d, 1, 1, env, env, monkeypatch)
    Q, T = info["bake_splits"], info["bake_units_per_wg"]
    assert Q > 2 and info["bake_lds_bytes"] == T * Q * 8 * 1024
    y2, _, _ = _emulate(d, 1, 1)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


STAGED_CASES = [  # N, C, H, W, M, R, S, stride, pad, keep, seed
    (2, 20, 13, 16, 9, 3, 3, 1, 1, 0.3, 41),   # wide layout (16-byte DMA), 3 chunks, the last partial
    (3, 19, 9, 12, 30, 3, 3, 1, 1, 0.4, 42),   # wide, several images per workgroup
    (2, 5, 13, 11, 9, 3, 3, 1, 1, 0.3, 43),    # narrow layout (4-byte DMA), one partial chunk
    (1, 9, 6, 70, 9, 3, 7, 1, 3, 0.5, 44),     # pad 3: narrow, 7 taps per step
    (2, 11, 8, 8, 7, 5, 5, 1, 2, 0.4, 45),     # 5x5, pad 2, wide
    (2, 17, 9, 9, 6, 1, 1, 1, 0, 0.5, 46),     # 1x1
    (2, 7, 17, 19, 13, 3, 3, 1, 1, 0.0, 47),   # no non-zero at all: +0 everywhere
]
STAGED_ENVS = ["STAGE=1", "STAGE=1,T=1", "STAGE=1,T=2", "STAGE=1,G=3,T=3", "NB=3,RA=2", "NB=4,CC=3,RA=4,T=2,CB=0",
               "CB=0", "CB=1,RA=2,T=2", "SEQ=1,G=2", "SEQ=1,G=3,T=2,NB=3", "SEQ=1,G=4,CB=0", "GW=1,G=2",
               "GW=1,G=5,T=3,CC=3", "GW=1,G=4,CB=0,NB=3", "C0=1", "C0=2,CC=5,NB=3", "GW=1,G=2,C0=1,CC=4", "ES=-1,ORD=1", "ES=2,ESNT=1,CC=3,ORD=1",
               "SEQ=1,G=2,ES=1,ESNT=2,CC=4", "GW=1,G=2,ES=-1,ORD=1,CC=3", "CB=2", "CB=2,T=2,CC=5",
               "GW=1,G=2,CB=2", "SEQ=1,G=2,CB=2,CC=3", "CB=2,ES=-1,ORD=1,C0=1", "PB=1", "PB=1,NB=3,CC=5,C0=2",
               "PB=1,GW=1,G=2,RA=2", "PB=1,SEQ=1,G=2,ES=-1,ORD=1", "PB=1,CB=2", "PB=0", "PB=0,RA=2,CC=5",
               "PB=0,GW=1,G=2"]


@pytest.mark.parametrize("env", STAGED_ENVS)
@pytest.mark.parametrize("c", STAGED_CASES, ids=lambda c: "N{}C{}H{}W{}M{}R{}S{}p{}k{}".format(*c[:7], c[8], c[9]))
def test_staged_kernels(c, env, monkeypatch):
    """Staged kernels: per chunk of channels every wavefront of a workgroup copies part of the
    workgroup's input window into LDS (LDS DMA, double-buffered, a barrier per chunk) and reads
    its taps from there.  The emulator checks that no LDS word is read before the DMA that
    writes it has been waited for, and the wait state after writing m0.  The FMAs are the same
    as the default plan's in the same order, so the outputs equal its outputs bit for bit.
    Options: T wavefronts per workgroup, G groups, NB chunk buffers (the DMA runs NB - 1
    chunks ahead), CC channels per chunk, RA batches of tap reads in flight, CB=1 a channel's
    taps read as one batch (pairs by ds_read2_b32 from a per-channel base register; the
    default where the filter's reach allows; from fixed base registers, one per chunk slot and
    buffer, set in the prologue, or with PB=0 from a base made per channel), CB=2 two channels'
    taps per batch (a tap of both
    channels in one ds_read2st64_b32 from a base register per tap), CB=0 one step's taps per
    batch, SEQ=1 every
    workgroup runs all G groups in turn (the DMA pipeline continues across groups, each
    group's stores follow its last chunk), GW=1 a workgroup holds the wavefronts of all G groups
    for its T tiles, which stage one window together (every section passes every chunk, so all
    wavefronts pass the same barriers, which the emulator checks), C0 channels in the first
    chunk (later chunks double up to CC), ES the unit from the end at which the stores of
    output channels that are already final start (-1: at once; 0, the default: all stores
    after the walk), ESNT their cache policy, ORD=1 the walk's channel order that completes
    output channels early (every plan of the handle, the default plan too, takes it).  Early
    stores go out before the walk ends: the emulator checks each output is stored once, and the
    comparison with the oracle and the default plan shows it was stored after its last FMA; it
    models vector memory operations completing in issue order, which the waits rely on."""
    d = workloads.make_custom(*c)
    y, info = _check(d, c[7], c[8], env, env, monkeypatch)
    assert info["bake_stage"] == 1 and info["bake_valid_lanes"] == 64
    T = info["bake_units_per_wg"]
    assert info["bake_lds_bytes"] >= 2 * info["bake_chunk_channels"] * (64 * T) * 4
    if "ORD=1" in env:  # the default plans with the same channel order
        monkeypatch.setenv("SPARSECONV_BAKE", "ORD=1")
    else:
        monkeypatch.delenv("SPARSECONV_BAKE")
    y0, _, info0 = _emulate(d, c[7], c[8])
    assert info0["bake_stage"] == 0
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))
    if c[9] == 0.0:
        assert np.all(y == 0) and not np.signbit(y).any()


def _m0_next_to_dma(lines):
    """The kernel with each m0 write moved to just before its DMA (no wait state between)."""
    out, held = [], None
    for ln in lines:
        t = ln.strip()
        if t.startswith("s_add_u32 m0"):
            held = ln
        elif t == "s_nop 0" and held is not None:
            continue
        elif t.startswith("buffer_load") and t.endswith(" lds") and held is not None:
            out += [held, ln]
            held = None
        else:
            out.append(ln)
    return out


def _loosen_vmcnt(lines):
    """The kernel with every vmcnt wait one DMA looser."""
    out = []
    for ln in lines:
        t = ln.strip()
        if t.startswith("s_waitcnt vmcnt("):
            n = int(t[len("s_waitcnt vmcnt("):-1])
            ln = ln.replace(t, f"s_waitcnt vmcnt({n + 1})")
        out.append(ln)
    return out


@pytest.mark.parametrize("drop", ["m0 wait state", "s_waitcnt vmcnt", "vmcnt + 1", "s_barrier"])
def test_staged_synchronisation_is_checked(drop, monkeypatch):
    """The emulator rejects a staged kernel with its synchronisation taken out: with no wait
    state between the m0 write and the DMA that reads m0, without the vmcnt waits before the
    barriers or with each of them one DMA too loose (a wavefront would read words another
    wavefront's DMA has not finished writing), or without the barriers (a wavefront reads
    words nobody has staged yet, or overwrites a buffer others still read)."""
    d = workloads.make_custom(*STAGED_CASES[0])
    c = STAGED_CASES[0]
    monkeypatch.setenv("SPARSECONV_BAKE", "STAGE=1")
    x, w, mask = d["x"], d["w"], d["mask"]
    M, C, R, S = w.shape
    h = sc.Handle(M, C, R, S, x.shape[2], x.shape[3], c[7], c[8], values=w, mask=mask,
                  flags=sc.SC_PACK_HOST_ONLY)
    src = h.kernel_source()
    lines = src.split("\n")
    if drop == "m0 wait state":
        bad = "\n".join(_m0_next_to_dma(lines))
    elif drop == "vmcnt + 1":
        bad = "\n".join(_loosen_vmcnt(lines))
    else:
        bad = "\n".join(ln for ln in lines if not ln.strip().startswith(drop))
    assert bad != src
    r = oracle.reference(x, w, mask, c[7], c[8])
    try:
        y, _ = gcn_emu.run_baked(bad, h.info(), x, M, h.E, h.F)
    except gcn_emu.EmuError:
        return
    assert not oracle.within_tolerance(y, r["y64"], r["mag"], 1e-5).all()


@pytest.mark.parametrize("env", ["G=2,Q=8,T=2", "STAGE=1,T=16"])
def test_plan_that_does_not_fit_a_cu_is_refused(env, monkeypatch):
    """A workgroup runs on one CU: 16 wavefronts of 168 VGPRs (4 per SIMD) need more than the
    512 registers a SIMD's lanes have, and 16 staged tiles more LDS than the CU's 160 KB.  The
    packer refuses such a forced plan (no weights-in-code kernel; the reason is reported)
    instead of generating a kernel that cannot be dispatched."""
    monkeypatch.setenv("SPARSECONV_BAKE", env)
    d = workloads.make("late")
    L = d["layer"]
    h = sc.Handle(L.M, L.C, L.R, L.S, L.H, L.W, L.stride, L.pad, values=d["w"], mask=d["mask"],
                  flags=sc.SC_PACK_HOST_ONLY)
    assert h.info()["mapping"] != 2
    with pytest.raises(sc.SparseConvError, match="than a CU has"):
        h.kernel_source()
