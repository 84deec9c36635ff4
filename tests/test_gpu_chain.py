"""Layer stacks (chain.LayerChain): each layer's output against the oracle applied to that
layer's actual input, and graph replays against the eager run.

A stack runs the same kernels in the same order whether launched eagerly or replayed from
a captured graph, and the kernel's summation order is fixed by the schedule, so every
replay must equal the eager output bit for bit.  Replays are interleaved with other eager
GPU work and checked one by one (a graph that recorded state-dependent nodes would drift
on later replays)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_weight_direct_amd as sc
import workloads
from gpu_util import assert_parity
from sparse_weight_direct_amd.chain import LayerChain

pytestmark = pytest.mark.gpu


def _chain(name, flags=(0,)):
    """The stack with layer i packed with flags[i % len(flags)]."""
    layers = workloads.make_chain(name)
    handles = [sc.Handle(values=d["w"], mask=d["mask"], flags=flags[i % len(flags)], **d["geom"])
               for i, d in enumerate(layers)]
    ch = LayerChain(handles, N=layers[0]["x"].shape[0])
    ch.x.copy_(torch.from_numpy(layers[0]["x"]))
    return layers, ch


@pytest.mark.parametrize("name", list(workloads.CHAINS))
def test_chain_each_layer_matches_oracle(name):
    layers, ch = _chain(name)
    ch.run()
    torch.cuda.synchronize()
    src = layers[0]["x"]
    for i, (d, out) in enumerate(zip(layers, ch.outs)):
        g = d["geom"]
        ref = oracle.reference(src, d["w"], d["mask"], g["stride"], g["pad"])
        y = out.cpu().numpy()
        assert_parity(y, ref["y64"], ref["mag"], f"{name} layer {i}")
        src = y  # the next layer's oracle input is this layer's GPU output


@pytest.mark.parametrize("repeat", [1, 3])
@pytest.mark.parametrize("name", list(workloads.CHAINS))
def test_chain_graph_replays_equal_eager(name, repeat):
    """repeat > 1: the graph runs the stack several times on the same input; the last output
    is still the eager one."""
    _, ch = _chain(name)
    eager = ch.run().clone()
    torch.cuda.synchronize()
    ch.capture(repeat=repeat)
    other = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        for o in ch.outs:
            o.fill_(float("nan"))
        _ = (other * 2.0).sum()  # unrelated eager work between replays
        ch.replay()
        torch.cuda.synchronize()
        got = ch.outs[-1]
        assert torch.equal(got, eager), f"replay {rep}: {int((got != eager).sum())} outputs differ"


def test_mixed_chain_fp16_word_and_escoin_layers():
    """A stack mixing the default handle, a packed-word handle and an Escoin-mapping handle
    (which needs the chain's workspace): each layer against the oracle of its own form, and
    graph replays equal to the eager run."""
    layers, ch = _chain("tiny4", flags=(0, sc.SC_PACK_FP16_WORD, sc.SC_PACK_ESCOIN_MAP))
    assert ch.ws is not None
    eager = ch.run().clone()
    torch.cuda.synchronize()
    src = layers[0]["x"]
    for i, (d, out) in enumerate(zip(layers, ch.outs)):
        g = d["geom"]
        ref_fn = oracle.reference_fp16 if i % 3 == 1 else oracle.reference
        ref = ref_fn(src, d["w"], d["mask"], g["stride"], g["pad"])
        y = out.cpu().numpy()
        assert_parity(y, ref["y64"], ref["mag"], f"mixed layer {i}")
        src = y
    ch.capture()
    for rep in range(3):
        for o in ch.outs:
            o.fill_(float("nan"))
        ch.replay()
        torch.cuda.synchronize()
        assert torch.equal(ch.outs[-1], eager), f"replay {rep}"
