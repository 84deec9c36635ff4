"""A stack of sparse direct convolutions run back to back, eagerly or as one HIP graph.

Small layers (a few MB of traffic) are bound by kernel-launch latency rather than by the
kernel, so a stack of them is replayed from a captured graph: one launch of the graph for
the whole stack instead of one host launch per layer.  Layer i+1 reads layer i's output.
The forward passes themselves are the library's (sparseconv_forward through Handle); this
module only allocates the intermediate buffers and drives torch's graph capture, whose
stream the forward launches go to.  sparseconv_forward allocates nothing and records no
memset, so it can be captured.  Handles that need a workspace (the Escoin mapping) share
one, allocated here once for the largest of them; the layers run one after another on
one stream, so the shared workspace is never used by two at once.
"""
from __future__ import annotations

import torch

from . import Handle


class LayerChain:
    def __init__(self, handles: list[Handle], N: int, device="cuda"):
        self.handles = handles
        self.N = N
        for a, b in zip(handles, handles[1:]):
            ga, gb = a.geom, b.geom
            if (gb["C"], gb["H"], gb["W"]) != (ga["M"], a.E, a.F):
                raise ValueError("layer shapes do not chain")
        g0 = handles[0].geom
        self.x = torch.empty((N, g0["C"], g0["H"], g0["W"]), dtype=torch.float32, device=device)
        self.outs = [torch.empty((N, h.geom["M"], h.E, h.F), dtype=torch.float32, device=device) for h in handles]
        ws = max(h.workspace_size(N) for h in handles)
        self.ws = torch.empty((ws + 3) // 4, dtype=torch.float32, device=device) if ws else None
        self.graph = None

    def run(self, stream=None):
        """All layers on the current (or given) stream, from self.x into self.outs."""
        src = self.x
        for h, out in zip(self.handles, self.outs):
            h.forward(src, out, stream=stream, workspace=self.ws if h.workspace_size(self.N) else None)
            src = out
        return self.outs[-1]

    def capture(self, repeat: int = 1):
        """Capture run() into a graph (on a side stream, as torch requires).  With repeat > 1
        the graph runs the stack that many times in a row (the same input each time): one
        graph launch per `repeat` stacks, for measuring the stack's time on the GPU apart from
        the host's cost of launching the graph."""
        if repeat < 1:
            raise ValueError("repeat must be >= 1")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run()  # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for _ in range(repeat):
                self.run()
        return self.graph

    def replay(self):
        if self.graph is None:
            raise RuntimeError("capture() first")
        self.graph.replay()
        return self.outs[-1]
