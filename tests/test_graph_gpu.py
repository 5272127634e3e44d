"""A whole step (block metadata, forward, backward) captured in a HIP graph.

The library allocates nothing, never synchronises and launches every kernel
on the stream it is given, so a caller can capture a step with
torch.cuda.graph and replay it.  Each replay here starts from outputs filled
with NaN, runs with eager steps and synchronisations between replays, and
must reproduce the eager step bitwise: same kernels, same inputs, same
fixed summation orders.  The eager step itself is checked against the fp64
oracle in test_attention_gpu.  Cases: a varlen-causal GQA table at d = 128,
and a table with several slices per query row run as two calls (d = 128 and
d = 64) captured in one graph.
"""
import random

import pytest
import torch

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
OUTS = ("o", "lse", "dq", "dk", "dv")


class Step:
    def __init__(self, slices, Tq, Tk, Hq, Hkv, d, seed):
        g = torch.Generator(device=DEV).manual_seed(seed)
        self.q = torch.randn(Tq, Hq, d, generator=g, device=DEV).to(torch.bfloat16)
        self.k = torch.randn(Tk, Hkv, d, generator=g, device=DEV).to(torch.bfloat16)
        self.v = torch.randn(Tk, Hkv, d, generator=g, device=DEV).to(torch.bfloat16)
        self.do = torch.randn(Tq, Hq, d, generator=g, device=DEV).to(torch.bfloat16)
        host = torch.tensor(slices, dtype=torch.int32).reshape(-1, 5)
        self.slices = host.to(DEV)
        self.shape = (len(slices), Tq, Tk, d)
        self.meta_buf = torch.empty(ffa.meta_workspace_size(len(slices), Tq, Tk, d, host),
                                    dtype=torch.uint8, device=DEV)
        self.meta = ffa.build_meta(self.slices, Tq, Tk, d, out=self.meta_buf)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(Hq, Tq, dtype=torch.float32, device=DEV)
        self.dq, self.dk, self.dv = (torch.empty_like(self.q), torch.empty_like(self.k),
                                     torch.empty_like(self.v))
        self.ws = torch.empty(max(256, ffa.bwd_workspace_size(self.q, self.k)), dtype=torch.uint8,
                              device=DEV)

    def run(self):
        n, Tq, Tk, d = self.shape
        ffa._check(ffa.lib().ffa_build_block_meta(self.slices.data_ptr(), n, Tq, Tk, d,
                                                  self.meta_buf.data_ptr(), self.meta_buf.numel(),
                                                  ffa._stream()), "ffa_build_block_meta")
        ffa.fwd(self.q, self.k, self.v, self.meta, out=self.o, lse=self.lse)
        ffa.bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.meta, dq=self.dq, dk=self.dk,
                dv=self.dv, workspace=self.ws)


def _same(a, b):
    """Bitwise equal, NaN where the other is NaN (rows without keys give -inf
    LSE, never NaN, so any NaN left means a replay did not write it)."""
    return bool(torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                            b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)))


@pytest.mark.parametrize("which", ["varlen_causal_gqa", "several_slices_per_row"])
def test_graph_replay_matches_eager_step(which):
    rng = random.Random(11)
    if which == "varlen_causal_gqa":
        T = 2048
        lens = wl.trimmed_lengths(rng, T, 128, 1024)
        steps = [Step(wl.varlen_slices(lens, wl.CAUSAL), T, T, 8, 2, 128, 5)]
    else:
        T = 1536
        sl = wl.random_banded_slices(rng, T, T, bands=3)
        steps = [Step(sl, T, T, 4, 4, 128, 6), Step(sl, T, T, 2, 1, 64, 7)]
    for _ in range(2):
        for s in steps:
            s.run()
    torch.cuda.synchronize()
    ref = [[getattr(s, n).clone() for n in OUTS] for s in steps]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in steps:
            s.run()
    torch.cuda.synchronize()
    for replay in range(3):
        for s in steps:
            for n in OUTS:
                getattr(s, n).fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (s, r) in enumerate(zip(steps, ref)):
            for n, x in zip(OUTS, r):
                assert _same(getattr(s, n), x), f"replay {replay}, call {i}: {n} differs from the eager step"
        # eager work between replays
        for s in steps:
            s.run()
        torch.cuda.synchronize()
        for s, r in zip(steps, ref):
            for n, x in zip(OUTS, r):
                assert _same(getattr(s, n), x), f"eager step after replay {replay}: {n} differs"
