"""ffa_attention (torch.autograd) on the GPU: gradients equal (bitwise) those of
a direct fwd/bwd call and match the fp64 oracle; with several masks in one
launch as well."""
import random

import pytest
import torch

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl
from oracle import ffa_oracle as orc
from tests.test_attention_gpu import check_grad, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _leaf(t):
    return t.to(DEV).requires_grad_(True)


def test_autograd_single_mask():
    rng = random.Random(5)
    Tq, Tk = 700, 600
    sl = wl.random_slices(rng, Tq, Tk, 4)
    c = wl.Call(sl, Tq, Tk, 4, 2, 128)
    T = wl.make_tensors(c, 55)
    q, k, v = (_leaf(T[n]) for n in ("q", "k", "v"))
    do = T["do"].to(DEV)
    meta = ffa.build_meta(sl, Tq, Tk, 128)
    o = ffa.ffa_attention(q, k, v, meta, 0.1)
    o.backward(do)
    o2, lse2 = ffa.fwd(q.detach(), k.detach(), v.detach(), meta, 0.1)
    g2 = ffa.bwd(q.detach(), k.detach(), v.detach(), o2, lse2, do, meta, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for a, b in zip((q.grad, k.grad, v.grad), g2):
        assert torch.equal(a, b)
    o_ref, _ = orc.forward(T["q"], T["k"], T["v"], sl, 0.1)
    check_o(o.detach(), o_ref)
    for a, r, n in zip((q.grad, k.grad, v.grad), orc.backward(T["q"], T["k"], T["v"], T["do"], sl, 0.1),
                       ("dQ", "dK", "dV")):
        check_grad(a, r, n)


def test_autograd_grouped_masks():
    Tq = Tk = 512
    tables = [wl.varlen_slices([200, 312], ffa.CAUSAL), [(0, 512, 0, 512, ffa.FULL)]]
    c = wl.Call(tables[0], Tq, Tk, 4, 2, 64)
    T = wl.make_tensors(c, 77)
    q, k, v = (_leaf(T[n]) for n in ("q", "k", "v"))
    metas = [ffa.build_meta(t, Tq, Tk, 64) for t in tables]
    o = ffa.ffa_attention(q, k, v, metas, None, [1, 2])
    o.backward(T["do"].to(DEV))
    torch.cuda.synchronize()
    for g, sl in enumerate(tables):
        hq, hk = slice(2 * g, 2 * g + 2), slice(g, g + 1)
        sub = {n: T[n][:, hq].contiguous() for n in ("q", "do")}
        sub.update({n: T[n][:, hk].contiguous() for n in ("k", "v")})
        o_ref, _ = orc.forward(sub["q"], sub["k"], sub["v"], sl)
        check_o(o.detach()[:, hq], o_ref)
        dq, dk, dv = orc.backward(sub["q"], sub["k"], sub["v"], sub["do"], sl)
        check_grad(q.grad[:, hq], dq, "dQ")
        check_grad(k.grad[:, hk], dk, "dK")
        check_grad(v.grad[:, hk], dv, "dV")
