"""Several masks in one launch (ffa_fwd_grouped / ffa_bwd_grouped) on the GPU.

Each kv-head group (with its query heads) has its own slice table.  Checks:
every output element against the fp64 oracle run per group on that group's
heads; O, LSE and dQ identical (bitwise) to one single-mask call per group on
the sliced heads; dK, dV within the test tolerance of those calls (the dK/dV
load balancing weighs all groups, so the split of long key blocks can
differ); and the 128K block-causal / sliding-window workload, whose two head
groups normally run as two calls, as one grouped call over one 16-head
tensor set, against those two calls."""
import random

import pytest
import torch

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl
from oracle import ffa_oracle as orc
from tests.test_attention_gpu import check_grad, check_lse, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _window(T, lens, w):
    out, s = [], 0
    for L in lens:
        e = s + L
        if L <= w:
            out.append((s, e, s, e, ffa.CAUSAL))
        else:
            out.append((s, s + w, s, s + w, ffa.CAUSAL))
            out.append((s + w, e, s + 1, e, ffa.BI_CAUSAL))
        s = e
    return out


def _run_grouped(T, tables, kv_end, Tq, Tk, d):
    q, k, v, do = (T[n].to(DEV) for n in ("q", "k", "v", "do"))
    metas = [ffa.build_meta(sl, Tq, Tk, d) for sl in tables]
    o, lse = ffa.fwd_grouped(q, k, v, metas, kv_end)
    dq, dk, dv = ffa.bwd_grouped(q, k, v, o, lse, do, metas, kv_end)
    torch.cuda.synchronize()
    assert all(m.status() == 0 for m in metas)
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
def test_grouped_against_oracle_and_single_calls(d):
    rng = random.Random(31 + d)
    Tq = Tk = 1500
    Hkv, G = 4, 2
    Hq = Hkv * G
    tables = [wl.varlen_slices([400, 700, 400], ffa.CAUSAL),
              _window(Tq, [900, 600], 256),
              wl.random_slices(rng, Tq, Tk, 5)]
    kv_end = [1, 3, 4]
    call = wl.Call(tables[0], Tq, Tk, Hq, Hkv, d)
    T = wl.make_tensors(call, 99 + d)
    print(f"grouped d={d}: groups {kv_end}", flush=True)
    o, lse, dq, dk, dv = _run_grouped(T, tables, kv_end, Tq, Tk, d)
    k0 = 0
    for sl, k1 in zip(tables, kv_end):
        hq = slice(k0 * G, k1 * G)
        hk = slice(k0, k1)
        sub = {n: T[n][:, hq].contiguous() for n in ("q", "do")}
        sub.update({n: T[n][:, hk].contiguous() for n in ("k", "v")})
        o_ref, l_ref = orc.forward(sub["q"], sub["k"], sub["v"], sl)
        check_o(o[:, hq], o_ref, f"O group kv[{k0},{k1})")
        check_lse(lse[hq], l_ref, f"LSE group kv[{k0},{k1})")
        g_ref = orc.backward(sub["q"], sub["k"], sub["v"], sub["do"], sl)
        check_grad(dq[:, hq], g_ref[0], "dQ")
        check_grad(dk[:, hk], g_ref[1], "dK")
        check_grad(dv[:, hk], g_ref[2], "dV")
        # one single-mask call on the group's heads
        qs, ks, vs, dos = (sub[n].to(DEV) for n in ("q", "k", "v", "do"))
        meta = ffa.build_meta(sl, Tq, Tk, d)
        o1, l1 = ffa.fwd(qs, ks, vs, meta)
        g1 = ffa.bwd(qs, ks, vs, o1, l1, dos, meta)
        torch.cuda.synchronize()
        assert torch.equal(o1, o[:, hq]) and torch.equal(l1, lse[hq])
        assert torch.equal(g1[0], dq[:, hq])
        for a, b in ((g1[1], dk[:, hk]), (g1[2], dv[:, hk])):
            rel = float((a.double() - b.double()).norm() / max(float(a.double().norm()), 1e-30))
            assert rel <= 1e-2
        k0 = k1


def test_video_workload_as_one_grouped_call():
    """The 128K block-causal + sliding-window workload (two head groups of 8)
    as one launch over a 16-head tensor set, against its two calls."""
    W = wl.workload(4)
    ca, cb = W.calls
    assert ca.Tq == cb.Tq and ca.Hkv == cb.Hkv == 8
    Ta = wl.make_tensors(ca, 100 * W.seed)
    Tb = wl.make_tensors(cb, 100 * W.seed + 1)
    T = {n: torch.cat([Ta[n], Tb[n]], dim=1) for n in ("q", "k", "v", "do")}
    o, lse, dq, dk, dv = _run_grouped(T, [ca.slices, cb.slices], [8, 16], ca.Tq, ca.Tk, ca.d)
    for g, (c, Tg) in enumerate(((ca, Ta), (cb, Tb))):
        h = slice(8 * g, 8 * g + 8)
        q, k, v, do = (Tg[n].to(DEV) for n in ("q", "k", "v", "do"))
        meta = ffa.build_meta(c.slices, c.Tq, c.Tk, c.d)
        o1, l1 = ffa.fwd(q, k, v, meta)
        g1 = ffa.bwd(q, k, v, o1, l1, do, meta)
        torch.cuda.synchronize()
        assert torch.equal(o1, o[:, h]) and torch.equal(l1, lse[h])
        assert torch.equal(g1[0], dq[:, h])
        for a, b in ((g1[1], dk[:, h]), (g1[2], dv[:, h])):
            rel = float((a.double() - b.double()).norm() / max(float(a.double().norm()), 1e-30))
            assert rel <= 1e-2


def test_grouped_with_accumulate_over_split_tables():
    """Each group's table split into two tables with disjoint valid sets, run as
    two grouped calls: the second merges into the first (forward) and adds to
    it (backward, given the whole forward's O and LSE).  Against the oracle of
    each group's whole table."""
    from tests.test_accumulate_gpu import prefix_table, split
    rng = random.Random(808)
    Tq = Tk = 900
    Hkv, G, d = 2, 2, 128
    whole = [prefix_table(rng, Tq, 4), wl.varlen_slices([300, 600], ffa.CAUSAL)]
    parts = [split(t, rng) for t in whole]
    call = wl.Call(whole[0], Tq, Tk, Hkv * G, Hkv, d)
    T = wl.make_tensors(call, 808)
    q, k, v, do = (T[n].to(DEV) for n in ("q", "k", "v", "do"))
    ends = [1, 2]
    m1 = [ffa.build_meta(p[0], Tq, Tk, d) for p in parts]
    m2 = [ffa.build_meta(p[1], Tq, Tk, d) for p in parts]
    mw = [ffa.build_meta(t, Tq, Tk, d) for t in whole]
    o, lse = ffa.fwd_grouped(q, k, v, m1, ends)
    ffa.fwd_grouped(q, k, v, m2, ends, out=o, lse=lse, accumulate=True)
    ow, lw = ffa.fwd_grouped(q, k, v, mw, ends)     # the whole forward for the backward
    dq, dk, dv = ffa.bwd_grouped(q, k, v, ow, lw, do, m1, ends)
    ffa.bwd_grouped(q, k, v, ow, lw, do, m2, ends, dq=dq, dk=dk, dv=dv, accumulate=True)
    torch.cuda.synchronize()
    for g, sl in enumerate(whole):
        hq, hk = slice(g * G, g * G + G), slice(g, g + 1)
        sub = {n: T[n][:, hq].contiguous() for n in ("q", "do")}
        sub.update({n: T[n][:, hk].contiguous() for n in ("k", "v")})
        o_ref, l_ref = orc.forward(sub["q"], sub["k"], sub["v"], sl)
        check_o(o[:, hq], o_ref, f"merged O group {g}")
        check_lse(lse[hq], l_ref, f"merged LSE group {g}")
        g_ref = orc.backward(sub["q"], sub["k"], sub["v"], sub["do"], sl)
        check_grad(dq[:, hq], g_ref[0], "dQ")
        check_grad(dk[:, hk], g_ref[1], "dK")
        check_grad(dv[:, hk], g_ref[2], "dV")


def test_grouped_phases_match_one_call():
    """PRE, DKDV and DQ as three grouped calls equal one grouped call."""
    Tq = Tk = 700
    tables = [wl.varlen_slices([200, 500], ffa.CAUSAL), [(0, 700, 0, 700, ffa.FULL)]]
    call = wl.Call(tables[0], Tq, Tk, 8, 2, 128)
    T = wl.make_tensors(call, 31)
    q, k, v, do = (T[n].to(DEV) for n in ("q", "k", "v", "do"))
    metas = [ffa.build_meta(t, Tq, Tk, 128) for t in tables]
    o, lse = ffa.fwd_grouped(q, k, v, metas, [1, 2])
    g1 = ffa.bwd_grouped(q, k, v, o, lse, do, metas, [1, 2])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ffa.bwd_workspace_size(q, k), dtype=torch.uint8, device=DEV)
    for ph in (ffa.BWD_PRE, ffa.BWD_DKDV, ffa.BWD_DQ):
        ffa.bwd_grouped(q, k, v, o, lse, do, metas, [1, 2], dq=dq, dk=dk, dv=dv, workspace=ws, phases=ph)
    torch.cuda.synchronize()
    for a, b in zip(g1, (dq, dk, dv)):
        rel = float((a.double() - b.double()).norm() / max(float(a.double().norm()), 1e-30))
        assert rel <= 1e-3
