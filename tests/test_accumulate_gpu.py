"""Partial-result accumulation (ffa_fwd_ex / ffa_bwd_ex with FFA_ACCUMULATE)
against the fp64 oracle of the whole slice table.

An attention whose slice table is split into two tables with disjoint valid
sets is computed in two calls: the forward merges the second call into the
first call's (O, LSE) with the log-sum-exp identity, the backward (given the
whole forward's O and LSE) adds the second call's dQ, dK, dV to the first
call's.  Both must equal the oracle's forward and backward over the whole
table, within the tolerances of test_attention_gpu (the merge adds one bf16
rounding of the first call's O).  The tables are built so that most rows get
keys from both parts, some from one part only, and some from none.
"""
import random

import pytest
import torch

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl
from oracle import ffa_oracle as orc
from tests.test_attention_gpu import check_grad, check_lse, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda"


def prefix_table(rng, T, nseq):
    """Sequences [s, e) with a FULL prefix [s, e) x [s, p) and a CAUSAL rest
    [p, e) x [p, e): rows past each prefix get keys from two slices."""
    cuts = sorted(rng.sample(range(64, T - 64), nseq - 1))
    bounds = [0] + cuts + [T]
    sl = []
    for s, e in zip(bounds[:-1], bounds[1:]):
        if e - s < 8:
            continue
        p = s + max(1, (e - s) // rng.choice([2, 3, 4]))
        sl.append((s, e, s, p, wl.FULL))
        sl.append((p, e, p, e, wl.CAUSAL))
    return sl


def split(sl, rng):
    a, b = [], []
    for x in sl:
        (a if rng.random() < 0.5 else b).append(x)
    if not a:
        a.append(b.pop())
    if not b:
        b.append(a.pop())
    return a, b


def cases():
    out = []
    for seed in range(3):
        rng = random.Random(500 + seed)
        T = rng.randint(400, 1100)
        d = 64 if seed == 1 else 128
        Hkv = rng.choice([1, 2])
        Hq = Hkv * rng.choice([1, 4])
        sl = prefix_table(rng, T, rng.randint(2, 4))
        # cut one FULL slice along its keys into two FULL slices (the context-parallel split)
        # (its two halves go to different calls, so those rows always need the merge)
        i = next(j for j, x in enumerate(sl) if x[4] == wl.FULL and x[3] - x[2] >= 2)
        q0, q1, k0, k1, _ = sl.pop(i)
        km = (k0 + k1) // 2
        a, b = split(sl, rng)
        a.append((q0, q1, k0, km, wl.FULL))
        b.append((q0, q1, km, k1, wl.FULL))
        out.append((seed, wl.Call(sorted(a + b), T, T, Hq, Hkv, d), (a, b)))
    return out


@pytest.mark.parametrize("case", cases(), ids=lambda c: f"seed{c[0]}")
def test_fwd_then_accumulate_equals_whole(case):
    seed, call, (sa, sb) = case
    print(f"accumulate fwd seed={seed} T={call.Tq} Hq={call.Hq} Hkv={call.Hkv} d={call.d} "
          f"A={sa} B={sb}", flush=True)
    T = wl.make_tensors(call, 700 + seed)
    q, k, v = (T[n].to(DEV) for n in ("q", "k", "v"))
    ma = ffa.build_meta(sa, call.Tq, call.Tk, call.d)
    mb = ffa.build_meta(sb, call.Tq, call.Tk, call.d)
    o, lse = ffa.fwd(q, k, v, ma)
    ffa.fwd(q, k, v, mb, out=o, lse=lse, accumulate=True)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.forward(T["q"], T["k"], T["v"], call.slices)
    check_o(o, o_ref)
    check_lse(lse, l_ref)


@pytest.mark.parametrize("case", cases(), ids=lambda c: f"seed{c[0]}")
def test_bwd_accumulate_equals_whole(case):
    seed, call, (sa, sb) = case
    print(f"accumulate bwd seed={seed} T={call.Tq} Hq={call.Hq} Hkv={call.Hkv} d={call.d}", flush=True)
    T = wl.make_tensors(call, 800 + seed)
    q, k, v, do = (T[n].to(DEV) for n in ("q", "k", "v", "do"))
    whole = ffa.build_meta(call.slices, call.Tq, call.Tk, call.d)
    o, lse = ffa.fwd(q, k, v, whole)
    ma = ffa.build_meta(sa, call.Tq, call.Tk, call.d)
    mb = ffa.build_meta(sb, call.Tq, call.Tk, call.d)
    dq, dk, dv = ffa.bwd(q, k, v, o, lse, do, ma)
    ffa.bwd(q, k, v, o, lse, do, mb, dq=dq, dk=dk, dv=dv, accumulate=True)
    torch.cuda.synchronize()
    rdq, rdk, rdv = orc.backward(T["q"], T["k"], T["v"], T["do"], call.slices)
    check_grad(dq, rdq, "dQ")
    check_grad(dk, rdk, "dK")
    check_grad(dv, rdv, "dV")


def test_accumulate_with_empty_second_part_keeps_results():
    """A second call whose table touches no row leaves O, LSE, dQ, dK, dV unchanged (bitwise)."""
    call = wl.Call([(0, 300, 0, 300, wl.CAUSAL)], 300, 300, 2, 1, 64)
    T = wl.make_tensors(call, 901)
    q, k, v, do = (T[n].to(DEV) for n in ("q", "k", "v", "do"))
    m = ffa.build_meta(call.slices, 300, 300, 64)
    empty = ffa.build_meta([], 300, 300, 64)
    o, lse = ffa.fwd(q, k, v, m)
    o0, l0 = o.clone(), lse.clone()
    ffa.fwd(q, k, v, empty, out=o, lse=lse, accumulate=True)
    dq, dk, dv = ffa.bwd(q, k, v, o, lse, do, m)
    g0 = [t.clone() for t in (dq, dk, dv)]
    ffa.bwd(q, k, v, o, lse, do, empty, dq=dq, dk=dk, dv=dv, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)
    for a, b in zip((dq, dk, dv), g0):
        assert torch.equal(a, b)
