"""FFA forward / backward on the GPU against the fp64 oracle.

Tolerances (bf16 inputs, fp32 accumulation): O elementwise |d| <= 1e-2 + 1e-2|ref|;
LSE |d| <= 1e-3 with -inf matching -inf; dQ, dK, dV relative Frobenius error
<= 2e-2 over the checked rows (a zero reference: norm <= 2^-16 sqrt(n)), and
the same 2e-2 for every group of 32 consecutive checked rows of each head (the
rows one wave of the kernels owns), a group being measured against at least a
tenth of the norm an average group has (so that groups whose reference nearly
vanishes, where D = dO . O formed from the bf16 O dominates, are not judged by
their own rounding noise).

* small and medium cases (several tiles, ragged tails, every mask type, GQA,
  both head dims): every output element against the oracle;
* the 16K varlen-causal GQA workload: every element of O, LSE, dQ, dK, dV;
* the 64K dense, 128K block-causal / sliding-window and 256K x 1M workloads at
  full size, in the configuration the benchmark times: random inputs checked
  on 4096 sampled query rows (O, LSE, dQ computed row by row by the oracle)
  and on 4096 sampled key rows of one or two kv heads with all their query
  heads (dK, dV), and structured inputs (equal keys, rank-1 values) whose exact
  O and LSE for every row and dK, dV for 4096 sampled keys follow from
  interval sums (tests/_props.py, pinned against the oracle in
  tests/test_props.py).
"""
import math
import random

import numpy as np
import pytest
import torch

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl
from oracle import ffa_oracle as orc
from tests import _props

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------- checks ----

def check_o(got, ref, what="O"):
    g = got.double().cpu().numpy()
    err = np.abs(g - ref)
    bad = err > 1e-2 + 1e-2 * np.abs(ref)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} out of tolerance, max err {err.max():.3g}"


def check_lse(got, ref, what="LSE"):
    g = got.double().cpu().numpy()
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(g[fin]))
    if fin.any():
        err = np.abs(g[fin] - ref[fin]).max()
        assert err <= 1e-3, f"{what}: max err {err:.3g}"


GROUP = 32          # rows of one wave's output tile


def check_grad(got, ref, what, group=GROUP):
    g = got.double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    nr = np.linalg.norm(ref)
    ne = np.linalg.norm(g - ref)
    if nr == 0:
        # a zero reference, e.g. a row whose single key makes dS = P (dP - D)
        # vanish: the kernel forms P and D in fp32 from the bf16 O and the fp32
        # LSE, so it returns rounding noise; bound it at fp32 level
        assert ne <= 2.0 ** -16 * math.sqrt(g.size), f"{what}: expected zero, got norm {ne:.3g}"
        return
    rel = ne / nr
    assert rel <= 2e-2, f"{what}: relative Frobenius error {rel:.3g}"
    if g.ndim != 3 or g.shape[0] == 0:
        return
    # per group of `group` consecutive rows of each head
    n, H, d = g.shape
    pad = (-n) % group
    e2 = np.pad((g - ref) ** 2, ((0, pad), (0, 0), (0, 0))).reshape(-1, group, H, d).sum(axis=(1, 3))
    r2 = np.pad(ref ** 2, ((0, pad), (0, 0), (0, 0))).reshape(-1, group, H, d).sum(axis=(1, 3))
    typical = nr * math.sqrt(group / (n * H))
    en, rn = np.sqrt(e2), np.sqrt(r2)
    zero = rn == 0
    if zero.any():
        worst0 = en[zero].max()
        assert worst0 <= 2.0 ** -16 * math.sqrt(group * d), f"{what}: zero group with error norm {worst0:.3g}"
    grel = np.where(zero, 0.0, en / np.maximum(rn, 0.1 * typical))
    gi, hi = np.unravel_index(np.argmax(grel), grel.shape)
    assert grel.max() <= 2e-2, (f"{what}: rows {gi * group}..{gi * group + group - 1} of head {hi}: "
                                f"group relative error {grel.max():.3g} (reference norm {rn[gi, hi]:.3g}, "
                                f"typical group {typical:.3g})")


def run(call, T, meta=None, scale=None, bwd=True):
    """GPU forward (+ backward) of one call; T holds q, k, v, do (any device)."""
    q, k, v = (T[n].to(DEV) for n in ("q", "k", "v"))
    meta = meta if meta is not None else ffa.build_meta(call.slices, call.Tq, call.Tk, call.d)
    o, lse = ffa.fwd(q, k, v, meta, scale)
    out = {"o": o, "lse": lse, "meta": meta}
    if bwd:
        do = T["do"].to(DEV)
        dq, dk, dv = ffa.bwd(q, k, v, o, lse, do, meta, scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return out


def full_check(call, T, scale=None):
    r = run(call, T, scale=scale)
    assert r["meta"].status() == 0
    o_ref, l_ref = orc.forward(T["q"], T["k"], T["v"], call.slices, scale)
    check_o(r["o"], o_ref)
    check_lse(r["lse"], l_ref)
    dq, dk, dv = orc.backward(T["q"], T["k"], T["v"], T["do"], call.slices, scale)
    check_grad(r["dq"], dq, "dQ")
    check_grad(r["dk"], dk, "dK")
    check_grad(r["dv"], dv, "dV")
    return r


# ---------------------------------------------------- small / medium ----

@pytest.mark.parametrize("variant", ["causal", "mixed", "two_full"])
def test_tiny_varlen(variant):
    W = wl.tiny_varlen(variant)
    c = W.calls[0]
    _say(f"tiny varlen {variant}")
    full_check(c, wl.make_tensors(c, W.seed))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_tables(d, seed):
    rng = random.Random(seed * 10 + d)
    Tq, Tk = rng.randint(300, 900), rng.randint(300, 900)
    Hkv = rng.choice([1, 2])
    Hq = Hkv * rng.choice([1, 2, 4])
    sl = wl.random_slices(rng, Tq, Tk, rng.randint(2, 7))
    c = wl.Call(sl, Tq, Tk, Hq, Hkv, d)
    _say(f"random table seed={seed} d={d}: Tq={Tq} Tk={Tk} Hq={Hq} Hkv={Hkv} slices={sl}")
    full_check(c, wl.make_tensors(c, 1000 + seed))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_banded_tables_several_slices_per_row(d, seed):
    """Tables where query rows attend to the union of several slices with
    disjoint key bands and different types: the per-row OR over a query
    block's slice list in the forward and dQ kernels, and over the column
    intervals of the enclosing block's slices in dK/dV."""
    rng = random.Random(5000 + 10 * seed + d)
    Tq, Tk = rng.randint(300, 1100), rng.randint(300, 1100)
    Hkv = rng.choice([1, 2])
    Hq = Hkv * rng.choice([1, 2, 4])
    sl = wl.random_banded_slices(rng, Tq, Tk, bands=rng.randint(2, 4))
    c = wl.Call(sl, Tq, Tk, Hq, Hkv, d)
    _say(f"banded table seed={seed} d={d}: Tq={Tq} Tk={Tk} Hq={Hq} Hkv={Hkv} slices={sl}")
    full_check(c, wl.make_tensors(c, 2000 + seed))


@pytest.mark.parametrize("mask", [wl.FULL, wl.CAUSAL])
def test_forward_rescale_after_first_stage(mask):
    """Key tiles whose scores grow from tile to tile (keys scaled by 1, 1.5, 4,
    6, 16, 24, 64, 96 per 64-key tile): the running row max rises by more
    than the forward's lazy-rescale threshold (2^8 in the exp2 domain) after
    the first stages, so the branch that rescales O and l runs, and by less
    in between, so P also exceeds 1 between rescales.  Forward against the
    oracle (the backward takes LSE, not the running max)."""
    T, d = 512, 128
    c = wl.Call([(0, T, 0, T, mask)], T, T, 4, 2, d)
    base = wl.make_tensors(c, 4242)
    f = torch.tensor([1, 1.5, 4, 6, 16, 24, 64, 96], dtype=torch.float32).repeat_interleave(64)
    k = (base["k"].float() * f[:, None, None]).to(torch.bfloat16)
    T2 = dict(base, k=k)
    r = run(c, T2, bwd=False)
    o_ref, l_ref = orc.forward(T2["q"], T2["k"], T2["v"], c.slices)
    check_o(r["o"], o_ref)
    check_lse(r["lse"], l_ref)
    # the inputs do what the docstring says: row max after tile 2 exceeds the
    # max over tile 0 by more than the threshold for most rows
    s = torch.einsum("ihd,jhd->hij", T2["q"].double(), k.double().repeat_interleave(2, dim=1))
    thr = 8.0 / ((1.0 / math.sqrt(d)) * 1.4426950408889634)
    jump = s[:, :, 128:192].amax(-1) - s[:, :, 0:64].amax(-1)
    assert float((jump > thr).double().mean()) > 0.5


@pytest.mark.parametrize("Tq,Tk,Hq,Hkv,d", [
    (1, 1, 1, 1, 64), (1, 300, 2, 1, 128), (300, 1, 2, 2, 64), (129, 65, 8, 1, 128),
    (64, 64, 16, 2, 64), (257, 511, 3, 3, 128)])
def test_boundary_shapes(Tq, Tk, Hq, Hkv, d):
    """Single-token query or key ranges, one head, GQA with 8 query heads per
    kv head, sizes one past a tile boundary: every mask type where it fits."""
    rng = random.Random(Tq * 1000 + Tk)
    sl = []
    if Tq >= 2 and Tk >= 2:
        a, b = Tq // 2, Tk // 2
        sl = [(0, a, 0, b, ffa.CAUSAL), (a, Tq, b, Tk, ffa.INV_CAUSAL),
              (0, a, b, Tk, ffa.BI_CAUSAL), (a, Tq, 0, b, ffa.FULL)]
    else:
        sl = [(0, Tq, 0, Tk, rng.choice([ffa.FULL, ffa.CAUSAL]))]
    c = wl.Call(sl, Tq, Tk, Hq, Hkv, d)
    _say(f"boundary Tq={Tq} Tk={Tk} Hq={Hq} Hkv={Hkv} d={d}: {sl}")
    full_check(c, wl.make_tensors(c, Tq + 7 * Tk))


def test_multi_query_many_heads():
    """One kv head shared by 32 query heads (multi-query attention): each dK/dV
    step walks 32 query heads per tile, the split rule sees one kv head with
    a very uneven causal walk, and the block map takes its non-multiple-of-8
    kv-head path.  Varlen causal plus a FULL look-back slice, every output
    against the oracle."""
    sl = wl.varlen_slices([300, 500, 224], ffa.CAUSAL) + [(524, 1024, 0, 300, ffa.FULL)]
    c = wl.Call(sl, 1024, 1024, 32, 1, 128)
    _say(f"multi-query Hq=32 Hkv=1: {sl}")
    full_check(c, wl.make_tensors(c, 77))


def _ws_layout(Tq, Tk, Hq, Hkv, d):
    """Byte offsets of the backward workspace regions (include/ffa.h layout)."""
    a256 = lambda x: (x + 255) // 256 * 256          # noqa: E731
    rows = a256(4 * Hq * Tq)
    E = min(-(-Tk // 128), min(32, max(4, 128 // Hkv)))
    cnt = 3 * rows                                    # -D, LSE log2 e, -LSE / scale
    part = cnt + a256(4 * E * Hkv)
    return {"E": E, "cnt": cnt, "part": part, "end": part + E * Hkv * 2 * 2 * 128 * d * 4}


def test_split_blocks_write_both_partials():
    """One 8K causal sequence: every split candidate (the 32 longest key
    blocks) exceeds a resident workgroup's share, so both halves of each store
    their fp32 partials.  The partial region is filled with NaN before the
    call and must hold no NaN after it (both halves of every candidate ran),
    and dK, dV match the oracle per group of 32 keys (a half that dropped or
    double-added its wave's keys would show in that group)."""
    T = 8192
    c = wl.Call([(0, T, 0, T, ffa.CAUSAL)], T, T, 1, 1, 128)
    tens = wl.make_tensors(c, 99)
    q, k, v, do = (tens[n].to(DEV) for n in ("q", "k", "v", "do"))
    meta = ffa.build_meta(c.slices, T, T, c.d)
    o, lse = ffa.fwd(q, k, v, meta)
    L = _ws_layout(T, T, 1, 1, 128)
    need = ffa.bwd_workspace_size(q, k)
    assert need == L["end"]
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    ws[L["part"]:].view(torch.float32).fill_(float("nan"))
    dq, dk, dv = ffa.bwd(q, k, v, o, lse, do, meta, workspace=ws)
    torch.cuda.synchronize()
    part = ws[L["part"]:].view(torch.float32)
    assert L["E"] == 32 and not bool(torch.isnan(part).any()), "a split half did not store its partial"
    assert bool((ws[L["cnt"]:L["cnt"] + 4 * L["E"]].view(torch.int32) == 0).all()), "counters not reset"
    gq, gk, gv = orc.backward(tens["q"], tens["k"], tens["v"], tens["do"], c.slices)
    check_grad(dq, gq, "dQ")
    check_grad(dk, gk, "dK")
    check_grad(dv, gv, "dV")


def test_one_long_causal_sequence_one_head():
    """A single 8K causal sequence on one head pair: the first key blocks hold
    far more than a resident workgroup's share of the backward, so the dK/dV
    kernel splits its longest-first candidates into two halves (the fp32
    partials meet through the workspace counters); run twice to check that the
    counters are back at zero and the result is bitwise the same."""
    T = 8192
    c = wl.Call([(0, T, 0, T, ffa.CAUSAL)], T, T, 1, 1, 128)
    _say("one long causal sequence T=8192 Hq=Hkv=1 d=128")
    tens = wl.make_tensors(c, 88)
    full_check(c, tens)
    q, k, v, do = (tens[n].to(DEV) for n in ("q", "k", "v", "do"))
    meta = ffa.build_meta(c.slices, T, T, c.d)
    o, lse = ffa.fwd(q, k, v, meta)
    g1 = ffa.bwd(q, k, v, o, lse, do, meta)
    g2 = ffa.bwd(q, k, v, o, lse, do, meta)
    torch.cuda.synchronize()
    for a, b, n in zip(g1, g2, ("dQ", "dK", "dV")):
        assert torch.equal(a, b), f"{n} differs between two identical calls"


def test_backward_phases_separately_match_one_call():
    """PRE, DKDV and DQ run as three calls (standalone row-statistics kernel)
    give the gradients of the single call (row statistics folded into dQ),
    up to the summation order of D."""
    rng = random.Random(77)
    Tq, Tk = 700, 650
    sl = wl.random_slices(rng, Tq, Tk, 5)
    c = wl.Call(sl, Tq, Tk, 4, 2, 128)
    T = wl.make_tensors(c, 77)
    q, k, v, do = (T[n].to(DEV) for n in ("q", "k", "v", "do"))
    meta = ffa.build_meta(sl, Tq, Tk, 128)
    o, lse = ffa.fwd(q, k, v, meta)
    g1 = ffa.bwd(q, k, v, o, lse, do, meta)
    ws = torch.empty(ffa.bwd_workspace_size(q, k), dtype=torch.uint8, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for ph in (ffa.BWD_PRE, ffa.BWD_DKDV, ffa.BWD_DQ):
        ffa.bwd(q, k, v, o, lse, do, meta, dq=dq, dk=dk, dv=dv, workspace=ws, phases=ph)
    torch.cuda.synchronize()
    for a, b, n in zip(g1, (dq, dk, dv), ("dQ", "dK", "dV")):
        a64, b64 = a.double(), b.double()
        rel = float((a64 - b64).norm() / max(float(a64.norm()), 1e-30))
        assert rel <= 1e-3, f"{n}: phased vs single call relative difference {rel:.3g}"


def test_every_mask_type_lq_ne_lk():
    sl = [(0, 100, 0, 300, wl.CAUSAL), (100, 300, 300, 400, wl.CAUSAL),        # Lq > Lk: empty first rows
          (300, 450, 0, 200, wl.INV_CAUSAL), (450, 700, 400, 500, wl.INV_CAUSAL),
          (700, 800, 500, 700, wl.BI_CAUSAL), (800, 900, 700, 750, wl.BI_CAUSAL),  # Lk < Lq: empty
          (900, 1000, 750, 777, wl.FULL)]
    c = wl.Call(sl, 1003, 777, 4, 2, 128)
    full_check(c, wl.make_tensors(c, 7))


def test_softmax_scale_and_strided_inputs():
    c = wl.Call([(0, 200, 0, 260, wl.CAUSAL), (200, 333, 100, 300, wl.FULL)], 333, 300, 4, 2, 64)
    T = wl.make_tensors(c, 8)
    # q, k, v as views of packed buffers (non-contiguous head / token strides)
    qkv = torch.zeros(c.Tq, 3 * c.Hq, c.d, dtype=torch.bfloat16)
    qkv[:, :c.Hq] = T["q"]
    kv = torch.zeros(c.Tk, 4 * c.Hkv, c.d, dtype=torch.bfloat16)
    kv[:, :c.Hkv] = T["k"]
    kv[:, 2 * c.Hkv:3 * c.Hkv] = T["v"]
    qkv_d, kv_d = qkv.to(DEV), kv.to(DEV)
    q, k, v = qkv_d[:, :c.Hq], kv_d[:, :c.Hkv], kv_d[:, 2 * c.Hkv:3 * c.Hkv]
    meta = ffa.build_meta(c.slices, c.Tq, c.Tk, c.d)
    scale = 0.37
    o, lse = ffa.fwd(q, k, v, meta, scale)
    dq, dk, dv = ffa.bwd(q, k, v, o, lse, T["do"].to(DEV), meta, scale)
    o_ref, l_ref = orc.forward(T["q"], T["k"], T["v"], c.slices, scale)
    check_o(o, o_ref)
    check_lse(lse, l_ref)
    gq, gk, gv = orc.backward(T["q"], T["k"], T["v"], T["do"], c.slices, scale)
    check_grad(dq, gq, "dQ")
    check_grad(dk, gk, "dK")
    check_grad(dv, gv, "dV")


def test_empty_table_and_rows_without_keys():
    c = wl.Call([], 200, 150, 2, 1, 128)
    T = wl.make_tensors(c, 9)
    r = run(c, T)
    assert (r["o"] == 0).all() and torch.isneginf(r["lse"]).all()
    assert (r["dq"] == 0).all() and (r["dk"] == 0).all() and (r["dv"] == 0).all()
    # a single short key range, most rows empty, Tk smaller than one key tile
    c = wl.Call([(130, 140, 3, 20, wl.FULL)], 260, 20, 2, 2, 64)
    full_check(c, wl.make_tensors(c, 10))


def test_bad_table_writes_nothing():
    c = wl.Call([(0, 64, 0, 64, 0), (32, 96, 60, 70, 0)], 128, 128, 2, 2, 64)   # overlap
    T = wl.make_tensors(c, 11)
    q, k, v = (T[n].to(DEV) for n in ("q", "k", "v"))
    with pytest.raises(ffa.FFAError, match="overlapping"):
        ffa.build_meta(c.slices, c.Tq, c.Tk, c.d)          # validated by default
    meta = ffa.build_meta(c.slices, c.Tq, c.Tk, c.d, validate=False)
    assert meta.status() == ffa.META_ERR_OVERLAP
    o = torch.full_like(q, 7.0)
    lse = torch.full((c.Hq, c.Tq), 7.0, device=DEV)
    ffa.fwd(q, k, v, meta, out=o, lse=lse)
    torch.cuda.synchronize()
    assert (o == 7.0).all() and (lse == 7.0).all()


# ------------------------------------------------ 16K varlen causal GQA ----

_cache = {}


def _cfg2():
    if "cfg2" not in _cache:
        W = wl.varlen_causal_gqa()
        c = W.calls[0]
        T = wl.make_tensors(c, W.seed)
        _cache["cfg2"] = (c, T, run(c, T))
    return _cache["cfg2"]


def test_varlen_causal_gqa_forward_full():
    c, T, r = _cfg2()
    _say("16K varlen causal: oracle forward")
    o_ref, l_ref = orc.forward(T["q"], T["k"], T["v"], c.slices)
    check_o(r["o"], o_ref)
    check_lse(r["lse"], l_ref)


def test_varlen_causal_gqa_backward_full():
    c, T, r = _cfg2()
    _say("16K varlen causal: oracle backward")
    dq, dk, dv = orc.backward(T["q"], T["k"], T["v"], T["do"], c.slices)
    check_grad(r["dq"], dq, "dQ")
    check_grad(r["dk"], dk, "dK")
    check_grad(r["dv"], dv, "dV")


def test_varlen_causal_head_dim_64_full():
    """The 16K varlen-causal table at head_dim 64 (Hq 16, Hkv 8): every
    element of O, LSE, dQ, dK, dV against the oracle."""
    W = wl.workload(2)
    c = wl.Call(W.calls[0].slices, 16384, 16384, 16, 8, 64)
    T = wl.make_tensors(c, 64)
    _say("16K varlen causal, d = 64: GPU then oracle")
    full_check(c, T)


def test_determinism_and_table_invariance():
    c, T, r = _cfg2()
    r2 = run(c, T)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(r[key], r2[key]), key
    # the same mask written as a permuted and split table gives identical bits
    sl = list(reversed(c.slices))
    q0, q1, k0, k1, t = sl[0]
    mid = (q0 + q1) // 2
    sl = [(q0, mid, k0, mid, wl.CAUSAL), (mid, q1, k0, mid, wl.FULL), (mid, q1, mid, q1, wl.CAUSAL)] + sl[1:]
    c2 = wl.Call(sl, c.Tq, c.Tk, c.Hq, c.Hkv, c.d)
    r3 = run(c2, T)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(r[key], r3[key]), key


# ----------------------------------------------------- full-size cases ----

LARGE = [(3, 0), (4, 0), (4, 1), (5, 0)]


def _gpu_inputs(c, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    shp = {"q": (c.Tq, c.Hq, c.d), "k": (c.Tk, c.Hkv, c.d), "v": (c.Tk, c.Hkv, c.d), "do": (c.Tq, c.Hq, c.d)}
    return {n: torch.randn(*shp[n], generator=g, device=DEV).to(torch.bfloat16) for n in ("q", "k", "v", "do")}


# kv heads whose dK, dV are checked on sampled keys (each with all its query
# heads): the oracle needs the whole forward of those heads for D = dO . O
KEY_HEADS = {(3, 0): [7], (4, 0): [0, 5], (4, 1): [2, 7], (5, 0): [3]}


def _large_results(idx, call):
    """GPU forward + backward of one large workload on random inputs (cached
    for the three parts of test_large_sampled): CPU copies of the inputs, O,
    LSE, dQ and the dK, dV of the KEY_HEADS."""
    key = ("rand", idx, call)
    if key not in _cache:
        _cache.clear()
        W = wl.workload(idx)
        c = W.calls[call]
        _say(f"workload {idx} call {call}: random inputs, GPU fwd+bwd")
        T = _gpu_inputs(c, 100 * idx + call)
        r = run(c, T)
        heads = KEY_HEADS[(idx, call)]
        Tc = {n: t.cpu() for n, t in T.items()}
        res = {n: r[n].cpu() for n in ("o", "lse", "dq")}
        res["dk"], res["dv"] = r["dk"][:, heads].cpu(), r["dv"][:, heads].cpu()
        del T, r
        torch.cuda.empty_cache()
        _cache[key] = (c, Tc, res)
    return _cache[key]


@pytest.mark.parametrize("part", [0, 1, 2])
@pytest.mark.parametrize("idx,call", LARGE)
def test_large_sampled(idx, call, part):
    """Random N(0,1) inputs at full size.  Parts 0 and 1: 4096 sampled query
    rows (two halves), O, LSE, dQ of every head.  Part 2: 4096 sampled key rows,
    dK and dV of one or two kv heads with all their query heads."""
    c, Tc, res = _large_results(idx, call)
    if part < 2:
        rows = np.sort(np.random.default_rng(100 + idx).choice(c.Tq, 4096, replace=False))
        rows = rows[part::2]
        _say(f"workload {idx} call {call} part {part}: oracle on {len(rows)} rows")
        O, L, dQ = orc.forward_backward_rows(Tc["q"], Tc["k"], Tc["v"], Tc["do"], c.slices, rows)
        check_o(res["o"][rows], O)
        check_lse(res["lse"][:, rows], L)
        check_grad(res["dq"][rows], dQ, "dQ")
        return
    heads = KEY_HEADS[(idx, call)]
    keys = np.sort(np.random.default_rng(300 + 10 * idx + call).choice(c.Tk, 4096, replace=False))
    _say(f"workload {idx} call {call}: oracle dK, dV on {len(keys)} keys of kv heads {heads}")
    dK, dV = orc.backward_keys(Tc["q"], Tc["k"], Tc["v"], Tc["do"], c.slices, keys, kv_heads=heads,
                               max_elems=1 << 26, progress=_say)
    check_grad(res["dk"][keys], dK, "dK")
    check_grad(res["dv"][keys], dV, "dV")


@pytest.mark.parametrize("idx,call", LARGE)
def test_large_structured(idx, call):
    """Equal keys and rank-1 values at full size: exact O, LSE for every row,
    dK, dV for 4096 sampled keys, and V = 1 gives O = 1 on non-empty rows."""
    W = wl.workload(idx)
    c = W.calls[call]
    _cache.clear()
    _say(f"workload {idx} call {call}: structured inputs")
    inp = _props.structured_inputs(c.Tq, c.Tk, c.Hq, c.Hkv, c.d, 500 + idx, device=DEV)
    r = run(c, inp)
    o, lse, dk, dv = (r[n].cpu() for n in ("o", "lse", "dk", "dv"))
    ones = {"q": inp["q"], "k": inp["k"], "v": torch.ones_like(inp["v"]), "do": inp["do"]}
    o1 = run(c, ones, meta=r["meta"], bwd=False)["o"].cpu()
    del r
    st = _props.Structured(inp, c.slices, c.Tq, c.Tk)
    for h in range(c.Hq):
        O, L = st.rows(h)
        check_o(o[:, h], O, f"O head {h}")
        check_lse(lse[h], L, f"LSE head {h}")
        want1 = np.where(st.nz[:, None], 1.0, 0.0) * np.ones((1, c.d))
        check_o(o1[:, h], want1, f"O (V=1) head {h}")
    keys = np.sort(np.random.default_rng(200 + idx).choice(c.Tk, 4096, replace=False))
    for g in range(c.Hkv):
        dK, dV = st.keys(g, keys)
        check_grad(dk[keys, g], dK, f"dK head {g}")
        check_grad(dv[keys, g], dV, f"dV head {g}")
