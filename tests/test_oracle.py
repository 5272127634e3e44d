"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: values the pages
print (tests/golden), library attention (torch SDPA in float64), brute force on
a materialised mask, closed forms, finite differences, or an identity the
mathematics fixes.  The mutation tests at the end plant a mistake in the
oracle and check that a pin catches it.
"""
import math
import os
import random

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

from oracle import ffa_oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")
TYPES = (orc.FULL, orc.CAUSAL, orc.INV_CAUSAL, orc.BI_CAUSAL)


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64)


def _sdpa(q, k, v, mask=None, is_causal=False, scale=None):
    """q [Tq,H,d], k/v [Tk,H,d] (same H) -> O [Tq,H,d] via torch SDPA (float64)."""
    qt, kt, vt = (x.permute(1, 0, 2).unsqueeze(0) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, is_causal=is_causal, scale=scale)
    return o.squeeze(0).permute(1, 0, 2)


# ---------------------------------------------------------------- masks ----

@pytest.mark.parametrize("t", TYPES)
def test_row_and_col_intervals_match_predicate(t):
    for Lq in range(0, 9):
        for Lk in range(0, 9):
            s = (2, 2 + Lq, 3, 3 + Lk, t)
            for i in range(0, Lq + 5):
                want = [j for j in range(0, Lk + 6) if orc.valid(i, j, s)]
                iv = orc.row_interval(s, i)
                got = [] if iv is None else list(range(iv[0], iv[1] + 1))
                assert got == want, (s, i)
                lo, hi, ok = orc.row_intervals_vec(s, np.array([i]))
                got_v = list(range(lo[0], hi[0] + 1)) if ok[0] else []
                assert got_v == want
            for j in range(0, Lk + 6):
                want = [i for i in range(0, Lq + 5) if orc.valid(i, j, s)]
                iv = orc.col_interval(s, j)
                got = [] if iv is None else list(range(iv[0], iv[1] + 1))
                assert got == want, (s, j)
                lo, hi, ok = orc.col_intervals_vec(s, np.array([j]))
                got_v = list(range(lo[0], hi[0] + 1)) if ok[0] else []
                assert got_v == want


def test_dense_mask_matches_predicate():
    rng = random.Random(7)
    for _ in range(20):
        Tq, Tk = rng.randint(1, 14), rng.randint(1, 14)
        sl = [(rng.randint(0, Tq), 0, rng.randint(0, Tk), 0, rng.choice(TYPES)) for _ in range(3)]
        sl = [(a, rng.randint(a, Tq), c, rng.randint(c, Tk), t) for (a, _, c, _, t) in sl]
        m = orc.dense_mask(sl, Tq, Tk)
        for i in range(Tq):
            for j in range(Tk):
                assert m[i, j] == sum(orc.valid(i, j, s) for s in sl)


@pytest.mark.parametrize("t", TYPES)
def test_area_closed_form_vs_brute_force(t):
    for Lq in range(0, 13):
        for Lk in range(0, 13):
            s = (1, 1 + Lq, 0, Lk, t)
            assert orc.slice_area(s) == orc.dense_mask([s], 1 + Lq, max(Lk, 1)).sum(), s


def test_area_values_printed_on_pages():
    with open(os.path.join(GOLD, "mask_area.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 8
    for typ, L, area in rows:
        L, area = int(L), int(area)
        t = {"FULL": orc.FULL, "CAUSAL": orc.CAUSAL}[typ]
        assert orc.slice_area((0, L, 0, L, t)) == area
        assert orc.slice_area((5, 5 + L, 9, 9 + L, t)) == area
    # small ones also by brute force on the materialised mask
    for L in (1, 2, 7):
        assert orc.dense_mask([(0, L, 0, L, orc.CAUSAL)], L, L).sum() == L * (L + 1) // 2


def test_flops_values_printed_on_pages():
    with open(os.path.join(GOLD, "flops.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for typ, L, b, hq, d, ff, fb in rows:
        t = {"FULL": orc.FULL, "CAUSAL": orc.CAUSAL}[typ]
        area = orc.slice_area((0, int(L), 0, int(L), t))
        f, bwd = orc.flops(area, int(hq), int(d), int(b))
        assert f == int(ff) and bwd == float(fb)


def test_inclusion_exclusion_causal_inv():
    """CAUSAL u INV = FULL and CAUSAL n INV = BI when Lk >= Lq (mask and area level)."""
    for Lq in range(1, 10):
        for Lk in range(Lq, 12):
            c = orc.dense_mask([(0, Lq, 0, Lk, orc.CAUSAL)], Lq, Lk).astype(bool)
            i = orc.dense_mask([(0, Lq, 0, Lk, orc.INV_CAUSAL)], Lq, Lk).astype(bool)
            f = orc.dense_mask([(0, Lq, 0, Lk, orc.FULL)], Lq, Lk).astype(bool)
            b = orc.dense_mask([(0, Lq, 0, Lk, orc.BI_CAUSAL)], Lq, Lk).astype(bool)
            assert np.array_equal(c | i, f) and np.array_equal(c & i, b)
            a = lambda t: orc.slice_area((0, Lq, 0, Lk, t))
            assert a(orc.CAUSAL) + a(orc.INV_CAUSAL) - a(orc.FULL) == a(orc.BI_CAUSAL)


def test_inv_causal_is_token_reversed_causal():
    for Lq in range(1, 10):
        for Lk in range(1, 10):
            c = orc.dense_mask([(0, Lq, 0, Lk, orc.CAUSAL)], Lq, Lk)
            i = orc.dense_mask([(0, Lq, 0, Lk, orc.INV_CAUSAL)], Lq, Lk)
            assert np.array_equal(i, c[::-1, ::-1])
    # attention level: INV(Q,K,V) = flip(CAUSAL(flip Q, flip K, flip V))
    q, k, v = _rand((11, 2, 8), 1), _rand((15, 2, 8), 2), _rand((15, 2, 8), 3)
    oi, li = orc.forward(q, k, v, [(0, 11, 0, 15, orc.INV_CAUSAL)])
    oc, lc = orc.forward(q.flip(0), k.flip(0), v.flip(0), [(0, 11, 0, 15, orc.CAUSAL)])
    np.testing.assert_allclose(oi, oc[::-1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(li, lc[:, ::-1], rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- forward ----

def test_full_slice_equals_sdpa():
    q, k, v = _rand((37, 3, 16), 10), _rand((53, 3, 16), 11), _rand((53, 3, 16), 12)
    o, lse = orc.forward(q, k, v, [(0, 37, 0, 53, orc.FULL)])
    np.testing.assert_allclose(o, _sdpa(q, k, v).numpy(), rtol=1e-12, atol=1e-12)
    ref_lse = torch.logsumexp(torch.einsum("ihd,jhd->hij", q, k) / 4.0, dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_causal_square_equals_sdpa_is_causal():
    q, k, v = _rand((40, 2, 8), 13), _rand((40, 2, 8), 14), _rand((40, 2, 8), 15)
    o, _ = orc.forward(q, k, v, [(0, 40, 0, 40, orc.CAUSAL)])
    np.testing.assert_allclose(o, _sdpa(q, k, v, is_causal=True).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Lq,Lk", [(10, 30), (30, 30), (7, 8)])
def test_causal_rectangular_equals_sdpa_lower_right(Lq, Lk):
    q, k, v = _rand((Lq, 2, 8), 16), _rand((Lk, 2, 8), 17), _rand((Lk, 2, 8), 18)
    o, _ = orc.forward(q, k, v, [(0, Lq, 0, Lk, orc.CAUSAL)])
    ref = _sdpa(q, k, v, mask=causal_lower_right(Lq, Lk))
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_varlen_causal_equals_per_sequence_sdpa():
    lens = [5, 17, 1, 30, 11]
    T = sum(lens)
    q, k, v = _rand((T, 2, 8), 19), _rand((T, 2, 8), 20), _rand((T, 2, 8), 21)
    sl, s = [], 0
    for L in lens:
        sl.append((s, s + L, s, s + L, orc.CAUSAL))
        s += L
    o, _ = orc.forward(q, k, v, sl)
    s = 0
    for L in lens:
        ref = _sdpa(q[s:s + L], k[s:s + L], v[s:s + L], is_causal=True)
        np.testing.assert_allclose(o[s:s + L], ref.numpy(), rtol=1e-12, atol=1e-12)
        s += L


def _random_table(rng, Tq, Tk, n):
    cuts = sorted(rng.sample(range(1, Tq), n - 1))
    b = [0] + cuts + [Tq]
    out = []
    for q0, q1 in zip(b[:-1], b[1:]):
        k0 = rng.randint(0, Tk - 1)
        out.append((q0, q1, k0, rng.randint(k0 + 1, Tk), rng.choice(TYPES)))
    return out


def _banded_table(rng, Tq, Tk):
    """Disjoint table with several slices per query row: query bands, each with
    2-4 disjoint key ranges of random types (the workload generator's recipe,
    restated here so that the oracle pins do not depend on it)."""
    cuts = sorted(rng.sample(range(1, Tq), 2))
    b = [0] + cuts + [Tq]
    out = []
    for q0, q1 in zip(b[:-1], b[1:]):
        n = rng.randint(2, 4)
        pts = sorted(rng.sample(range(0, Tk + 1), 2 * n))
        for i in range(n):
            a, z = rng.randint(q0, q1 - 1), rng.randint(q0 + 1, q1)
            qa, qz = min(a, z - 1), max(a + 1, z)
            out.append((qa, qz, pts[2 * i], pts[2 * i + 1], rng.choice(TYPES)))
    return out


def test_random_tables_equal_sdpa_with_materialised_mask():
    rng = random.Random(3)
    for trial in range(12):
        Tq, Tk, H, Hkv = rng.randint(8, 60), rng.randint(8, 60), 4, rng.choice([1, 2, 4])
        sl = _random_table(rng, Tq, Tk, rng.randint(1, 5)) if trial % 2 else _banded_table(rng, Tq, Tk)
        q, k, v = _rand((Tq, H, 8), 100 + trial), _rand((Tk, Hkv, 8), 200 + trial), _rand((Tk, Hkv, 8), 300 + trial)
        assert orc.validate(sl, Tq, Tk) == 0
        o, lse = orc.forward(q, k, v, sl)
        mask = torch.from_numpy(orc.dense_mask(sl, Tq, Tk).astype(bool))
        rep = H // Hkv
        kk, vv = k.repeat_interleave(rep, dim=1), v.repeat_interleave(rep, dim=1)
        ref = _sdpa(q, kk, vv, mask=mask).numpy()
        empty = ~mask.numpy().any(axis=1)
        np.testing.assert_allclose(o[~empty], ref[~empty], rtol=1e-11, atol=1e-12)
        assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[:, empty]))
        S = torch.einsum("ihd,jhd->hij", q, kk) / math.sqrt(8)
        ref_lse = torch.logsumexp(S.masked_fill(~mask, -math.inf), dim=-1).numpy()
        np.testing.assert_allclose(lse[:, ~empty], ref_lse[:, ~empty], rtol=1e-12, atol=1e-12)


def test_split_along_k_lse_merge():
    """Restricting M to keys < t and >= t and LSE-merging gives the whole result."""
    q, k, v = _rand((48, 2, 8), 30), _rand((64, 2, 8), 31), _rand((64, 2, 8), 32)
    # FULL -> FULL + FULL
    o, l = orc.forward(q, k, v, [(0, 48, 0, 64, orc.FULL)])
    o1, l1 = orc.forward(q, k, v, [(0, 48, 0, 20, orc.FULL)])
    o2, l2 = orc.forward(q, k, v, [(0, 48, 20, 64, orc.FULL)])
    om, lm = orc.lse_merge(o1, l1, o2, l2)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lm, l, rtol=1e-12, atol=1e-12)
    # CAUSAL (square) -> {CAUSAL [0,t)^2, FULL [t,L)x[0,t)} + {CAUSAL [t,L)^2}
    L, t = 48, 19
    o, l = orc.forward(q, k[:L], v[:L], [(0, L, 0, L, orc.CAUSAL)])
    o1, l1 = orc.forward(q, k[:L], v[:L], [(0, t, 0, t, orc.CAUSAL), (t, L, 0, t, orc.FULL)])
    o2, l2 = orc.forward(q, k[:L], v[:L], [(t, L, t, L, orc.CAUSAL)])
    om, lm = orc.lse_merge(o1, l1, o2, l2)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lm, l, rtol=1e-12, atol=1e-12)


def test_empty_rows_and_special_inputs():
    # BI_CAUSAL with Lk < Lq is entirely empty; CAUSAL with Lq > Lk empties its first rows
    q, k, v = _rand((12, 1, 4), 40), _rand((12, 1, 4), 41), _rand((12, 1, 4), 42)
    o, l = orc.forward(q, k, v, [(0, 6, 0, 4, orc.BI_CAUSAL), (6, 12, 0, 3, orc.CAUSAL)])
    assert np.all(o[:6] == 0) and np.all(np.isneginf(l[:, :6]))
    assert np.all(o[6:9] == 0) and np.all(np.isfinite(l[:, 9:]))
    # Q = 0: LSE_i = ln |J_i| and O_i = mean of V over J_i
    sl = [(0, 12, 2, 10, orc.BI_CAUSAL)]
    o, l = orc.forward(torch.zeros(12, 1, 4, dtype=torch.float64), k, v, sl)
    for i in range(12):
        J = orc.valid_keys(sl, i)
        if len(J):
            assert abs(l[0, i] - math.log(len(J))) < 1e-13
            np.testing.assert_allclose(o[i, 0], v[J, 0].numpy().mean(axis=0), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- backward ----

def test_backward_equals_autograd_through_sdpa():
    rng = random.Random(5)
    for trial in range(6):
        Tq, Tk, H, Hkv = rng.randint(8, 40), rng.randint(8, 40), 4, rng.choice([1, 2, 4])
        sl = _random_table(rng, Tq, Tk, rng.randint(1, 4))
        q, k, v = _rand((Tq, H, 8), 50 + trial), _rand((Tk, Hkv, 8), 60 + trial), _rand((Tk, Hkv, 8), 70 + trial)
        do = _rand((Tq, H, 8), 80 + trial)
        mask = torch.from_numpy(orc.dense_mask(sl, Tq, Tk).astype(bool))
        empty = ~mask.any(dim=1)
        mask_f = mask.clone()
        mask_f[empty] = True          # keep SDPA finite; those rows are zeroed below
        qq, kk, vv = (x.clone().requires_grad_(True) for x in (q, k, v))
        rep = H // Hkv
        o = _sdpa(qq, kk.repeat_interleave(rep, 1), vv.repeat_interleave(rep, 1), mask=mask_f)
        o = o * (~empty).to(o.dtype)[:, None, None]
        (o * do).sum().backward()
        dq, dk, dv = orc.backward(q, k, v, do, sl)
        np.testing.assert_allclose(dq, qq.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, kk.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, vv.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("t", TYPES)
def test_backward_finite_differences(t):
    Tq, Tk, H, Hkv, d = 6, 7, 2, 1, 3
    sl = [(0, 6, 0, 7, t)] if t != orc.BI_CAUSAL else [(0, 4, 0, 7, t), (4, 6, 0, 2, orc.FULL)]
    q, k, v, do = (_rand(s, 90 + n).numpy() for n, s in enumerate(
        [(Tq, H, d), (Tk, Hkv, d), (Tk, Hkv, d), (Tq, H, d)]))
    dq, dk, dv = orc.backward(q, k, v, do, sl)

    def loss(q_, k_, v_):
        o, _ = orc.forward(q_, k_, v_, sl)
        return float((o * do).sum())

    eps = 1e-6
    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.linalg.norm(num - g) <= 1e-6 * max(1.0, np.linalg.norm(g)), which


def _autograd_dkdv(q, k, v, do, sl):
    """dK, dV through torch SDPA (float64) with a materialised mask."""
    Tq, H = q.shape[0], q.shape[1]
    Tk, Hkv = k.shape[0], k.shape[1]
    mask = torch.from_numpy(orc.dense_mask(sl, Tq, Tk).astype(bool))
    empty = ~mask.any(dim=1)
    mask_f = mask.clone()
    mask_f[empty] = True
    kk, vv = k.clone().requires_grad_(True), v.clone().requires_grad_(True)
    rep = H // Hkv
    o = _sdpa(q, kk.repeat_interleave(rep, 1), vv.repeat_interleave(rep, 1), mask=mask_f)
    o = o * (~empty).to(o.dtype)[:, None, None]
    (o * do).sum().backward()
    return kk.grad.numpy(), vv.grad.numpy()


def test_backward_keys_equals_autograd_on_sampled_keys():
    """dK, dV restricted to sampled key rows and a subset of kv heads equal
    the autograd gradient at those rows (several slices per query row, GQA,
    rows without keys, a tiny batch budget so rows and windows are split)."""
    rng = random.Random(21)
    for trial in range(6):
        Tq, Tk, Hkv = rng.randint(20, 70), rng.randint(20, 70), rng.choice([1, 2, 3])
        H = Hkv * rng.choice([1, 2])
        sl = _banded_table(rng, Tq, Tk)
        q, k, v, do = (_rand(s, 500 + 10 * trial + n) for n, s in enumerate(
            [(Tq, H, 8), (Tk, Hkv, 8), (Tk, Hkv, 8), (Tq, H, 8)]))
        dk_ref, dv_ref = _autograd_dkdv(q, k, v, do, sl)
        keys = np.array(rng.sample(range(Tk), rng.randint(1, Tk)))      # unsorted, distinct
        heads = sorted(rng.sample(range(Hkv), rng.randint(1, Hkv)))
        dK, dV = orc.backward_keys(q, k, v, do, sl, keys, kv_heads=heads,
                                   max_elems=rng.choice([1 << 25, 97]))
        np.testing.assert_allclose(dK, dk_ref[keys][:, heads], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dV, dv_ref[keys][:, heads], rtol=1e-10, atol=1e-12)


def test_backward_keys_scale_and_key_order():
    """A non-default scale, repeated and unsorted keys: each output row is
    the gradient of its own key."""
    sl = [(0, 30, 0, 40, orc.CAUSAL), (0, 30, 40, 55, orc.BI_CAUSAL), (30, 50, 10, 55, orc.FULL)]
    q, k, v, do = _rand((50, 2, 8), 1), _rand((55, 1, 8), 2), _rand((55, 1, 8), 3), _rand((50, 2, 8), 4)
    dq, dk, dv = orc.backward(q, k, v, do, sl, scale=0.3)
    keys = np.array([54, 3, 3, 40, 0, 39])
    dK, dV = orc.backward_keys(q, k, v, do, sl, keys, scale=0.3)
    np.testing.assert_allclose(dK, dk[keys], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dV, dv[keys], rtol=1e-12, atol=1e-13)


def test_dk_sums_to_zero_and_dq_rows():
    rng = random.Random(9)
    sl = _random_table(rng, 50, 70, 4)
    q, k, v, do = _rand((50, 4, 8), 1), _rand((70, 2, 8), 2), _rand((70, 2, 8), 3), _rand((50, 4, 8), 4)
    dq, dk, dv = orc.backward(q, k, v, do, sl)
    assert np.abs(dk.sum(axis=0)).max() < 1e-12
    rows = np.array([0, 3, 17, 49])
    np.testing.assert_allclose(orc.backward_dq_rows(q, k, v, do, sl, rows), dq[rows], rtol=1e-12, atol=1e-13)
    o_rows, l_rows = orc.forward(q, k, v, sl, rows=rows)
    o_all, l_all = orc.forward(q, k, v, sl)
    np.testing.assert_allclose(o_rows, o_all[rows], rtol=1e-13, atol=1e-14)


def test_row_batching_does_not_change_results():
    rng = random.Random(11)
    sl = _random_table(rng, 90, 80, 6)
    q, k, v = _rand((90, 2, 8), 5), _rand((80, 2, 8), 6), _rand((80, 2, 8), 7)
    o1, l1 = orc.forward(q, k, v, sl, max_elems=1 << 22)
    o2, l2 = orc.forward(q, k, v, sl, max_elems=1)        # one row per batch
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------ metadata ----

@pytest.mark.parametrize("BM,BN", [(4, 4), (8, 3), (5, 16), (128, 64), (64, 128)])
def test_tile_counts_interval_form_vs_brute_force(BM, BN):
    rng = random.Random(BM * 100 + BN)
    for _ in range(8):
        Tq, Tk = rng.randint(1, 300), rng.randint(1, 300)
        sl = _random_table(rng, Tq, Tk, rng.randint(1, min(6, Tq))) if Tq > 1 else [(0, 1, 0, Tk, 0)]
        dense = orc.tile_counts_dense(sl, Tq, Tk, BM, BN)
        sparse = orc.tile_counts(sl, Tq, Tk, BM, BN)
        for m in range(dense.shape[0]):
            got = sparse.get(m, np.zeros(dense.shape[1], dtype=np.int64))
            assert np.array_equal(got, dense[m])
        for direction in ("q2k", "k2q"):
            a = orc.block_meta(sl, Tq, Tk, BM, BN, direction, dense=True)
            b = orc.block_meta(sl, Tq, Tk, BM, BN, direction, dense=False)
            for key in a:
                assert np.array_equal(a[key], b[key]), key
        assert a["area"] == orc.total_area(sl) == orc.dense_mask(sl, Tq, Tk).sum()


def test_block_meta_out_of_bounds_rule_from_pages():
    with open(os.path.join(GOLD, "block_meta_oob.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    Tq, Tk, BM, BN = map(int, rows[0])
    sl = [(0, Tq, 0, Tk, orc.FULL)]
    metas = {d: orc.block_meta(sl, Tq, Tk, BM, BN, d) for d in ("q2k", "k2q")}
    for r in rows[1:]:
        direction, owner = r[0], int(r[1])
        semi = r.index(";")
        full = [int(x) for x in r[2:semi]]
        mask = [int(x) for x in r[semi + 1:]]
        m = metas[direction]
        fo, mo = m["full_block_offset"], m["mask_block_offset"]
        assert list(m["full_block_idx"][fo[owner]:fo[owner + 1]]) == full
        assert list(m["mask_block_idx"][mo[owner]:mo[owner + 1]]) == mask


def test_block_meta_depends_only_on_the_mask():
    """Permuting a table, or splitting its slices, leaves the metadata unchanged."""
    rng = random.Random(12)
    sl = [(0, 40, 0, 40, orc.CAUSAL), (40, 100, 10, 90, orc.FULL), (100, 150, 60, 170, orc.BI_CAUSAL),
          (150, 200, 0, 30, orc.INV_CAUSAL)]
    perm = sl[:]
    rng.shuffle(perm)
    split = [(0, 17, 0, 17, orc.CAUSAL), (17, 40, 0, 17, orc.FULL), (17, 40, 17, 40, orc.CAUSAL),
             (40, 70, 10, 90, orc.FULL), (70, 100, 10, 50, orc.FULL), (70, 100, 50, 90, orc.FULL),
             (100, 150, 60, 170, orc.BI_CAUSAL), (150, 200, 0, 30, orc.INV_CAUSAL)]
    assert np.array_equal(orc.dense_mask(split, 200, 170), orc.dense_mask(sl, 200, 170))
    for direction in ("q2k", "k2q"):
        ref = orc.block_meta(sl, 200, 170, 16, 32, direction)
        for other in (perm, split):
            got = orc.block_meta(other, 200, 170, 16, 32, direction)
            for key in ref:
                assert np.array_equal(ref[key], got[key])


def test_validate_flags():
    assert orc.validate([(0, 10, 0, 10, 1), (10, 20, 0, 20, 0)], 20, 20) == 0
    assert orc.validate([(0, 21, 0, 10, 1)], 20, 20) == orc.ERR_BOUNDS
    assert orc.validate([(5, 4, 0, 10, 1)], 20, 20) == orc.ERR_BOUNDS
    assert orc.validate([(0, 10, 0, 10, 7)], 20, 20) == orc.ERR_TYPE
    assert orc.validate([(0, 10, 0, 10, 0), (5, 15, 9, 12, 0)], 20, 20) == orc.ERR_OVERLAP
    # CAUSAL and INV_CAUSAL on the same square share the diagonal
    assert orc.validate([(0, 8, 0, 8, 1), (0, 8, 0, 8, 2)], 8, 8) == orc.ERR_OVERLAP
    # CAUSAL and its strict complement do not overlap
    comp = [(0, 8, 0, 8, orc.CAUSAL)] + [(i, i + 1, i + 1, 8, orc.FULL) for i in range(7)]
    assert orc.validate(comp, 8, 8) == 0
    assert orc.dense_mask(comp, 8, 8).max() == 1


def test_validate_overlap_equals_dense_count():
    """The overlap flag against its definition: two slices share a valid
    (i, j) iff the materialised count of slices containing some cell exceeds
    one.  Random small tables of every mask type, many of them overlapping,
    with Lq != Lk and slices touching along the diagonal."""
    rng = random.Random(31)
    seen = [0, 0]
    for _ in range(600):
        T = rng.choice([6, 11, 24])
        sl = []
        for _ in range(rng.randint(2, 5)):
            a, b = sorted(rng.sample(range(T + 1), 2))
            c, d = sorted(rng.sample(range(T + 1), 2))
            sl.append((a, b, c, d, rng.randint(0, 3)))
        want = orc.ERR_OVERLAP if orc.dense_mask(sl, T, T).max() > 1 else 0
        assert orc.validate(sl, T, T) == want, sl
        seen[want != 0] += 1
    assert min(seen) > 100


# ------------------------------------------------- planted mistakes ----

def test_pins_catch_planted_mistakes(monkeypatch):
    """A wrong diagonal offset in the interval form must break the SDPA pin, and
    a wrong causal area must break the pages' area values."""
    real = orc.row_intervals_vec

    def off_by_one(s, rows):
        lo, hi, ok = real(s, rows)
        return lo, hi - (1 if s[4] == orc.CAUSAL else 0), ok

    monkeypatch.setattr(orc, "row_intervals_vec", off_by_one)
    with pytest.raises(AssertionError):
        test_causal_square_equals_sdpa_is_causal()
    monkeypatch.setattr(orc, "row_intervals_vec", real)

    real_area = orc.slice_area
    monkeypatch.setattr(orc, "slice_area",
                        lambda s: real_area(s) - (s[1] - s[0]) * (s[4] == orc.CAUSAL))
    with pytest.raises(AssertionError):
        test_area_values_printed_on_pages()
    monkeypatch.setattr(orc, "slice_area", real_area)

    real_bwd = orc.backward

    def bad_bwd(*a, **kw):
        dq, dk, dv = real_bwd(*a, **kw)
        return dq, -dk, dv
    monkeypatch.setattr(orc, "backward", bad_bwd)
    with pytest.raises(AssertionError):
        test_backward_finite_differences(orc.CAUSAL)
