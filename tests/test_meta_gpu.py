"""Block metadata on the GPU must equal the oracle's bit for bit (integer work)."""
import random

import numpy as np
import pytest
import torch

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl
from oracle import ffa_oracle as orc

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _expected_slice_lists(slices, Tq, Tk, BM):
    nq = -(-Tq // BM)
    out = [[] for _ in range(nq)]
    for i, (q0, q1, k0, k1, t) in enumerate(slices):
        if not (0 <= q0 <= q1 <= Tq and 0 <= k0 <= k1 <= Tk and 0 <= t <= 3):
            continue
        if q1 <= q0 or k1 <= k0:
            continue
        for m in range(q0 // BM, (q1 - 1) // BM + 1):
            out[m].append(i)
    return out


def check_meta(slices, Tq, Tk, d=128, meta=None):
    m = meta if meta is not None else ffa.build_meta(slices, Tq, Tk, d, validate=False)
    csr = m.csr()
    BMf, BNf, BMb, BNb = csr["tiles"]
    assert m.status() == orc.validate(slices, Tq, Tk)
    if m.status():
        return m, csr
    assert m.area() == orc.total_area(slices)
    for direction, (BM, BN) in (("q2k", (BMf, BNf)), ("k2q", (BMb, BNb))):
        ref = orc.block_meta(slices, Tq, Tk, BM, BN, direction)
        got = csr[direction]
        for key in ("full_block_offset", "full_block_idx", "mask_block_offset", "mask_block_idx"):
            assert np.array_equal(got[key].numpy(), ref[key]), (direction, key)
    lists = _expected_slice_lists(slices, Tq, Tk, BMf)
    qs_off, qs_idx = csr["qblock_slice_offset"].numpy(), csr["qblock_slice_idx"].numpy()
    for mblk, want in enumerate(lists):
        assert list(qs_idx[qs_off[mblk]:qs_off[mblk + 1]]) == want
    for sched, which in ((csr["schedule_fwd"], "q2k"), (csr["schedule_bwd"], "k2q")):
        s = sched.numpy()
        assert sorted(s.tolist()) == list(range(len(s)))
        fo = csr[which]["full_block_offset"].numpy()
        mo = csr[which]["mask_block_offset"].numpy()
        cost = 4 * np.diff(fo) + 5 * np.diff(mo)
        assert np.all(np.diff(cost[s]) <= 0)
        check_records(csr, which, s, fo, mo)
    return m, csr


def check_records(csr, which, s, fo, mo):
    """Block records in schedule order: owner, list offsets and counts, and the
    first (q2k) or last (k2q) entry of each list, -1 for an empty list."""
    rec = csr["records_fwd" if which == "q2k" else "records_bwd"].numpy()
    fi = csr[which]["full_block_idx"].numpy()
    mi = csr[which]["mask_block_idx"].numpy()
    nf, nm = fo[s + 1] - fo[s], mo[s + 1] - mo[s]
    assert np.array_equal(rec[:, 0], s)
    assert np.array_equal(rec[:, 1], fo[s]) and np.array_equal(rec[:, 2], nf)
    assert np.array_equal(rec[:, 3], mo[s]) and np.array_equal(rec[:, 4], nm)
    if which == "q2k":
        qs = csr["qblock_slice_offset"].numpy()
        assert np.array_equal(rec[:, 5], qs[s]) and np.array_equal(rec[:, 6], qs[s + 1] - qs[s])
        tf = np.where(nf > 0, fi[np.minimum(fo[s], max(len(fi) - 1, 0))] if len(fi) else -1, -1)
        tp = np.where(nm > 0, mi[np.minimum(mo[s], max(len(mi) - 1, 0))] if len(mi) else -1, -1)
        assert np.array_equal(rec[:, 7], tf) and np.array_equal(rec[:, 8], tp)
    else:
        tf = np.where(nf > 0, fi[np.clip(fo[s] + nf - 1, 0, max(len(fi) - 1, 0))] if len(fi) else -1, -1)
        tp = np.where(nm > 0, mi[np.clip(mo[s] + nm - 1, 0, max(len(mi) - 1, 0))] if len(mi) else -1, -1)
        assert np.array_equal(rec[:, 5], tf) and np.array_equal(rec[:, 6], tp)


@pytest.mark.parametrize("variant", ["causal", "mixed", "two_full"])
def test_meta_tiny(variant):
    c = wl.tiny_varlen(variant).calls[0]
    check_meta(c.slices, c.Tq, c.Tk, c.d)


@pytest.mark.parametrize("idx,call", [(2, 0), (3, 0), (4, 0), (4, 1), (5, 0)])
def test_meta_workloads(idx, call):
    c = wl.workload(idx).calls[call]
    _say(f"meta parity: workload {idx} call {call}: {len(c.slices)} slices, Tq={c.Tq} Tk={c.Tk}")
    check_meta(c.slices, c.Tq, c.Tk, c.d)


def test_meta_random_tables():
    rng = random.Random(1234)
    for trial in range(40):
        Tq, Tk = rng.randint(1, 700), rng.randint(1, 700)
        n = rng.randint(1, min(8, Tq))
        sl = wl.random_slices(rng, Tq, Tk, n) if Tq > 1 else [(0, 1, 0, Tk, rng.randint(0, 3))]
        _say(f"random table {trial}: Tq={Tq} Tk={Tk} n={len(sl)}")
        check_meta(sl, Tq, Tk, rng.choice([64, 128]))


def test_meta_multi_slice_tiles_and_empty():
    # several slices share tiles; zero-area slices; a BI_CAUSAL with Lk < Lq (empty)
    sl = [(0, 50, 0, 30, wl.CAUSAL), (0, 50, 30, 90, wl.FULL), (50, 70, 10, 15, wl.BI_CAUSAL),
          (70, 70, 0, 10, wl.FULL), (70, 200, 90, 91, wl.INV_CAUSAL), (200, 333, 0, 300, wl.BI_CAUSAL)]
    check_meta(sl, 333, 300)
    check_meta([], 100, 100)


def test_meta_invariant_under_permutation_and_splitting():
    sl = [(0, 40, 0, 40, 1), (40, 100, 10, 90, 0), (100, 150, 60, 170, 3), (150, 200, 0, 30, 2)]
    split = [(0, 17, 0, 17, 1), (17, 40, 0, 17, 0), (17, 40, 17, 40, 1), (40, 70, 10, 90, 0),
             (70, 100, 10, 50, 0), (70, 100, 50, 90, 0), (100, 150, 60, 170, 3), (150, 200, 0, 30, 2)]
    _, a = check_meta(sl, 200, 170)
    _, b = check_meta(list(reversed(sl)), 200, 170)
    _, c = check_meta(split, 200, 170)
    for other in (b, c):
        for direction in ("q2k", "k2q"):
            for key in a[direction]:
                assert torch.equal(a[direction][key], other[direction][key])


def test_meta_status_flags():
    assert check_meta([(0, 10, 0, 10, 0), (5, 15, 9, 12, 0)], 20, 20)[0].status() == ffa.META_ERR_OVERLAP
    assert check_meta([(0, 8, 0, 8, 1), (0, 8, 0, 8, 2)], 8, 8)[0].status() == ffa.META_ERR_OVERLAP
    assert check_meta([(0, 21, 0, 10, 1)], 20, 20)[0].status() == ffa.META_ERR_BOUNDS
    assert check_meta([(3, 2, 0, 10, 1)], 20, 20)[0].status() == ffa.META_ERR_BOUNDS
    assert check_meta([(0, 10, 0, 10, 9)], 20, 20)[0].status() == ffa.META_ERR_TYPE
    # a buffer too small for the lists sets the capacity flag (and nothing is written past it)
    sl = wl.varlen_causal_gqa().calls[0].slices
    need = ffa.meta_workspace_size(len(sl), 16384, 16384, 128, torch.tensor(sl, dtype=torch.int32))
    fixed = ffa.meta_workspace_size(len(sl), 16384, 16384, 128, torch.zeros(len(sl), 5, dtype=torch.int32))
    guard = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    m = ffa.build_meta(sl, 16384, 16384, 128, out=guard[:fixed + 256], validate=False)
    assert m.status() & ffa.META_ERR_CAPACITY
    assert bool((guard[fixed + 256:] == 0x5A).all())


def test_meta_and_attention_with_thousands_of_slices():
    """3,000 short causal sequences plus FULL cross-sequence blocks (long
    per-block slice lists, many slices per tile): metadata bit-exact, and the
    attention on it against the oracle."""
    rng = random.Random(99)
    lens = [rng.randint(1, 16) for _ in range(3000)]
    sl, s = [], 0
    for L in lens:
        sl.append((s, s + L, s, s + L, wl.CAUSAL))
        s += L
    T = s
    # every 50th sequence also sees the 8 tokens before its start (a FULL
    # slice over keys left of its own range: disjoint from the causal ones)
    s = 0
    for i, L in enumerate(lens):
        if i % 50 == 0 and s >= 8:
            sl.append((s, s + L, s - 8, s, wl.FULL))
        s += L
    _say(f"{len(sl)} slices over {T} tokens")
    check_meta(sl, T, T, 64)
    from tests.test_attention_gpu import full_check
    c = wl.Call(sl, T, T, 2, 1, 64)
    full_check(c, wl.make_tensors(c, 5))


def test_meta_overlap_flag_random_tables():
    """The disjointness test on random small tables of every mask type (many
    overlapping, many touching along a diagonal, Lq != Lk): the status word
    equals the oracle's flags table by table."""
    rng = random.Random(1234)
    seen = [0, 0]
    for n in range(1500):
        T = rng.choice([8, 40, 200, 700])
        sl = []
        for _ in range(rng.randint(2, 4)):
            a, b = sorted(rng.sample(range(T + 1), 2))
            c, d = sorted(rng.sample(range(T + 1), 2))
            sl.append((a, b, c, d, rng.randint(0, 3)))
        m = ffa.build_meta(sl, T, T, 64, validate=False)
        want = orc.validate(sl, T, T)
        assert m.status() == want, (n, T, sl)
        seen[want != 0] += 1
    _say(f"tables with an overlap: {seen[1]}, without: {seen[0]}")
    assert min(seen) > 300


def _causal_and_strict_upper(lens):
    """Per sequence a CAUSAL slice and an INV_CAUSAL slice one key to the
    right over one row less: the strict upper triangle.  The two share their
    bounding box but no (query, key) pair."""
    sl, s = [], 0
    for L in lens:
        sl.append((s, s + L, s, s + L, wl.CAUSAL))
        if L > 1:
            sl.append((s, s + L - 1, s + 1, s + L, wl.INV_CAUSAL))
        s += L
    return sl, s


def test_meta_validation_ten_thousand_slices():
    """A table of 10,000 slices whose pairs share bounding boxes but not valid
    pairs (status 0, as the oracle finds), then the same table with one
    planted overlap, one out-of-bounds slice and one bad type: the status
    word equals the oracle's flags in each case."""
    rng = random.Random(77)
    lens = [rng.randint(2, 24) for _ in range(5000)]
    sl, T = _causal_and_strict_upper(lens)
    assert len(sl) == 10000
    _say(f"{len(sl)} slices over {T} tokens")
    m = ffa.build_meta(sl, T, T, 128, validate=False)
    assert orc.validate(sl, T, T) == 0
    assert m.status() == 0
    # the two slices of a sequence tile its square exactly
    assert m.area() == orc.total_area(sl) == sum(L * L for L in lens)
    # one INV_CAUSAL slice moved onto its sequence's diagonal
    i = 2 * 2500 + 1
    q0, q1, k0, k1, t = sl[i]
    bad = list(sl)
    bad[i] = (q0, q1, k0 - 1, k1 - 1, t)
    assert orc.validate(bad, T, T) == orc.ERR_OVERLAP
    assert ffa.build_meta(bad, T, T, 128, validate=False).status() == orc.ERR_OVERLAP
    # plus a slice past the end and one of an unknown type
    worse = bad + [(T - 4, T + 1, 0, 4, wl.FULL), (0, 1, T - 1, T, 7)]
    want = orc.validate(worse, T, T)
    assert want == orc.ERR_OVERLAP | orc.ERR_BOUNDS | orc.ERR_TYPE
    assert ffa.build_meta(worse, T, T, 128, validate=False).status() == want
