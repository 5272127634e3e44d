"""Context-parallel dispatch (host-only entry points of the library) against
the oracle in oracle/dispatch_oracle.py, and that oracle against brute force
and closed forms.

Pins of the oracle:
  * chunk areas counted on the materialised mask equal the closed form of a
    causal / full slice (sum of row lengths over the chunk's rows) and the
    row-interval sum;
  * the greedy keeps equal chunk counts and the total area, is never better
    than the exhaustive optimum, reaches it where the optimum is known (equal
    areas; a causal sequence cut into 2 * cp chunks, where pairing chunk i with
    chunk n - 1 - i balances exactly), and a planted mistake (lightest-bucket
    rule dropped) is caught;
  * the exhaustive optimum equals a plain enumeration of equal-count
    labellings on small inputs and a worked example, and a search that drops
    the equal-count rule is caught.
Library checks: chunk areas and bucket choices identical to the oracle's; a
rank's local slice table reproduces the global mask on its queries and the
keys it receives exactly, and every valid key of those queries is received.
"""
import itertools
import random

import numpy as np
import pytest

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl
from oracle import dispatch_oracle as dor
from oracle import ffa_oracle as orc


def _block_causal_table(rng, T, block):
    """Varlen block-causal table: several FULL slices per sample share q rows
    with disjoint k ranges only when blocks differ, so q ranges repeat across
    slices of different samples' keys (exercises slices cut inside q)."""
    cuts = sorted(rng.sample(range(1, T), 3))
    b = [0] + cuts + [T]
    out = []
    for S, E in zip(b[:-1], b[1:]):
        for bs in range(S, E, block):
            be = min(bs + block, E)
            out.append((bs, be, S, be, ffa.FULL))
    return out


def _tables():
    rng = random.Random(7)
    yield "varlen_causal", wl.varlen_slices([300, 700, 1048], ffa.CAUSAL), 2048, 2048
    yield "block_causal", _block_causal_table(rng, 1500, 128), 1500, 1500
    for i in range(4):
        Tq, Tk = rng.randint(200, 900), rng.randint(100, 900)
        yield f"random{i}", wl.random_slices(rng, Tq, Tk, rng.randint(1, 7)), Tq, Tk
    # every type with Lq != Lk, and an INV / BI pair split across chunks
    yield "types", [(0, 200, 50, 120, ffa.CAUSAL), (200, 300, 0, 300, ffa.INV_CAUSAL),
                    (300, 500, 100, 400, ffa.BI_CAUSAL), (500, 640, 600, 700, ffa.FULL)], 640, 700


# --------------------------------------------------------------- oracle pins

@pytest.mark.parametrize("L,chunk", [(1000, 128), (512, 512), (777, 100)])
def test_oracle_chunk_areas_closed_form(L, chunk):
    causal = [(0, L, 0, L, orc.CAUSAL)]
    full = [(0, L, 0, L // 2, orc.FULL)]
    n = dor.num_chunks(L, chunk)
    exp_c = [sum(r + 1 for r in range(c * chunk, min((c + 1) * chunk, L))) for c in range(n)]
    exp_f = [(min((c + 1) * chunk, L) - c * chunk) * (L // 2) for c in range(n)]
    assert dor.chunk_areas_dense(causal, L, L, chunk) == exp_c
    assert dor.chunk_areas_dense(full, L, L // 2, chunk) == exp_f
    assert dor.chunk_areas_rows(causal, L, chunk) == exp_c
    assert sum(exp_c) == L * (L + 1) // 2


def test_oracle_chunk_areas_rows_vs_dense():
    for name, sl, Tq, Tk in _tables():
        for chunk in (64, 100, 512):
            assert dor.chunk_areas_rows(sl, Tq, chunk) == dor.chunk_areas_dense(sl, Tq, Tk, chunk), name


def test_oracle_greedy_invariants_and_optimum():
    rng = random.Random(3)
    for _ in range(60):
        cp = rng.choice([1, 2, 3])
        n = cp * rng.choice([1, 2, 3]) if cp > 1 else rng.randint(1, 6)
        areas = [rng.choice([0, 1, 5, 9, rng.randint(0, 50)]) for _ in range(n)]
        b = dor.greedy_dispatch(areas, cp)
        assert sorted(b) == sorted([x for x in range(cp) for _ in range(n // cp)])
        g = dor.max_load(areas, b, cp)
        opt = dor.best_max_load(areas, cp)
        assert g >= opt
        assert g >= -(-sum(areas) // cp)
        if cp == 1 or n == cp:
            assert g == opt
    # equal areas: perfect balance
    assert dor.max_load([4] * 12, dor.greedy_dispatch([4] * 12, 4), 4) == 12


def _brute_max_load(areas, cp):
    """Min over every labelling of the chunks with cp buckets, each bucket
    taking n / cp chunks, of the heaviest bucket."""
    n, cap, best = len(areas), len(areas) // cp, None
    for lab in itertools.product(range(cp), repeat=n):
        if any(lab.count(b) != cap for b in range(cp)):
            continue
        m = max(sum(a for a, l in zip(areas, lab) if l == b) for b in range(cp))
        best = m if best is None else min(best, m)
    return best


def test_oracle_best_max_load_vs_brute_force():
    """The exhaustive search (recursive choice of each bucket's members) against
    a plain enumeration of labellings, plus a worked example: six chunks
    8, 7, 6, 5, 4, 3 into two buckets of three sum to 33, so the heavier bucket
    holds at least 17, and {8, 6, 3} / {7, 5, 4} reaches it."""
    assert dor.best_max_load([8, 7, 6, 5, 4, 3], 2) == 17
    rng = random.Random(11)
    for _ in range(80):
        cp = rng.choice([2, 3])
        n = cp * rng.choice([1, 2]) if cp == 3 else cp * rng.choice([1, 2, 3, 4])
        areas = [rng.randint(0, 30) for _ in range(n)]
        assert dor.best_max_load(areas, cp) == _brute_max_load(areas, cp), (areas, cp)


def test_oracle_best_max_load_pin_catches_dropped_count_rule(monkeypatch):
    """An exhaustive search that forgets the equal-count rule (any subset per
    bucket) reports a lower optimum on some input and fails the pin."""
    def unconstrained(areas, cp):
        return min(max(sum(a for a, l in zip(areas, lab) if l == b) for b in range(cp))
                   for lab in itertools.product(range(cp), repeat=len(areas)))
    monkeypatch.setattr(dor, "best_max_load", unconstrained)
    with pytest.raises(AssertionError):
        test_oracle_best_max_load_vs_brute_force()


@pytest.mark.parametrize("cp,chunk", [(2, 64), (4, 32), (8, 16)])
def test_oracle_greedy_balances_causal_exactly(cp, chunk):
    L = 2 * cp * chunk
    areas = dor.chunk_areas_rows([(0, L, 0, L, orc.CAUSAL)], L, chunk)
    b = dor.greedy_dispatch(areas, cp)
    assert dor.max_load(areas, b, cp) == sum(areas) // cp == L * (L + 1) // 2 // cp
    for c in range(2 * cp):
        assert b[c] == b[2 * cp - 1 - c]


def test_oracle_pins_catch_planted_mistake(monkeypatch):
    """Replacing the lightest-bucket rule by round robin breaks the causal pin."""
    def round_robin(areas, cp):
        order = sorted(range(len(areas)), key=lambda c: (-areas[c], c))
        out = [0] * len(areas)
        for k, c in enumerate(order):
            out[c] = k % cp
        return out
    monkeypatch.setattr(dor, "greedy_dispatch", round_robin)
    with pytest.raises(AssertionError):
        test_oracle_greedy_balances_causal_exactly(4, 32)


# --------------------------------------------------------------- library

def test_chunk_areas_match_oracle():
    for name, sl, Tq, Tk in _tables():
        for chunk in (64, 100, 512):
            got = ffa.chunk_areas(sl, Tq, Tk, chunk)
            assert got.tolist() == dor.chunk_areas_dense(sl, Tq, Tk, chunk), name


def test_chunk_areas_workloads_sum_to_mask_area():
    for idx in (2, 4, 5):
        for c in wl.workload(idx).calls:
            got = ffa.chunk_areas(c.slices, c.Tq, c.Tk, 4096)
            assert int(got.sum()) == orc.total_area(c.slices)
            assert got.tolist() == dor.chunk_areas_rows(c.slices, c.Tq, 4096)


def test_dispatch_matches_oracle_greedy():
    rng = random.Random(11)
    for _ in range(200):
        cp = rng.choice([1, 2, 4, 8])
        n = cp * rng.randint(1, 16)
        areas = [rng.choice([0, 3, 3, 7, rng.randint(0, 10 ** 12)]) for _ in range(n)]
        got = ffa.dispatch_chunks(areas, cp)
        assert got.tolist() == dor.greedy_dispatch(areas, cp)


def test_dispatch_varlen_causal_16k_balance():
    """16K varlen causal table, 1024-token chunks over 4 ranks: equal counts and
    the greedy's largest bucket within 5 % of the mean."""
    c = wl.workload(2).calls[0]
    areas = ffa.chunk_areas(c.slices, c.Tq, c.Tk, 1024)
    b = ffa.dispatch_chunks(areas, 4)
    loads = np.bincount(b, weights=areas, minlength=4)
    assert np.all(np.bincount(b, minlength=4) == 4)
    assert loads.max() <= 1.05 * areas.sum() / 4
    assert b.tolist() == dor.greedy_dispatch(areas.tolist(), 4)


def _check_share(sl, Tq, Tk, chunk, chunks):
    loc, kv, tk = ffa.rank_slices(sl, Tq, Tk, chunk, chunks)
    # received key ranges: sorted, disjoint, not adjacent, packed back to back
    off = 0
    for i, (a, b, o) in enumerate(kv.tolist()):
        assert 0 <= a < b <= Tk and o == off
        off += b - a
        if i:
            assert a > kv[i - 1][1]
    assert tk == off
    rows = dor.share_rows(Tq, chunk, chunks)
    keys = np.concatenate([np.arange(a, b) for a, b, _ in kv.tolist()]) if len(kv) else np.zeros(0, int)
    assert orc.validate([tuple(s) for s in loc.tolist()], len(rows), tk) == 0
    local = orc.dense_mask([tuple(s) for s in loc.tolist()], len(rows), tk) > 0
    assert np.array_equal(local, dor.share_mask(sl, Tq, Tk, rows, keys))
    # nothing outside the received keys is valid for these rows
    full = orc.dense_mask(sl, Tq, Tk)[rows] > 0
    assert int(full.sum()) == int(local.sum())
    return loc, kv, tk


def test_rank_slices_reproduce_the_global_mask():
    rng = random.Random(5)
    for name, sl, Tq, Tk in _tables():
        for chunk, cp in ((64, 2), (100, 3), (128, 4)):
            n = dor.num_chunks(Tq, chunk)
            chunks = list(range(n))
            rng.shuffle(chunks)
            for r in range(cp):
                _check_share(sl, Tq, Tk, chunk, chunks[r::cp])


def test_rank_slices_from_dispatch_cover_every_pair_once():
    """All ranks of a dispatch together hold every valid pair exactly once."""
    for name, sl, Tq, Tk in _tables():
        chunk, cp = 64, 2
        n = dor.num_chunks(Tq, chunk)
        n -= n % cp
        if n == 0:
            continue
        areas = ffa.chunk_areas(sl, Tq, Tk, chunk)[:n]
        b = ffa.dispatch_chunks(areas, cp)
        total = 0
        for r in range(cp):
            loc, kv, tk = _check_share(sl, Tq, Tk, chunk, [c for c in range(n) if b[c] == r])
            total += orc.total_area([tuple(s) for s in loc.tolist()])
        assert total == int(areas.sum())


def test_cp_share_workload_is_a_rank_share():
    """The 256K x 1M workload is the share of chunks 0, 4, 8, ... of the first
    half of its 2M-token block-causal table: rank_slices reproduces its slice
    table exactly once the receive-buffer key columns are mapped back to
    global keys (the workload keeps the whole first half as its key buffer;
    the share needs only part of it)."""
    import random as _r
    W = wl.workload(5)
    call = W.calls[0]
    N, block, chunk = 2_097_152, 4096, 4096
    lens = wl.trimmed_lengths(_r.Random(W.seed), N, 16384, 262144)
    glob, S = [], 0
    for L in lens:
        for bs in range(S, S + L, block):
            glob.append((bs, min(bs + block, S + L), S, min(bs + block, S + L), ffa.FULL))
        S += L
    chunks = list(range(0, N // 2 // chunk, 4))
    loc, kv, tk = ffa.rank_slices(glob, N, N, chunk, chunks)
    assert kv[-1][1] <= call.Tk and tk < call.Tk
    starts = kv[:, 2]
    back = []
    for q0, q1, k0, k1, t in loc.tolist():
        m = int(np.searchsorted(starts, k0, side="right")) - 1
        shift = int(kv[m][0] - kv[m][2])
        assert k1 <= kv[m][2] + kv[m][1] - kv[m][0]
        back.append((q0, q1, k0 + shift, k1 + shift, t))
    assert back == [tuple(s) for s in call.slices]


def test_rank_slices_errors_and_capacity():
    sl = [(0, 100, 0, 100, ffa.CAUSAL)]
    with pytest.raises(ffa.FFAError):
        ffa.rank_slices(sl, 100, 100, 50, [0, 0])            # repeated chunk
    with pytest.raises(ffa.FFAError):
        ffa.rank_slices(sl, 100, 100, 50, [2])               # out of range
    with pytest.raises(ffa.FFAError):
        ffa.rank_slices([(0, 100, 0, 101, 0)], 100, 100, 50, [0])   # key range out of bounds
    with pytest.raises(ffa.FFAError):
        ffa.chunk_areas([(0, 10, 0, 10, 4)], 100, 100, 50)   # unknown type
    with pytest.raises(ffa.FFAError):
        ffa.dispatch_chunks([1, 2, 3], 2)                    # 3 chunks over 2 buckets
    import ctypes
    L = ffa.lib()
    h = np.asarray(sl, dtype=np.int32)
    c = np.asarray([0, 1], dtype=np.int32)
    nl, nk = ctypes.c_int32(), ctypes.c_int32()
    out = np.full((1, 5), -7, dtype=np.int32)
    kv = np.full((1, 3), -7, dtype=np.int32)
    code = L.ffa_rank_slices(h.ctypes.data, 1, 100, 100, 50, c.ctypes.data, 2, out.ctypes.data, 1,
                             ctypes.byref(nl), kv.ctypes.data, 1, ctypes.byref(nk))
    assert code == 3 and nl.value == 2 and nk.value == 1 and (out == -7).all() and (kv == -7).all()
    # an empty share
    loc, kv, tk = ffa.rank_slices(sl, 100, 100, 50, [])
    assert len(loc) == 0 and len(kv) == 0 and tk == 0
