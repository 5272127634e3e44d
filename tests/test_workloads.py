"""Seeded workload generators: exact, in bounds, disjoint, and with the areas
the closed forms give (CPU only)."""
import random

import numpy as np
import pytest

from flexible_mask_attention_amd import workloads as wl
from oracle import ffa_oracle as orc


def test_tiny_variants_areas():
    # closed forms: CAUSAL L(L+1)/2 per sequence, FULL L^2
    assert orc.total_area(wl.tiny_varlen("causal").calls[0].slices) == 2080 + 528 + 4656 + 2080
    assert orc.total_area(wl.tiny_varlen("mixed").calls[0].slices) == 2080 + 1024 + 4656 + 4096
    assert orc.total_area(wl.tiny_varlen("two_full").calls[0].slices) == 2 * 128 * 128


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_workloads_valid_and_deterministic(idx):
    a, b = wl.workload(idx), wl.workload(idx)
    assert [c.slices for c in a.calls] == [c.slices for c in b.calls]
    for c in a.calls:
        assert orc.validate(c.slices, c.Tq, c.Tk) == 0
        assert c.Hq % c.Hkv == 0


def test_varlen_lengths_recipe():
    c = wl.varlen_causal_gqa().calls[0]
    lens = [s[1] - s[0] for s in c.slices]
    assert sum(lens) == 16384
    assert all(256 <= L <= 4096 for L in lens[:-1]) and 1 <= lens[-1] <= 4096
    assert all(s[4] == wl.CAUSAL and s[0] == s[2] and s[1] == s[3] for s in c.slices)


def test_block_causal_video_recipe():
    a, b = wl.block_causal_video().calls
    assert a.Tq == a.Tk == b.Tq == 131072 and a.head_offset == 0 and b.head_offset == 8
    # block-causal: the union over slices of a sample is the lower block triangle
    m = orc.dense_mask([s for s in a.slices if s[1] <= 8192], 8192, 8192)
    assert m.max() == 1
    # sliding window: query i sees exactly keys [max(start, i-4095), i]
    for s in b.slices:
        if s[4] == wl.BI_CAUSAL:
            i = s[0] + 5
            lo, hi = orc.row_interval(s, i)
            assert (lo, hi) == (i - 4095, i)


def test_cp_share_recipe():
    c = wl.cp_share().calls[0]
    assert (c.Tq, c.Tk) == (262144, 1048576)
    assert all(s[4] == wl.FULL for s in c.slices)
    covered = np.zeros(c.Tq, dtype=np.int64)
    for s in c.slices:
        covered[s[0]:s[1]] += 1
        assert s[3] <= c.Tk
    assert covered.min() == 1 and covered.max() == 1     # every local row in exactly one slice


def test_random_slices_disjoint():
    rng = random.Random(0)
    for _ in range(20):
        sl = wl.random_slices(rng, 300, 200, rng.randint(1, 8))
        assert orc.validate(sl, 300, 200) == 0


def test_tensor_generation_is_seeded():
    c = wl.tiny_varlen().calls[0]
    t1, t2 = wl.make_tensors(c, 1), wl.make_tensors(c, 1)
    for k in t1:
        assert t1[k].dtype.is_floating_point and (t1[k] == t2[k]).all()
    assert not (wl.make_tensors(c, 2)["q"] == t1["q"]).all()


def test_banded_tables_put_several_slices_on_one_row():
    """The banded generator gives valid, disjoint tables in which some query
    rows are covered by two or more slices."""
    for seed in range(20):
        rng = random.Random(seed)
        Tq, Tk = rng.randint(50, 900), rng.randint(50, 900)
        sl = wl.random_banded_slices(rng, Tq, Tk)
        assert orc.validate(sl, Tq, Tk) == 0
        cover = np.zeros(Tq, dtype=int)
        for q0, q1, k0, k1, t in sl:
            cover[q0:q1] += 1
        assert cover.max() >= 2
