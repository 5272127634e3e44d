"""Plain oracle of the context-parallel dispatch (TEST INFRASTRUCTURE ONLY:
only tests use it; it shares no code with the library).

What it follows (MagiAttention blog deep-dive, section "Dispatch Solver"):
  * the sequence is cut into n = seqlen / chunk_size query chunks (chunk-count
    equation); each chunk C_i has an area Area(C_i), its valid mask pairs;
  * the chunks are put into cp_size buckets B_j with |B_j| = n / cp_size
    (constraint equation), aiming at min over assignments of the largest
    bucket area (objective equation);
  * the pages solve it greedily with a min-heap: estimate every chunk's area,
    then keep giving the heavier chunks to the bucket that is lightest so far.

Readings where the pages are silent (listed in the design notes): the last
chunk may be shorter than chunk_size; heavier-first means by decreasing area
with equal areas taken in chunk order; a full bucket (n / cp_size chunks)
takes no more chunks; among equally light buckets the lower index wins.

Shares (section "通信与重叠", GroupCast: a rank receives only the key ranges its
query slices touch): ``share_mask`` gives the global mask restricted to one
rank's queries and to the keys it would receive, the reference the library's
rank-local slice table must reproduce exactly.
"""
from __future__ import annotations

import heapq
import itertools
from typing import List, Sequence

import numpy as np

from oracle import ffa_oracle as orc


def num_chunks(seqlen: int, chunk: int) -> int:
    return -(-seqlen // chunk)


def chunk_areas_dense(slices: Sequence, Tq: int, Tk: int, chunk: int) -> List[int]:
    """Area of every chunk by counting the materialised mask (small inputs)."""
    m = orc.dense_mask(slices, Tq, Tk) > 0
    per_row = m.sum(axis=1)
    return [int(per_row[c * chunk:(c + 1) * chunk].sum()) for c in range(num_chunks(Tq, chunk))]


def chunk_areas_rows(slices: Sequence, Tq: int, chunk: int) -> List[int]:
    """Same, summing each row's valid-key interval lengths (larger inputs)."""
    out = [0] * num_chunks(Tq, chunk)
    for s in slices:
        rows = np.arange(s[0], s[1])
        if len(rows) == 0:
            continue
        lo, hi, ok = orc.row_intervals_vec(s, rows)
        ln = np.where(ok, hi - lo + 1, 0)
        for c in range(s[0] // chunk, num_chunks(Tq, chunk)):
            if c * chunk >= s[1]:
                break
            sel = (rows >= c * chunk) & (rows < (c + 1) * chunk)
            out[c] += int(ln[sel].sum())
    return out


def greedy_dispatch(areas: Sequence[int], cp: int) -> List[int]:
    """The pages' greedy: chunks heaviest first, each to the lightest bucket
    that still has room.  Returns the bucket of every chunk."""
    n = len(areas)
    assert n > 0 and n % cp == 0
    cap = n // cp
    order = sorted(range(n), key=lambda c: (-areas[c], c))
    heap = [(0, b) for b in range(cp)]
    count = [0] * cp
    bucket = [-1] * n
    for c in order:
        load, b = heapq.heappop(heap)
        bucket[c] = b
        count[b] += 1
        if count[b] < cap:
            heapq.heappush(heap, (load + areas[c], b))
    return bucket


def max_load(areas: Sequence[int], bucket: Sequence[int], cp: int) -> int:
    loads = [0] * cp
    for a, b in zip(areas, bucket):
        loads[b] += a
    return max(loads)


def best_max_load(areas: Sequence[int], cp: int) -> int:
    """Exact optimum of the min-max objective over every equal-count
    assignment, by exhaustive search (n up to about 10)."""
    n = len(areas)
    cap = n // cp
    best = [sum(areas)]

    def rec(rest: List[int], buckets_left: int, cur_max: int):
        if cur_max >= best[0]:
            return
        if buckets_left == 1:
            best[0] = min(best[0], max(cur_max, sum(areas[c] for c in rest)))
            return
        first, others = rest[0], rest[1:]
        for comb in itertools.combinations(others, cap - 1):
            grp = (first,) + comb
            load = sum(areas[c] for c in grp)
            left = [c for c in others if c not in comb]
            rec(left, buckets_left - 1, max(cur_max, load))

    rec(list(range(n)), cp, 0)
    return best[0]


def share_rows(Tq: int, chunk: int, chunks: Sequence[int]) -> np.ndarray:
    """Global query rows of a share, in local order (its chunks concatenated)."""
    return np.concatenate([np.arange(c * chunk, min((c + 1) * chunk, Tq)) for c in chunks]) \
        if len(chunks) else np.zeros(0, dtype=np.int64)


def share_mask(slices: Sequence, Tq: int, Tk: int, rows: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Global mask on (rows x keys), in the given orders."""
    m = orc.dense_mask(slices, Tq, Tk) > 0
    return m[np.ix_(rows, keys)]
