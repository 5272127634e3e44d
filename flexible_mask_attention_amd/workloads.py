"""Seeded synthetic workloads for Flex-Flash-Attention: slice tables and tensors.

This module only *builds inputs*.  It holds none of the method's arithmetic
(no mask predicate, no areas, no attention), so that the CPU oracle and the
HIP path can both be fed from it without sharing any computation.

A slice is ``(q_start, q_end, k_start, k_end, mask_type)`` with half-open token
ranges, the AttnSlice of the MagiAttention blog ("Flex-Flash-Attention 与
AttnSlice": a contiguous 2-D QK sub-mask plus a mask type).  Mask-type codes are
the library's ABI values: FULL=0, CAUSAL=1, INV_CAUSAL=2, BI_CAUSAL=3.

The pages draw varlen lengths from a private training-data length distribution
(blog, "训练和 Benchmark 设置": shuffled real lengths, packed, each sample at most
a quarter of the total).  That data is not available, so uniform integer draws
stand in for it; every recipe below is seeded and exact.
"""
from __future__ import annotations

import random
from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import torch

FULL, CAUSAL, INV_CAUSAL, BI_CAUSAL = 0, 1, 2, 3

Slice = Tuple[int, int, int, int, int]


@dataclass
class Call:
    """One library call: a slice table over one (q, k, v) tensor set."""
    slices: List[Slice]
    Tq: int
    Tk: int
    Hq: int
    Hkv: int
    d: int
    head_offset: int = 0   # which heads of the workload this call covers


@dataclass
class Workload:
    name: str
    seed: int
    calls: List[Call] = field(default_factory=list)


def trimmed_lengths(rng: random.Random, total: int, lo: int, hi: int) -> List[int]:
    """Draw integer lengths uniform in [lo, hi] until they reach ``total``; cut the
    last one so the sum is exactly ``total`` (it may end up shorter than ``lo``)."""
    out: List[int] = []
    acc = 0
    while acc < total:
        x = rng.randint(lo, hi)
        if acc + x > total:
            x = total - acc
        out.append(x)
        acc += x
    return out


def varlen_slices(lengths: Sequence[int], mask_type: int) -> List[Slice]:
    out, s = [], 0
    for L in lengths:
        out.append((s, s + L, s, s + L, mask_type))
        s += L
    return out


def tiny_varlen(variant: str = "causal") -> Workload:
    """256 tokens as sequences [64, 32, 96, 64], Hq=Hkv=2, d=64.

    variants: "causal" (4 CAUSAL slices), "mixed" (the 32- and 64-token
    sequences at positions 1 and 3 FULL instead), "two_full" ([0,128)^2 and
    [128,256)^2 FULL)."""
    lens = [64, 32, 96, 64]
    if variant == "causal":
        sl = varlen_slices(lens, CAUSAL)
    elif variant == "mixed":
        sl = varlen_slices(lens, CAUSAL)
        sl = [(a, b, c, d_, FULL if i in (1, 3) else t) for i, (a, b, c, d_, t) in enumerate(sl)]
    elif variant == "two_full":
        sl = [(0, 128, 0, 128, FULL), (128, 256, 128, 256, FULL)]
    else:
        raise ValueError(variant)
    return Workload(f"tiny_varlen_{variant}", 1, [Call(sl, 256, 256, 2, 2, 64)])


def varlen_causal_gqa(seed: int = 2) -> Workload:
    """16384 tokens, lengths U[256,4096] trimmed to the total, one CAUSAL slice
    per sequence, Hq=32, Hkv=8, d=128."""
    lens = trimmed_lengths(random.Random(seed), 16384, 256, 4096)
    return Workload("varlen_causal_gqa_16k", seed,
                    [Call(varlen_slices(lens, CAUSAL), 16384, 16384, 32, 8, 128)])


def dense_full(seed: int = 3) -> Workload:
    """One 65536-token sequence as a single FULL slice, Hq=Hkv=16, d=128."""
    T = 65536
    return Workload("dense_full_64k", seed, [Call([(0, T, 0, T, FULL)], T, T, 16, 16, 128)])


def block_causal_video(seed: int = 4, block: int = 2048, window: int = 4096) -> Workload:
    """131072 tokens as 8 samples whose lengths are multiples of ``block``.

    Heads 0-7: within each sample, block b attends to blocks 0..b (one FULL slice
    per block).  Heads 8-15: a causal sliding window of ``window`` tokens, as one
    CAUSAL slice for the first ``window`` tokens of a sample and one BI_CAUSAL
    slice for the rest (query i sees keys [i-window+1, i], clipped at the sample
    start).  The two head groups are two calls with their own tensors."""
    T = 131072
    units = T // block
    rng = random.Random(seed)
    cuts = sorted(rng.sample(range(1, units), 7))
    bounds = [0] + [c * block for c in cuts] + [T]
    a_sl: List[Slice] = []
    b_sl: List[Slice] = []
    for s, e in zip(bounds[:-1], bounds[1:]):
        for b in range((e - s) // block):
            a_sl.append((s + block * b, s + block * (b + 1), s, s + block * (b + 1), FULL))
        if e - s <= window:
            b_sl.append((s, e, s, e, CAUSAL))
        else:
            b_sl.append((s, s + window, s, s + window, CAUSAL))
            b_sl.append((s + window, e, s + 1, e, BI_CAUSAL))
    return Workload("block_causal_video_128k", seed,
                    [Call(a_sl, T, T, 8, 8, 128, head_offset=0),
                     Call(b_sl, T, T, 8, 8, 128, head_offset=8)])


def cp_share(seed: int = 5, block: int = 4096, chunk: int = 4096) -> Workload:
    """One rank's share of a 2M-token varlen block-causal mask.

    Global lengths U[16384, 262144] trimmed to 2,097,152.  Block-causal with
    ``block``-token blocks counted from each sample start (last block may be
    short).  K/V = global tokens [0, 1048576).  Local Q = the 4096-token chunks
    c = 0, 4, 8, ... of that first half (64 chunks), concatenated in order.  One
    FULL slice per (chunk, sample, block) intersection; q ranges are local rows,
    k ranges global token indices (== K/V buffer rows)."""
    N = 2_097_152
    half = N // 2
    lens = trimmed_lengths(random.Random(seed), N, 16384, 262144)
    starts = [0]
    for L in lens:
        starts.append(starts[-1] + L)
    sl: List[Slice] = []
    nchunks = half // chunk
    for c in range(0, nchunks, 4):
        c0, c1 = c * chunk, (c + 1) * chunk
        local0 = (c // 4) * chunk
        for si in range(len(lens)):
            S, E = starts[si], starts[si + 1]
            if E <= c0 or S >= c1:
                continue
            b_first = (max(S, c0) - S) // block
            b_last = (min(E, c1) - 1 - S) // block
            for b in range(b_first, b_last + 1):
                bs, be = S + b * block, min(S + (b + 1) * block, E)
                a, z = max(bs, c0), min(be, c1)
                if a < z:
                    sl.append((a - c0 + local0, z - c0 + local0, S, be, FULL))
    return Workload("cp_share_256k_x_1m", seed, [Call(sl, half // 4, half, 8, 8, 128)])


WORKLOADS = {
    1: tiny_varlen,
    2: varlen_causal_gqa,
    3: dense_full,
    4: block_causal_video,
    5: cp_share,
}


def workload(idx: int, **kw) -> Workload:
    return WORKLOADS[idx](**kw)


def randn_bf16(shape, gen: torch.Generator, chunk: int = 1 << 24) -> torch.Tensor:
    """fp32 N(0,1) drawn from ``gen`` in chunks of ``chunk`` elements, rounded to bf16."""
    n = 1
    for s in shape:
        n *= s
    out = torch.empty(n, dtype=torch.bfloat16)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        out[a:b] = torch.randn(b - a, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    return out.view(*shape)


def make_tensors(call: Call, seed: int, names=("q", "k", "v", "do")) -> dict:
    """Seeded CPU bf16 tensors in token-major layout: q, do [Tq, Hq, d]; k, v [Tk, Hkv, d].
    Drawn in the fixed order q, k, v, do from one generator seeded with ``seed``."""
    gen = torch.Generator().manual_seed(seed)
    shapes = {"q": (call.Tq, call.Hq, call.d), "k": (call.Tk, call.Hkv, call.d),
              "v": (call.Tk, call.Hkv, call.d), "do": (call.Tq, call.Hq, call.d)}
    out = {}
    for nm in ("q", "k", "v", "do"):
        t = randn_bf16(shapes[nm], gen)
        if nm in names:
            out[nm] = t
    return out


def random_slices(rng: random.Random, Tq: int, Tk: int, n: int, types=(0, 1, 2, 3),
                  max_len: int = 0) -> List[Slice]:
    """Random *disjoint* slice table: slices take disjoint q ranges (so their
    valid sets cannot overlap); k ranges are arbitrary.  Used for small parity
    cases with every mask type, Lq != Lk and ragged tails."""
    cuts = sorted(rng.sample(range(1, Tq), min(n - 1, Tq - 1))) if n > 1 else []
    bounds = [0] + cuts + [Tq]
    out: List[Slice] = []
    for q0, q1 in zip(bounds[:-1], bounds[1:]):
        if max_len and q1 - q0 > max_len:
            q1 = q0 + max_len
        k0 = rng.randint(0, Tk - 1)
        k1 = rng.randint(k0 + 1, Tk)
        out.append((q0, q1, k0, k1, rng.choice(types)))
    return out


def random_banded_slices(rng: random.Random, Tq: int, Tk: int, bands: int = 3,
                         per_band=(2, 4), types=(0, 1, 2, 3)) -> List[Slice]:
    """Random *disjoint* slice table with several slices on one query row: the
    query axis is cut into ``bands`` bands, and each band gets 2-4 slices with
    pairwise disjoint key ranges (so their valid sets cannot overlap) and
    random types, each over a random sub-range of the band's queries.  A row
    then attends to the union of several slices' keys, which the kernels
    combine bit by bit per tile."""
    cuts = sorted(rng.sample(range(1, Tq), min(bands - 1, Tq - 1))) if bands > 1 else []
    bounds = [0] + cuts + [Tq]
    out: List[Slice] = []
    for q0, q1 in zip(bounds[:-1], bounds[1:]):
        n = rng.randint(per_band[0], per_band[1])
        n = min(n, Tk // 2)
        if n < 1:
            continue
        pts = sorted(rng.sample(range(0, Tk + 1), 2 * n))
        for i in range(n):
            a, z = rng.randint(q0, q1 - 1), rng.randint(q0 + 1, q1)
            qa, qz = min(a, z - 1), max(a + 1, z)
            out.append((qa, qz, pts[2 * i], pts[2 * i + 1], rng.choice(types)))
    return out
