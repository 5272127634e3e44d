"""Plain fp64 CPU oracle for Flex-Flash-Attention (FFA) over AttnSlices.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use
it.  It shares no code with the HIP path.

What it follows (MagiAttention pages):
  * AttnSlice = (QRange, KRange, MaskType), a contiguous 2-D QK sub-mask; mask
    types FULL, CAUSAL, INV-CAUSAL, BI-CAUSAL are named but not defined (blog
    deep-dive, section "Flex-Flash-Attention 与 AttnSlice", AttnSlice equation).
  * Mask semantics fixed by the build contract: CAUSAL is bottom-right aligned,
    INV-CAUSAL top-left aligned, BI-CAUSAL their intersection; slices disjoint;
    an empty row gives O = 0 and LSE = -inf.
  * MaskArea: full = L^2, causal = L(L+1)/2, and FLOPs_fwd = 2*2*area*b*Hq*d,
    FLOPs_bwd = 2.5*FLOPs_fwd (blog deep-dive, section "训练和 Benchmark 设置",
    FLOPs equation and the area sentence after it).
  * Block classes Full / Partial / Empty, q2k for forward and k2q for backward,
    blocks out of bounds only in q counted as Full, CSR offsets
    full_block_offset / mask_block_offset (documentation page, "FFA_FA4"
    optimisations list, items 1 and 2).

Readings where the pages are silent (each listed in the design notes):
  ranges half-open; softmax scale default 1/sqrt(d); natural-log LSE including
  the scale; GQA head h uses kv head h // (Hq/Hkv); k2q mirrors the q2k
  out-of-bounds rule with the axes swapped; CSR lists ascending, Full and
  Partial kept apart.

Everything is float64 (bf16 inputs upcast exactly), written with numpy and plain
PyTorch CPU ops (library matmul, exp, log).  The forward is two-pass
(LSE first, then O), unlike the GPU's online softmax.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

FULL, CAUSAL, INV_CAUSAL, BI_CAUSAL = 0, 1, 2, 3

# status flags for a slice table (bitwise OR, same meaning as the library's
# device status word)
ERR_BOUNDS, ERR_TYPE, ERR_OVERLAP = 1, 2, 4


# ---------------------------------------------------------------------------
# c.2  the mask predicate (definition) and the row / column interval forms
# ---------------------------------------------------------------------------

def valid(i: int, j: int, s) -> bool:
    """Is (query i, key j) in slice s?  The defining predicate.

    r = i - q0, c = j - k0, Lq = q1 - q0, Lk = k1 - k0;
      FULL:        inside the rectangle
      CAUSAL:      c <= r + (Lk - Lq)     (bottom-right aligned diagonal)
      INV_CAUSAL:  c >= r                 (top-left aligned diagonal)
      BI_CAUSAL:   both
    """
    q0, q1, k0, k1, t = s
    if not (q0 <= i < q1 and k0 <= j < k1):
        return False
    r, c, Lq, Lk = i - q0, j - k0, q1 - q0, k1 - k0
    if t == FULL:
        return True
    if t == CAUSAL:
        return c <= r + (Lk - Lq)
    if t == INV_CAUSAL:
        return c >= r
    if t == BI_CAUSAL:
        return c <= r + (Lk - Lq) and c >= r
    raise ValueError(f"unknown mask type {t}")


def dense_mask(slices: Sequence, Tq: int, Tk: int) -> np.ndarray:
    """Materialised [Tq, Tk] int count of slices containing each (i, j), from the
    predicate evaluated on the whole grid (brute force; small inputs only).
    Disjoint tables give a 0/1 array."""
    ii = np.arange(Tq)[:, None]
    jj = np.arange(Tk)[None, :]
    cnt = np.zeros((Tq, Tk), dtype=np.int64)
    for (q0, q1, k0, k1, t) in slices:
        inside = (ii >= q0) & (ii < q1) & (jj >= k0) & (jj < k1)
        r, c, Lq, Lk = ii - q0, jj - k0, q1 - q0, k1 - k0
        if t == FULL:
            m = inside
        elif t == CAUSAL:
            m = inside & (c <= r + (Lk - Lq))
        elif t == INV_CAUSAL:
            m = inside & (c >= r)
        elif t == BI_CAUSAL:
            m = inside & (c <= r + (Lk - Lq)) & (c >= r)
        else:
            raise ValueError(t)
        cnt += m
    return cnt


def row_interval(s, i: int):
    """Keys valid for query i in slice s as an inclusive interval (lo, hi), or
    None.  Solving the predicate for c at fixed r gives
    c in [ (r if type in {INV,BI} else 0),  (min(Lk-1, r+Lk-Lq) if type in {CAUSAL,BI} else Lk-1) ]."""
    q0, q1, k0, k1, t = s
    if not (q0 <= i < q1) or k1 <= k0:
        return None
    r, Lq, Lk = i - q0, q1 - q0, k1 - k0
    lo = r if t in (INV_CAUSAL, BI_CAUSAL) else 0
    hi = min(Lk - 1, r + Lk - Lq) if t in (CAUSAL, BI_CAUSAL) else Lk - 1
    if lo > hi:
        return None
    return (k0 + lo, k0 + hi)


def col_interval(s, j: int):
    """Queries valid for key j in slice s as an inclusive interval, or None.
    Solving the predicate for r at fixed c: CAUSAL needs r >= c - (Lk-Lq),
    INV_CAUSAL needs r <= c."""
    q0, q1, k0, k1, t = s
    if not (k0 <= j < k1) or q1 <= q0:
        return None
    c, Lq, Lk = j - k0, q1 - q0, k1 - k0
    lo = max(0, c - (Lk - Lq)) if t in (CAUSAL, BI_CAUSAL) else 0
    hi = min(Lq - 1, c) if t in (INV_CAUSAL, BI_CAUSAL) else Lq - 1
    if lo > hi:
        return None
    return (q0 + lo, q0 + hi)


def row_intervals_vec(s, rows: np.ndarray):
    """Vectorised ``row_interval`` over an int array of rows: (lo, hi, ok)."""
    q0, q1, k0, k1, t = s
    rows = np.asarray(rows, dtype=np.int64)
    r, Lq, Lk = rows - q0, q1 - q0, k1 - k0
    lo = r if t in (INV_CAUSAL, BI_CAUSAL) else np.zeros_like(r)
    hi = np.minimum(Lk - 1, r + Lk - Lq) if t in (CAUSAL, BI_CAUSAL) else np.full_like(r, Lk - 1)
    ok = (rows >= q0) & (rows < q1) & (lo <= hi) & (Lk > 0)
    return k0 + lo, k0 + hi, ok


def col_intervals_vec(s, cols: np.ndarray):
    """Vectorised ``col_interval`` over an int array of keys: (lo, hi, ok)."""
    q0, q1, k0, k1, t = s
    cols = np.asarray(cols, dtype=np.int64)
    c, Lq, Lk = cols - k0, q1 - q0, k1 - k0
    lo = np.maximum(0, c - (Lk - Lq)) if t in (CAUSAL, BI_CAUSAL) else np.zeros_like(c)
    hi = np.minimum(Lq - 1, c) if t in (INV_CAUSAL, BI_CAUSAL) else np.full_like(c, Lq - 1)
    ok = (cols >= k0) & (cols < k1) & (lo <= hi) & (Lq > 0)
    return q0 + lo, q0 + hi, ok


def valid_keys(slices: Sequence, i: int) -> np.ndarray:
    """Sorted array J_i of keys valid for query i (union over slices)."""
    parts = []
    for s in slices:
        iv = row_interval(s, i)
        if iv is not None:
            parts.append(np.arange(iv[0], iv[1] + 1))
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.concatenate(parts))


# ---------------------------------------------------------------------------
# c.3  areas and FLOPs
# ---------------------------------------------------------------------------

def slice_area(s) -> int:
    """Number of valid (i, j) in one slice, closed form per mask type.

    FULL: Lq*Lk.  CAUSAL and INV_CAUSAL: Lq*Lk - Lq(Lq-1)/2 if Lk >= Lq, else
    Lk(Lk+1)/2.  BI_CAUSAL: Lq(Lk-Lq+1) if Lk >= Lq, else 0.  With Lq = Lk = L
    these are the pages' L^2 and L(L+1)/2."""
    q0, q1, k0, k1, t = s
    Lq, Lk = max(0, q1 - q0), max(0, k1 - k0)
    if Lq == 0 or Lk == 0:
        return 0
    if t == FULL:
        return Lq * Lk
    if t in (CAUSAL, INV_CAUSAL):
        return Lq * Lk - Lq * (Lq - 1) // 2 if Lk >= Lq else Lk * (Lk + 1) // 2
    if t == BI_CAUSAL:
        return Lq * (Lk - Lq + 1) if Lk >= Lq else 0
    raise ValueError(t)


def total_area(slices: Sequence) -> int:
    """Valid-mask area of a disjoint slice table: the sum of slice areas."""
    return sum(slice_area(s) for s in slices)


def flops(area: int, num_heads_q: int, head_dim: int, batch: int = 1) -> Tuple[int, float]:
    """(FLOPs_fwd, FLOPs_bwd) = (2*2*area*batch*Hq*d, 2.5 * FLOPs_fwd)."""
    f = 2 * 2 * area * batch * num_heads_q * head_dim
    return f, 2.5 * f


# ---------------------------------------------------------------------------
# slice-table validation
# ---------------------------------------------------------------------------

def validate(slices: Sequence, Tq: int, Tk: int) -> int:
    """Bit flags: ERR_BOUNDS (a range outside [0,T] or start > end), ERR_TYPE
    (mask type not 0..3), ERR_OVERLAP (two slices share a valid (i, j))."""
    flags = 0
    good = []
    for s in slices:
        q0, q1, k0, k1, t = s
        if not (0 <= q0 <= q1 <= Tq and 0 <= k0 <= k1 <= Tk):
            flags |= ERR_BOUNDS
            continue
        if t not in (FULL, CAUSAL, INV_CAUSAL, BI_CAUSAL):
            flags |= ERR_TYPE
            continue
        good.append(s)
    # overlap: some row has intersecting intervals from two slices.  Two
    # slices whose query ranges or key ranges do not intersect share no pair;
    # that test is done for all later slices at once, and only the pairs
    # passing it are compared row by row.
    G = np.asarray(good, dtype=np.int64).reshape(-1, 5)
    for a in range(len(good)):
        sa = good[a]
        rest = G[a + 1:]
        cand = np.nonzero((np.maximum(rest[:, 0], sa[0]) < np.minimum(rest[:, 1], sa[1])) &
                          (np.maximum(rest[:, 2], sa[2]) < np.minimum(rest[:, 3], sa[3])))[0]
        for c in cand:
            sb = good[a + 1 + int(c)]
            rows = np.arange(max(sa[0], sb[0]), min(sa[1], sb[1]))
            la, ha, oka = row_intervals_vec(sa, rows)
            lb, hb, okb = row_intervals_vec(sb, rows)
            if np.any(oka & okb & (np.maximum(la, lb) <= np.minimum(ha, hb))):
                return flags | ERR_OVERLAP
    return flags


# ---------------------------------------------------------------------------
# c.6  block metadata
# ---------------------------------------------------------------------------

def tile_counts_dense(slices: Sequence, Tq: int, Tk: int, BM: int, BN: int) -> np.ndarray:
    """v[m, n] = number of valid (i, j) in tile rows [m*BM, (m+1)*BM) x cols
    [n*BN, (n+1)*BN), counted on the materialised mask (brute force)."""
    mask = dense_mask(slices, Tq, Tk)
    nm, nn = -(-Tq // BM), -(-Tk // BN)
    pad = np.zeros((nm * BM, nn * BN), dtype=np.int64)
    pad[:Tq, :Tk] = mask
    return pad.reshape(nm, BM, nn, BN).sum(axis=(1, 3))


def tile_counts(slices: Sequence, Tq: int, Tk: int, BM: int, BN: int) -> Dict[int, np.ndarray]:
    """Same counts without materialising the mask, for large tables.

    For one q-block, every valid pair lies in some row's interval.  Let
    H(x) = number of valid pairs in the block with key < x
         = sum over intervals [lo, hi] of clip(x - lo, 0, hi - lo + 1).
    Then v[m, n] = H((n+1)*BN) - H(n*BN).  Returns {m: int64 array over n} for
    q-blocks that contain any valid pair."""
    nm, nn = -(-Tq // BM), -(-Tk // BN)
    per_block: Dict[int, List[Tuple[np.ndarray, np.ndarray]]] = {}
    for s in slices:
        q0, q1 = s[0], s[1]
        if q1 <= q0:
            continue
        for m in range(q0 // BM, (q1 - 1) // BM + 1):
            rows = np.arange(max(q0, m * BM), min(q1, (m + 1) * BM))
            lo, hi, ok = row_intervals_vec(s, rows)
            if ok.any():
                per_block.setdefault(m, []).append((lo[ok], hi[ok]))
    out: Dict[int, np.ndarray] = {}
    grid = np.arange(nn + 1, dtype=np.int64) * BN
    for m, parts in per_block.items():
        lo = np.concatenate([p[0] for p in parts])
        hi = np.concatenate([p[1] for p in parts])
        ln = hi - lo + 1
        # H(x) = sum_{lo < x} (x - lo) - sum_{hi+1 < x} (x - hi - 1)
        order_lo = np.sort(lo)
        order_end = np.sort(hi + 1)
        c_lo = np.concatenate([[0], np.cumsum(order_lo)])
        c_end = np.concatenate([[0], np.cumsum(order_end)])
        n_lo = np.searchsorted(order_lo, grid, side="left")     # lo < x
        n_end = np.searchsorted(order_end, grid, side="left")   # hi+1 < x
        H = (n_lo * grid - c_lo[n_lo]) - (n_end * grid - c_end[n_end])
        v = np.diff(H)
        assert v.sum() == ln.sum()
        out[m] = v
    return out


def block_meta(slices: Sequence, Tq: int, Tk: int, BM: int, BN: int, direction: str,
               dense: bool = False) -> dict:
    """CSR block metadata.

    Tiles are rows [m*BM, (m+1)*BM) x cols [n*BN, (n+1)*BN); v = valid count.
      q2k (forward):  rows past Tq are ignored; cols past Tk count as invalid.
                      Full iff v == rows_in_bounds(m) * BN.
      k2q (backward): mirror - cols past Tk ignored, rows past Tq invalid.
                      Full iff v == BM * cols_in_bounds(n).
      Empty iff v == 0, else Partial.
    q2k lists, per q-block m, ascending k-block indices; k2q lists, per k-block
    n, ascending q-block indices.  Returns full_block_offset, full_block_idx,
    mask_block_offset, mask_block_idx (int64 arrays) and the total area."""
    nm, nn = -(-Tq // BM), -(-Tk // BN)
    if dense:
        V = tile_counts_dense(slices, Tq, Tk, BM, BN)
        rows_v = {m: V[m] for m in range(nm) if V[m].any()}
    else:
        rows_v = tile_counts(slices, Tq, Tk, BM, BN)
    area = int(sum(int(v.sum()) for v in rows_v.values()))
    if direction == "q2k":
        full_lists: List[List[int]] = [[] for _ in range(nm)]
        mask_lists: List[List[int]] = [[] for _ in range(nm)]
        for m, v in rows_v.items():
            cap = (min((m + 1) * BM, Tq) - m * BM) * BN
            nz = np.nonzero(v)[0]
            full_lists[m] = [int(n) for n in nz if v[n] == cap]
            mask_lists[m] = [int(n) for n in nz if v[n] != cap]
    elif direction == "k2q":
        full_lists = [[] for _ in range(nn)]
        mask_lists = [[] for _ in range(nn)]
        for m in sorted(rows_v):
            v = rows_v[m]
            for n in np.nonzero(v)[0]:
                cap = BM * (min((n + 1) * BN, Tk) - n * BN)
                (full_lists if v[n] == cap else mask_lists)[int(n)].append(m)
    else:
        raise ValueError(direction)

    def csr(lists):
        off = np.zeros(len(lists) + 1, dtype=np.int64)
        off[1:] = np.cumsum([len(x) for x in lists])
        idx = np.array([i for x in lists for i in x], dtype=np.int64)
        return off, idx

    fo, fi = csr(full_lists)
    mo, mi = csr(mask_lists)
    return {"full_block_offset": fo, "full_block_idx": fi,
            "mask_block_offset": mo, "mask_block_idx": mi, "area": area}


# ---------------------------------------------------------------------------
# c.4 / c.5  attention forward and backward
# ---------------------------------------------------------------------------

def _row_batches(rows: np.ndarray, slices: Sequence, max_elems: int, max_rows: int = 256):
    """Split sorted rows into batches; for each batch give the key window
    [w0, w1) that contains every valid key of every row in it and the (rows x
    window) validity mask built from the row intervals.  Rows are independent
    and keys outside the window are invalid for all rows of the batch, so
    attention over the window equals attention over all keys.  A batch ends
    after max_rows rows, when rows x window would pass max_elems, or where the
    next row's keys do not touch the current window."""
    lo_all = np.full(len(rows), np.iinfo(np.int64).max, dtype=np.int64)
    hi_all = np.full(len(rows), -1, dtype=np.int64)
    ivs = []
    for s in slices:
        lo, hi, ok = row_intervals_vec(s, rows)
        if ok.any():
            ivs.append((lo, hi, ok))
            lo_all = np.where(ok, np.minimum(lo_all, lo), lo_all)
            hi_all = np.where(ok, np.maximum(hi_all, hi), hi_all)
    a = 0
    n = len(rows)
    while a < n:
        b = a + 1
        w0 = lo_all[a] if hi_all[a] >= 0 else 0
        w1 = hi_all[a] + 1 if hi_all[a] >= 0 else 0
        while b < n and b - a < max_rows:
            if hi_all[b] < 0:
                nw0, nw1 = w0, w1
            elif w1 <= w0:
                nw0, nw1 = lo_all[b], hi_all[b] + 1
            else:
                if lo_all[b] > w1 or hi_all[b] + 1 < w0:
                    break
                nw0, nw1 = min(w0, lo_all[b]), max(w1, hi_all[b] + 1)
            if (b + 1 - a) * max(1, nw1 - nw0) > max_elems:
                break
            w0, w1 = nw0, nw1
            b += 1
        w0, w1 = int(w0), int(max(w0, w1))
        mask = np.zeros((b - a, w1 - w0), dtype=bool)
        for lo, hi, ok in ivs:
            for r in np.nonzero(ok[a:b])[0]:
                mask[r, lo[a + r] - w0:hi[a + r] + 1 - w0] = True
        yield a, b, w0, w1, mask
        a = b


def _f64(x) -> "torch.Tensor":
    """torch tensor / ndarray -> contiguous float64 CPU torch tensor (exact upcast)."""
    import torch
    if isinstance(x, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    x = x.detach().to("cpu")
    if x.dtype == torch.bfloat16:
        x = x.to(torch.float32)
    return x.to(torch.float64).contiguous()


def _softmax_stats(S):
    """Two-pass masked softmax over the last axis of S (masked entries are -inf):
    pass 1 gives LSE = m + ln sum exp(S - m), pass 2 gives P = exp(S - LSE)
    (formed as exp(S - m) / sum).  Rows without a valid entry get LSE = -inf
    and P = 0."""
    import torch
    m = S.amax(dim=-1, keepdim=True)
    m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
    E = torch.exp(S - m)
    z = E.sum(dim=-1, keepdim=True)
    lse = m + torch.log(z)                                                    # pass 1
    P = E.div_(torch.where(z > 0, z, torch.ones_like(z)))                     # pass 2
    return lse, P


def _attend(Qb, Kg, Vg, mask, scale):
    """One row batch of one kv-head group: Qb [B, G, d], Kg/Vg [W, d] (the
    batch's key window), mask [B, W] bool.  Returns S-derived (lse, P) and O."""
    B, G, d = Qb.shape
    S = scale * (Qb.reshape(B * G, d) @ Kg.T).view(B, G, -1)
    S.masked_fill_(~mask[:, None, :], -math.inf)
    lse, P = _softmax_stats(S)
    O = (P.reshape(B * G, -1) @ Vg).view(B, G, d)
    return lse[..., 0], P, O


def forward(q, k, v, slices: Sequence, scale: float = None, rows=None,
            max_elems: int = 1 << 25):
    """O and LSE for the given query rows (default: all).

    For each head h and row i with valid key set J_i:
      s_ij = scale * q_i . k_j;  LSE_i = ln sum_{j in J_i} exp(s_ij)  (via max);
      O_i = sum_{j in J_i} exp(s_ij - LSE_i) v_j;
      J_i empty -> O_i = 0, LSE_i = -inf.
    Query head h uses kv head h // (Hq / Hkv).
    Returns O [len(rows), Hq, d] and LSE [Hq, len(rows)] (float64 ndarrays)."""
    import torch
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    rows_t = torch.from_numpy(rows)
    batches = list(_row_batches(rows, slices, max(1, max_elems // G)))
    O = torch.zeros(len(rows), Hq, d, dtype=torch.float64)
    L = torch.full((Hq, len(rows)), -math.inf, dtype=torch.float64)
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        for a, b, w0, w1, mask in batches:
            if w1 <= w0:
                continue
            Qb = _f64(q[rows_t[a:b], hs, :])
            Kw, Vw = _f64(k[w0:w1, g, :]), _f64(v[w0:w1, g, :])
            lse, _, Ob = _attend(Qb, Kw, Vw, torch.from_numpy(mask), scale)
            O[a:b, hs, :] = Ob
            L[hs, a:b] = lse.T
    return O.numpy(), L.numpy()


def backward(q, k, v, do, slices: Sequence, scale: float = None, max_elems: int = 1 << 25):
    """dQ, dK, dV (float64 ndarrays), the textbook gradient of ``forward``.

      P_ij = exp(s_ij - LSE_i) on J_i (0 elsewhere);  D_i = dO_i . O_i;
      dS_ij = P_ij (dO_i . v_j - D_i);
      dQ_i = scale sum_j dS_ij k_j;  dK_j = scale sum_{h in group} sum_i dS_ij q_i;
      dV_j = sum_{h in group} sum_i P_ij dO_i.
    O and LSE are recomputed here in float64."""
    import torch
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(Tq)
    batches = list(_row_batches(rows, slices, max(1, max_elems // G)))
    dq = torch.zeros(Tq, Hq, d, dtype=torch.float64)
    dk = torch.zeros(Tk, Hkv, d, dtype=torch.float64)
    dv = torch.zeros(Tk, Hkv, d, dtype=torch.float64)
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        dKg = torch.zeros(Tk, d, dtype=torch.float64)
        dVg = torch.zeros(Tk, d, dtype=torch.float64)
        for a, b, w0, w1, mask in batches:
            if w1 <= w0:
                continue
            Qb, dOb = _f64(q[a:b, hs, :]), _f64(do[a:b, hs, :])
            Kw, Vw = _f64(k[w0:w1, g, :]), _f64(v[w0:w1, g, :])
            _, P, Ob = _attend(Qb, Kw, Vw, torch.from_numpy(mask), scale)
            B = b - a
            D = (dOb * Ob).sum(dim=-1, keepdim=True)                        # [B, G, 1]
            dP = (dOb.reshape(B * G, d) @ Vw.T).view(B, G, -1)
            dS = P * (dP - D)
            dq[a:b, hs, :] = scale * (dS.reshape(B * G, -1) @ Kw).view(B, G, d)
            dKg[w0:w1] += scale * (dS.reshape(B * G, -1).T @ Qb.reshape(B * G, d))
            dVg[w0:w1] += P.reshape(B * G, -1).T @ dOb.reshape(B * G, d)
        dk[:, g, :] = dKg
        dv[:, g, :] = dVg
    return dq.numpy(), dk.numpy(), dv.numpy()


def forward_backward_rows(q, k, v, do, slices: Sequence, rows, scale: float = None,
                          max_elems: int = 1 << 25):
    """O, LSE and dQ for the given rows only, in one pass (each row needs only
    its own valid keys, O_i and LSE_i).  Returns O [n, Hq, d], LSE [Hq, n],
    dQ [n, Hq, d] as float64 ndarrays."""
    import torch
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    rows_t = torch.from_numpy(rows)
    batches = list(_row_batches(rows, slices, max(1, max_elems // G)))
    O = torch.zeros(len(rows), Hq, d, dtype=torch.float64)
    L = torch.full((Hq, len(rows)), -math.inf, dtype=torch.float64)
    dQ = torch.zeros(len(rows), Hq, d, dtype=torch.float64)
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        for a, b, w0, w1, mask in batches:
            if w1 <= w0:
                continue
            Qb, dOb = _f64(q[rows_t[a:b], hs, :]), _f64(do[rows_t[a:b], hs, :])
            Kw, Vw = _f64(k[w0:w1, g, :]), _f64(v[w0:w1, g, :])
            lse, P, Ob = _attend(Qb, Kw, Vw, torch.from_numpy(mask), scale)
            B = b - a
            D = (dOb * Ob).sum(dim=-1, keepdim=True)
            dS = P * ((dOb.reshape(B * G, d) @ Vw.T).view(B, G, -1) - D)
            O[a:b, hs, :] = Ob
            L[hs, a:b] = lse.T
            dQ[a:b, hs, :] = scale * (dS.reshape(B * G, -1) @ Kw).view(B, G, d)
    return O.numpy(), L.numpy(), dQ.numpy()


def backward_dq_rows(q, k, v, do, slices: Sequence, rows, scale: float = None,
                     max_elems: int = 1 << 25):
    """dQ for the given rows only."""
    return forward_backward_rows(q, k, v, do, slices, rows, scale, max_elems)[2]


def backward_keys(q, k, v, do, slices: Sequence, keys, scale: float = None, kv_heads=None,
                  max_elems: int = 1 << 25, progress=None):
    """dK and dV for the given key rows only, of the listed kv heads (default:
    all of them) with all their query heads: the gradient of ``backward``
    restricted to the columns j in ``keys``,
      dK_j = scale sum_{h in group} sum_i dS_ij q_i,
      dV_j = sum_{h in group} sum_i P_ij dO_i,
      P_ij = exp(s_ij - LSE_i),  dS_ij = P_ij (dO_i . v_j - D_i),  D_i = dO_i . O_i.
    P needs the LSE of each row over all of its valid keys and D needs the
    row's whole O, so every row is evaluated as in ``forward`` (two-pass, over
    the key window of its batch); only the listed columns enter the sums.
    ``progress`` (optional) is called with a short text after each kv head.
    Returns dK, dV [len(keys), len(kv_heads), d] (float64 ndarrays)."""
    import torch
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    keys = np.asarray(keys, dtype=np.int64)
    heads = list(range(Hkv)) if kv_heads is None else [int(g) for g in kv_heads]
    order = np.argsort(keys, kind="stable")
    skeys = keys[order]
    batches = list(_row_batches(np.arange(Tq), slices, max(1, max_elems // G)))
    dK = torch.zeros(len(keys), len(heads), d, dtype=torch.float64)
    dV = torch.zeros(len(keys), len(heads), d, dtype=torch.float64)
    for gi, g in enumerate(heads):
        hs = slice(g * G, (g + 1) * G)
        for a, b, w0, w1, mask in batches:
            lo, hi = np.searchsorted(skeys, [w0, w1])
            if w1 <= w0 or lo == hi:
                continue                      # no listed key in this batch's window
            pos = torch.from_numpy(order[lo:hi])          # output rows of those keys
            cols = torch.from_numpy(skeys[lo:hi] - w0)    # their window columns
            Qb, dOb = _f64(q[a:b, hs, :]), _f64(do[a:b, hs, :])
            Kw, Vw = _f64(k[w0:w1, g, :]), _f64(v[w0:w1, g, :])
            _, P, Ob = _attend(Qb, Kw, Vw, torch.from_numpy(mask), scale)
            B = b - a
            D = (dOb * Ob).sum(dim=-1, keepdim=True)                         # [B, G, 1]
            Ps = P[:, :, cols]                                                # [B, G, n]
            dS = Ps * ((dOb.reshape(B * G, d) @ Vw[cols].T).view(B, G, -1) - D)
            dK[pos, gi, :] += scale * (dS.reshape(B * G, -1).T @ Qb.reshape(B * G, d))
            dV[pos, gi, :] += Ps.reshape(B * G, -1).T @ dOb.reshape(B * G, d)
        if progress is not None:
            progress(f"kv head {g}: {len(keys)} keys done")
    return dK.numpy(), dV.numpy()


def lse_merge(o1, lse1, o2, lse2):
    """Merge two partial attentions over disjoint key sets (same rows):
    LSE = logaddexp(LSE1, LSE2), O = e^{LSE1-LSE} O1 + e^{LSE2-LSE} O2.
    o: [rows, H, d], lse: [H, rows]."""
    lse = np.logaddexp(lse1, lse2)
    safe = np.where(np.isfinite(lse), lse, 0.0)
    w1 = np.where(np.isfinite(lse1), np.exp(lse1 - safe), 0.0).T[:, :, None]
    w2 = np.where(np.isfinite(lse2), np.exp(lse2 - safe), 0.0).T[:, :, None]
    return w1 * o1 + w2 * o2, lse
