"""Expected values for structured inputs at any size (test helper, CPU).

With every key equal (k_j = kappa for all j of a kv head), all valid scores of
a query row are equal, so the softmax is uniform over the row's valid set J_i
(n_i = |J_i| keys).  With rank-1 values v_j = f_j u (u of powers of two, so the
bf16 products are exact) the forward and backward reduce to sums over
intervals:

  LSE_i = scale q_i.kappa + ln n_i          O_i = mean_{j in J_i}(f_j) u = fbar_i u
  D_i = dO_i.O_i = fbar_i g_i,  g_i = dO_i.u
  dS_ij = (f_j g_i - fbar_i g_i) / n_i  on J_i
  dV_j = sum_{i: j in J_i} dO_i / n_i
  dK_j = scale [ f_j sum_{i: j in J_i} (g_i/n_i) q_i - sum_{i: j in J_i} (fbar_i g_i/n_i) q_i ]
  dQ_i = scale kappa sum_j dS_ij = 0

Means over J_i use prefix sums of f over keys (row intervals), and the sums
over {i : j in J_i} use prefix sums over rows of the per-row vectors, read at
each slice's column interval of key j.  Row and column intervals come from the
oracle's interval forms (pinned there against the mask predicate).
tests/test_props.py pins these formulas against the oracle on small inputs.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import ffa_oracle as orc


def structured_inputs(Tq, Tk, Hq, Hkv, d, seed, device="cpu"):
    """q, do ~ N(0,1); k_j = kappa (per kv head); v_j = f_j u.  All bf16."""
    g = torch.Generator(device=device).manual_seed(seed)
    q = torch.randn(Tq, Hq, d, generator=g, device=device).to(torch.bfloat16)
    do = torch.randn(Tq, Hq, d, generator=g, device=device).to(torch.bfloat16)
    kappa = torch.randn(1, Hkv, d, generator=g, device=device).to(torch.bfloat16)
    f = torch.randn(Tk, Hkv, 1, generator=g, device=device).to(torch.bfloat16)
    sgn = torch.randint(0, 2, (1, Hkv, d), generator=g, device=device) * 2 - 1
    pw = torch.randint(-1, 2, (1, Hkv, d), generator=g, device=device)
    u = (sgn * torch.pow(2.0, pw.float())).to(torch.bfloat16)
    k = kappa.expand(Tk, Hkv, d).contiguous()
    v = (f * u).contiguous()
    return {"q": q, "k": k, "v": v, "do": do, "kappa": kappa, "f": f, "u": u}


class Structured:
    """Per-head expected values for one slice table and structured inputs."""

    def __init__(self, inp, slices, Tq, Tk, scale=None):
        self.q = inp["q"].cpu()
        self.do = inp["do"].cpu()
        self.kappa = inp["kappa"].cpu().double()[0]          # [Hkv, d]
        self.f = inp["f"].cpu().double()[:, :, 0]            # [Tk, Hkv]
        self.u = inp["u"].cpu().double()[0]                  # [Hkv, d]
        self.slices, self.Tq, self.Tk = slices, Tq, Tk
        self.Hq, self.d = self.q.shape[1], self.q.shape[2]
        self.Hkv = self.kappa.shape[0]
        self.G = self.Hq // self.Hkv
        self.scale = scale if scale is not None else 1.0 / math.sqrt(self.d)
        rows = np.arange(Tq)
        self.rivs = [orc.row_intervals_vec(s, rows) for s in slices]
        n = np.zeros(Tq, dtype=np.int64)
        for lo, hi, ok in self.rivs:
            n += np.where(ok, hi - lo + 1, 0)
        self.n = n
        self.nz = n > 0
        self.ninv = np.where(self.nz, 1.0 / np.maximum(n, 1), 0.0)
        self._fbar = {}

    def fbar(self, g):
        if g not in self._fbar:
            F = np.concatenate([[0.0], np.cumsum(self.f[:, g].numpy())])
            fsum = np.zeros(self.Tq)
            for lo, hi, ok in self.rivs:
                fsum += np.where(ok, F[np.clip(hi + 1, 0, self.Tk)] - F[np.clip(lo, 0, self.Tk)], 0.0)
            self._fbar[g] = fsum * self.ninv
        return self._fbar[g]

    def rows(self, h):
        """O [Tq, d] and LSE [Tq] of query head h (all rows)."""
        g = h // self.G
        qh = self.q[:, h, :].double().numpy()
        lse = np.where(self.nz, self.scale * (qh @ self.kappa[g].numpy()) + np.log(np.maximum(self.n, 1)), -np.inf)
        O = self.fbar(g)[:, None] * self.u[g].numpy()[None, :]
        return O, lse

    def keys(self, g, keys):
        """dK, dV [len(keys), d] of kv head g at the given key indices."""
        keys = np.asarray(keys, dtype=np.int64)
        d = self.d
        civs = [orc.col_intervals_vec(s, keys) for s in self.slices]
        acc = torch.zeros(len(keys), 3 * d, dtype=torch.float64)
        fbar = self.fbar(g)
        u = self.u[g].numpy()
        for h in range(g * self.G, (g + 1) * self.G):
            qh = self.q[:, h, :].double()
            doh = self.do[:, h, :].double()
            gi = doh.numpy() @ u
            w1 = torch.from_numpy(gi * self.ninv)[:, None]
            w2 = torch.from_numpy(fbar * gi * self.ninv)[:, None]
            w3 = torch.from_numpy(self.ninv)[:, None]
            vals = torch.cat([w1 * qh, w2 * qh, w3 * doh], dim=1)
            P = torch.cat([torch.zeros(1, 3 * d, dtype=torch.float64), torch.cumsum(vals, dim=0)])
            for lo, hi, ok in civs:
                sel = np.nonzero(ok)[0]
                if len(sel) == 0:
                    continue
                acc[sel] += P[torch.from_numpy(hi[sel] + 1)] - P[torch.from_numpy(lo[sel])]
        acc = acc.numpy()
        fj = self.f[keys, g].numpy()[:, None]
        dK = self.scale * (fj * acc[:, :d] - acc[:, d:2 * d])
        dV = acc[:, 2 * d:]
        return dK, dV
