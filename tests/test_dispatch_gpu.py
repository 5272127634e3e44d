"""Context-parallel shares end to end on the GPU: a global mask is dispatched
over 4 ranks (1 GPU plays every rank in turn); each rank builds its local
slice table, gathers its query rows and the key/value ranges it receives, and
runs the HIP forward and backward on them.  Against the fp64 oracle of the
global problem: every rank's O, LSE and dQ rows, and the sum over ranks of the
dK, dV each rank returns for its received keys (the reduction back to the key
owners), at the tolerances of test_attention_gpu."""
import random

import numpy as np
import pytest
import torch

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl
from oracle import ffa_oracle as orc
from tests.test_attention_gpu import check_grad, check_lse, check_o

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _tables():
    yield "varlen_causal", wl.varlen_slices([300, 1000, 748], ffa.CAUSAL), 2048, 2048
    rng = random.Random(9)
    bc = []
    for S, E in ((0, 900), (900, 2048)):
        for bs in range(S, E, 256):
            bc.append((bs, min(bs + 256, E), S, min(bs + 256, E), ffa.FULL))
    yield "block_causal", bc, 2048, 2048
    yield "random", wl.random_slices(rng, 1536, 1200, 6), 1536, 1200


@pytest.mark.parametrize("which", ["varlen_causal", "block_causal", "random"])
def test_dispatched_shares_match_global_oracle(which):
    name, sl, Tq, Tk = next(t for t in _tables() if t[0] == which)
    Hq, Hkv, d, chunk, cp = 4, 2, 128, 128, 4
    call = wl.Call(sl, Tq, Tk, Hq, Hkv, d)
    T = wl.make_tensors(call, 4242)
    print(f"share test {name}: Tq={Tq} Tk={Tk} chunk={chunk} cp={cp}", flush=True)
    o_ref, l_ref = orc.forward(T["q"], T["k"], T["v"], sl)
    dq_ref, dk_ref, dv_ref = orc.backward(T["q"], T["k"], T["v"], T["do"], sl)

    n = -(-Tq // chunk)
    areas = ffa.chunk_areas(sl, Tq, Tk, chunk)
    bucket = ffa.dispatch_chunks(areas, cp)
    dk_sum = torch.zeros(Tk, Hkv, d, dtype=torch.float64)
    dv_sum = torch.zeros(Tk, Hkv, d, dtype=torch.float64)
    for r in range(cp):
        chunks = [c for c in range(n) if bucket[c] == r]
        loc, kv, tk = ffa.rank_slices(sl, Tq, Tk, chunk, chunks)
        rows = np.concatenate([np.arange(c * chunk, min((c + 1) * chunk, Tq)) for c in chunks])
        keys = np.concatenate([np.arange(a, b) for a, b, _ in kv.tolist()])
        ri, ki = torch.from_numpy(rows), torch.from_numpy(keys)
        q, do = T["q"][ri].to(DEV), T["do"][ri].to(DEV)
        k, v = T["k"][ki].to(DEV), T["v"][ki].to(DEV)
        print(f"  rank {r}: chunks {chunks} local slices {len(loc)} received keys {tk}", flush=True)
        meta = ffa.build_meta([tuple(s) for s in loc.tolist()], len(rows), tk, d)
        o, lse = ffa.fwd(q, k, v, meta)
        dq, dk, dv = ffa.bwd(q, k, v, o, lse, do, meta)
        torch.cuda.synchronize()
        assert meta.status() == 0
        check_o(o, o_ref[rows], f"rank {r} O")
        check_lse(lse, l_ref[:, rows], f"rank {r} LSE")
        check_grad(dq, dq_ref[rows], f"rank {r} dQ")
        dk_sum[ki] += dk.double().cpu()
        dv_sum[ki] += dv.double().cpu()
    check_grad(dk_sum, dk_ref, "dK summed over ranks")
    check_grad(dv_sum, dv_ref, "dV summed over ranks")
