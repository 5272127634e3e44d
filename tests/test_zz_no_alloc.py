"""The backward for callers that cannot allocate (ffa_bwd_static_scratch, its
scratch in the library's static device array) against ffa_bwd with a caller
workspace: same kernels, so dq, dk, dv must be bitwise equal.  Two calls in a
row, the second with a smaller input, so the second runs on scratch the first
left behind (split counters, partials, row statistics)."""
import random

import pytest
import torch

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(call, seed):
    T = wl.make_tensors(call, seed)
    q, k, v, do = (T[n].to(DEV) for n in ("q", "k", "v", "do"))
    meta = ffa.build_meta(call.slices, call.Tq, call.Tk, call.d)
    o, lse = ffa.fwd(q, k, v, meta)
    return q, k, v, do, o, lse, meta


def test_static_scratch_backward_matches_workspace_backward():
    rng = random.Random(31)
    calls = [
        # one 8K causal sequence: its longest key blocks are split, so the
        # split counters and fp32 partials live in the static array
        wl.Call([(0, 8192, 0, 8192, wl.CAUSAL)], 8192, 8192, 2, 1, 128),
        # then a smaller table with several slices per row, head_dim 64
        wl.Call(wl.random_banded_slices(rng, 700, 650), 700, 650, 4, 2, 64),
    ]
    for i, c in enumerate(calls):
        print(f"call {i}: Tq={c.Tq} Tk={c.Tk} Hq={c.Hq} Hkv={c.Hkv} d={c.d}", flush=True)
        q, k, v, do, o, lse, meta = _inputs(c, 700 + i)
        assert ffa.bwd_workspace_size(q, k) <= ffa.STATIC_SCRATCH_BYTES
        want = ffa.bwd(q, k, v, o, lse, do, meta)
        got = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
        ffa.bwd_static_scratch(q, k, v, o, lse, do, meta, dq=got[0], dk=got[1], dv=got[2])
        torch.cuda.synchronize()
        for a, b, n in zip(want, got, ("dq", "dk", "dv")):
            assert torch.equal(a, b), f"call {i}: {n} differs from the workspace backward"


def test_static_scratch_refuses_oversized_shapes():
    """A shape whose workspace exceeds the static array gives FFA_ERR_TOO_LARGE
    and launches nothing (the outputs keep their values)."""
    Tq, Tk, H, d = 1 << 19, 128, 16, 64       # 2 x 32 MiB of row statistics
    q = torch.zeros(Tq, H, d, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(Tk, H, d, dtype=torch.bfloat16, device=DEV)
    assert ffa.bwd_workspace_size(q, k) > ffa.STATIC_SCRATCH_BYTES
    meta = ffa.build_meta([(0, 8, 0, 8, wl.FULL)], Tq, Tk, d)
    lse = torch.zeros(H, Tq, dtype=torch.float32, device=DEV)
    dk = torch.full_like(k, 3.0)
    with pytest.raises(ffa.FFAError, match="static array"):
        ffa.bwd_static_scratch(q, k, k, q, lse, q, meta, dk=dk)
    torch.cuda.synchronize()
    assert bool((dk == 3.0).all())
