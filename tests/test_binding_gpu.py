"""The Python binding refuses, before anything is enqueued, buffers that the
kernels would read or write in the wrong shape, type or layout, and metadata
built for another call.  Each case raises FFAError and leaves every output
buffer as it was: the good buffers of the call are filled with a sentinel
beforehand and checked after a synchronisation.  Shape, dtype and layout are
checked by the binding; outputs whose (token, head) rows overlap (an expanded
head axis) are refused by the C ABI's own argument checks."""
import pytest
import torch

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENT = 7.0


def _case():
    c = wl.Call([(0, 256, 0, 256, wl.CAUSAL)], 256, 256, 4, 2, 64)
    T = wl.make_tensors(c, 3)
    q, k, v, do = (T[n].to(DEV) for n in ("q", "k", "v", "do"))
    return c, q, k, v, do, ffa.build_meta(c.slices, c.Tq, c.Tk, c.d)


def _untouched(*ts):
    torch.cuda.synchronize()
    for t in ts:
        assert bool((t.float() == SENT).all()), "a refused call wrote an output"


def test_forward_refuses_bad_buffers_and_foreign_metadata():
    c, q, k, v, _, meta = _case()
    out = torch.full_like(q, SENT)
    lse = torch.full((c.Hq, c.Tq), SENT, device=DEV)
    bad_meta = {
        "other seqlen_q": ffa.build_meta([(0, 128, 0, 128, wl.CAUSAL)], 128, c.Tk, c.d),
        "other head_dim": ffa.build_meta(c.slices, c.Tq, c.Tk, 128),
    }
    for what, m in bad_meta.items():
        with pytest.raises(ffa.FFAError, match="was built for"):
            ffa.fwd(q, k, v, m, out=out, lse=lse)
        _untouched(out, lse)
    expanded_base = torch.full((c.Tq, 1, c.d), SENT, dtype=torch.bfloat16, device=DEV)
    bad_out = {
        "short": (torch.full((c.Tq - 1, c.Hq, c.d), SENT, dtype=torch.bfloat16, device=DEV), "shape"),
        "fp32": (torch.full((c.Tq, c.Hq, c.d), SENT, device=DEV), "bfloat16"),
        "head_dim strided": (torch.full((c.Tq, c.d, c.Hq), SENT, dtype=torch.bfloat16,
                                        device=DEV).transpose(1, 2), "contiguous"),
        # every head of a token on the same row: the C ABI's overlap check
        "expanded heads": (expanded_base.expand(c.Tq, c.Hq, c.d), "invalid argument"),
    }
    for what, (o, msg) in bad_out.items():
        with pytest.raises(ffa.FFAError, match=msg):
            ffa.fwd(q, k, v, meta, out=o, lse=lse)
        _untouched(lse, expanded_base)
    bad_lse = {
        "fp16": torch.full((c.Hq, c.Tq), SENT, dtype=torch.float16, device=DEV),
        "token-major": torch.full((c.Tq, c.Hq), SENT, device=DEV),
        "strided": torch.full((c.Tq, c.Hq), SENT, device=DEV).t(),
    }
    for what, l in bad_lse.items():
        with pytest.raises(ffa.FFAError, match="float32 tensor of shape"):
            ffa.fwd(q, k, v, meta, out=out, lse=l)
        _untouched(out, l)
    # the good buffers still work
    ffa.fwd(q, k, v, meta, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and not bool((out.float() == SENT).all())


def test_backward_refuses_bad_buffers_and_foreign_metadata():
    c, q, k, v, do, meta = _case()
    o, lse = ffa.fwd(q, k, v, meta)
    dq = torch.full_like(q, SENT)
    dk = torch.full_like(k, SENT)
    dv = torch.full_like(v, SENT)
    grads = dict(dq=dq, dk=dk, dv=dv)

    def call(**kw):
        args = dict(q=q, k=k, v=v, o=o, lse=lse, do=do, meta=meta, **grads)
        args.update(kw)
        ffa.bwd(**args)

    expanded_base = torch.full((c.Tk, 1, c.d), SENT, dtype=torch.bfloat16, device=DEV)
    cases = {
        "meta for another seqlen_k": (dict(meta=ffa.build_meta([(0, 256, 0, 128, wl.FULL)], c.Tq, 128, c.d)),
                                      "was built for"),
        "lse token-major": (dict(lse=lse.t().contiguous()), "float32 tensor of shape"),
        "o short": (dict(o=o[:-1]), "shape"),
        "do fp32": (dict(do=do.float()), "bfloat16"),
        "dq short": (dict(dq=torch.full((c.Tq - 1, c.Hq, c.d), SENT, dtype=torch.bfloat16, device=DEV)), "shape"),
        "dk fp32": (dict(dk=torch.full((c.Tk, c.Hkv, c.d), SENT, device=DEV)), "bfloat16"),
        "dv expanded heads": (dict(dv=expanded_base.expand(c.Tk, c.Hkv, c.d)), "invalid argument"),
    }
    for what, (kw, msg) in cases.items():
        with pytest.raises(ffa.FFAError, match=msg):
            call(**kw)
        _untouched(dq, dk, dv, expanded_base)
    call()
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        assert torch.isfinite(g.float()).all() and not bool((g.float() == SENT).all())
