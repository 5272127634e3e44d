"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad host-visible arguments before enqueuing."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import flexible_mask_attention_amd as ffa
from flexible_mask_attention_amd import workloads as wl
from oracle import ffa_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ffa.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"FFA_API\s+[\w\s\*]+?\b(ffa_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) == 17 and set(names) == set(ffa.EXPORTED)
    L = ffa.lib()
    for n in names:
        assert hasattr(L, n), n
    # and nothing else with the ffa_ prefix is exported
    out = os.popen(f"nm -D --defined-only {ffa.LIB_PATH}").read()
    exported = sorted(set(re.findall(r"\b(ffa_\w+)\b", out)))
    assert exported == names


def test_abi_version_and_strings():
    L = ffa.lib()
    assert L.ffa_abi_version() == 6
    for code in range(7):
        assert len(L.ffa_status_string(code)) > 0
    assert L.ffa_status_string(99) == b"unknown status"


def _shape(Tq=256, Tk=256, Hq=2, Hkv=2, d=64, scale=0.125):
    return ffa.Shape(Tq, Tk, Hq, Hkv, d, scale)


def test_host_validation_returns_before_enqueue():
    L = ffa.lib()
    good = ffa.TensorIn(0x1000, 128, 64)
    goodo = ffa.TensorOut(0x1000, 128, 64)
    meta = 0x10000
    lse = 0x2000
    P = ctypes.byref
    # unsupported head_dim
    assert L.ffa_fwd(P(_shape(d=96)), good, good, good, meta, goodo, lse, None) == 2
    # Hq not a multiple of Hkv
    assert L.ffa_fwd(P(_shape(Hq=3, Hkv=2)), good, good, good, meta, goodo, lse, None) == 1
    # non-finite / zero scale
    assert L.ffa_fwd(P(_shape(scale=float("nan"))), good, good, good, meta, goodo, lse, None) == 1
    assert L.ffa_fwd(P(_shape(scale=0.0)), good, good, good, meta, goodo, lse, None) == 1
    assert L.ffa_fwd(P(_shape(scale=-0.5)), good, good, good, meta, goodo, lse, None) == 1
    # token stride below head_dim
    assert L.ffa_fwd(P(_shape()), ffa.TensorIn(0x1000, 32, 64), good, good, meta, goodo, lse, None) == 1
    # ... also for a single token: its tile is read through a buffer range of
    # valid rows x token stride, which a short stride (0 from expand) would cut
    one_q, one_k = _shape(Tq=1), _shape(Tk=1)
    short = ffa.TensorIn(0x1000, 0, 64)
    short_o = ffa.TensorOut(0x1000, 8, 64)
    assert L.ffa_fwd(P(one_q), short, good, good, meta, goodo, lse, None) == 1
    assert L.ffa_fwd(P(one_q), good, good, good, meta, short_o, lse, None) == 1
    assert L.ffa_fwd(P(one_k), good, short, good, meta, goodo, lse, None) == 1
    assert L.ffa_fwd(P(one_k), good, good, short, meta, goodo, lse, None) == 1
    ws_big = 1 << 30
    assert L.ffa_bwd(P(one_q), good, good, good, good, lse, short, meta, goodo, goodo, goodo,
                     0x100000, ws_big, None) == 1
    assert L.ffa_bwd(P(one_q), good, good, good, short, lse, good, meta, goodo, goodo, goodo,
                     0x100000, ws_big, None) == 1
    assert L.ffa_bwd(P(one_q), good, good, good, good, lse, good, meta, short_o, goodo, goodo,
                     0x100000, ws_big, None) == 1
    assert L.ffa_bwd(P(one_k), good, short, good, good, lse, good, meta, goodo, goodo, goodo,
                     0x100000, ws_big, None) == 1
    assert L.ffa_bwd(P(one_k), good, good, good, good, lse, good, meta, goodo, short_o, goodo,
                     0x100000, ws_big, None) == 1
    assert L.ffa_bwd(P(one_k), good, good, good, good, lse, good, meta, goodo, goodo, short_o,
                     0x100000, ws_big, None) == 1
    assert L.ffa_fwd(P(_shape(Tq=1)), ffa.TensorIn(0x1000, 1 << 23, 64), good, good, meta, goodo, lse, None) == 1
    # null / misaligned tensor pointers, bad strides
    assert L.ffa_fwd(P(_shape()), ffa.TensorIn(0, 128, 64), good, good, meta, goodo, lse, None) == 1
    assert L.ffa_fwd(P(_shape()), ffa.TensorIn(0x1002, 128, 64), good, good, meta, goodo, lse, None) == 1
    assert L.ffa_fwd(P(_shape()), ffa.TensorIn(0x1000, 129, 64), good, good, meta, goodo, lse, None) == 1
    # misaligned metadata / lse
    assert L.ffa_fwd(P(_shape()), good, good, good, meta + 16, goodo, lse, None) == 1
    assert L.ffa_fwd(P(_shape()), good, good, good, meta, goodo, lse + 4, None) == 1
    assert L.ffa_fwd(None, good, good, good, meta, goodo, lse, None) == 1
    # backward workspace too small / null
    ws = ctypes.c_size_t()
    # -D, LSE log2 e and -LSE / scale rows (3 x 2 KB), the split counters of 2
    # candidate key blocks x 2 kv heads (one 256-byte line) and their fp32
    # partials (2 halves x (dK, dV) x 128 keys x 64)
    assert L.ffa_bwd_workspace_size(P(_shape()), P(ws)) == 0
    assert ws.value == 3 * (2 * 256 * 4) + 256 + 2 * 2 * (2 * 2 * 128 * 64 * 4)
    assert L.ffa_bwd(P(_shape()), good, good, good, good, lse, good, meta, goodo, goodo, goodo,
                     0x100000, ws.value - 1, None) == 3
    assert L.ffa_bwd(P(_shape()), good, good, good, good, lse, good, meta, goodo, goodo, goodo,
                     None, ws.value, None) == 1
    assert L.ffa_bwd_phases(P(_shape()), good, good, good, good, lse, good, meta, goodo, goodo, goodo,
                            0x100000, ws.value, 8, None) == 1
    # unknown flag bits of the accumulate entry points
    assert L.ffa_fwd_ex(P(_shape()), good, good, good, meta, goodo, lse, 2, None) == 1
    assert L.ffa_fwd_ex(P(_shape(d=96)), good, good, good, meta, goodo, lse, 1, None) == 2
    assert L.ffa_bwd_ex(P(_shape()), good, good, good, good, lse, good, meta, goodo, goodo, goodo,
                        0x100000, ws.value, 7, 4, None) == 1
    assert L.ffa_bwd_ex(P(_shape()), good, good, good, good, lse, good, meta, goodo, goodo, goodo,
                        0x100000, ws.value - 1, 7, 1, None) == 3
    # output rows that share elements (two workgroups would race on them):
    # an expanded head axis, token and head strides equal, heads reaching
    # into the next token; views into one packed [T][3 H][D] tensor and a
    # head-major [H][T][D] layout pass
    assert L.ffa_fwd(P(_shape()), good, good, good, meta, ffa.TensorOut(0x1000, 128, 0), lse, None) == 1
    assert L.ffa_fwd(P(_shape()), good, good, good, meta, ffa.TensorOut(0x1000, 64, 64), lse, None) == 1
    assert L.ffa_fwd(P(_shape(Hq=4)), good, good, good, meta, goodo, lse, None) == 1
    assert L.ffa_fwd(P(_shape(d=128)), good, good, good, meta, ffa.TensorOut(0x1000, 256, 64), lse, None) == 1
    packed_q, packed_k = ffa.TensorOut(0x1000, 3 * 2 * 64, 64), ffa.TensorOut(0x1080, 3 * 2 * 64, 64)
    head_major = ffa.TensorOut(0x1000, 64, 256 * 64)
    assert L.ffa_bwd(P(_shape()), good, good, good, good, lse, good, meta, packed_q, packed_k, head_major,
                     0x100000, ws.value - 1, None) == 3
    assert L.ffa_bwd(P(_shape()), good, good, good, good, lse, good, meta, ffa.TensorOut(0x1000, 64, 128),
                     goodo, goodo, 0x100000, ws.value, None) == 1
    assert L.ffa_bwd(P(_shape()), good, good, good, good, lse, good, meta, goodo,
                     ffa.TensorOut(0x1000, 128, 0), goodo, 0x100000, ws.value, None) == 1
    assert L.ffa_bwd(P(_shape()), good, good, good, good, lse, good, meta, goodo, goodo,
                     ffa.TensorOut(0x1000, 64, 64), 0x100000, ws.value, None) == 1
    # one token or one head: only head_dim matters along the other axis (each
    # call is given one byte less workspace than its shape needs, so that
    # passing the checks returns 3 and enqueues nothing)
    def ws_short(sh):
        need = ctypes.c_size_t()
        assert L.ffa_bwd_workspace_size(P(sh), P(need)) == 0 and need.value > 0
        return need.value - 1
    sh1 = _shape(Tq=1)
    assert L.ffa_bwd(P(sh1), good, good, good, good, lse, good, meta, ffa.TensorOut(0x1000, 64, 64),
                     goodo, goodo, 0x100000, ws_short(sh1), None) == 3
    sh1 = _shape(Hq=1, Hkv=1)
    flat = ffa.TensorOut(0x1000, 64, 0)
    assert L.ffa_bwd(P(sh1), good, good, good, good, lse, good, meta, flat, flat, flat,
                     0x100000, ws_short(sh1), None) == 3
    # grouped calls: group count, order, coverage of the kv heads, alignment
    Metas = ctypes.c_void_p * 3
    Ends = ctypes.c_int32 * 3
    sh = _shape(Hq=4, Hkv=2)
    goodo = ffa.TensorOut(0x1000, 256, 64)    # four query heads per token
    ok_m, ok_e = Metas(0x10000, 0x20000, 0), Ends(1, 2, 0)
    assert L.ffa_fwd_grouped(P(sh), good, good, good, 0, ok_m, ok_e, goodo, lse, 0, None) == 1
    assert L.ffa_fwd_grouped(P(sh), good, good, good, 9, ok_m, ok_e, goodo, lse, 0, None) == 1
    assert L.ffa_fwd_grouped(P(sh), good, good, good, 2, Metas(0x10000, 0x20010, 0), ok_e, goodo, lse, 0, None) == 1
    assert L.ffa_fwd_grouped(P(sh), good, good, good, 2, ok_m, Ends(2, 1, 0), goodo, lse, 0, None) == 1
    assert L.ffa_fwd_grouped(P(sh), good, good, good, 2, ok_m, Ends(1, 3, 0), goodo, lse, 0, None) == 1
    assert L.ffa_fwd_grouped(P(sh), good, good, good, 1, ok_m, Ends(1, 0, 0), goodo, lse, 0, None) == 1
    assert L.ffa_fwd_grouped(P(sh), good, good, good, 2, None, ok_e, goodo, lse, 0, None) == 1
    # the same checks pass for good groups (an empty query range then enqueues nothing)
    sh0 = _shape(Tq=0, Hq=4, Hkv=2)
    assert L.ffa_fwd_grouped(P(sh0), good, good, good, 2, ok_m, ok_e, goodo, lse, 0, None) == 0
    assert L.ffa_fwd_grouped(P(sh0), good, good, good, 2, ok_m, Ends(2, 2, 0), goodo, lse, 0, None) == 1
    wsg = ctypes.c_size_t()
    assert L.ffa_bwd_workspace_size(P(sh), P(wsg)) == 0
    assert L.ffa_bwd_grouped(P(sh), good, good, good, good, lse, good, 2, ok_m, Ends(1, 1, 0), goodo,
                             goodo, goodo, 0x100000, wsg.value, 7, 0, None) == 1
    assert L.ffa_bwd_grouped(P(sh), good, good, good, good, lse, good, 2, ok_m, ok_e, goodo,
                             goodo, goodo, 0x100000, wsg.value - 1, 7, 0, None) == 3
    # the static-scratch backward: a shape whose workspace exceeds the static
    # array is refused before the library touches the device
    big = _shape(Tq=1 << 22, Tk=1 << 20, Hq=8, Hkv=8, d=128)     # 2 x 128 MiB of row statistics
    need = ctypes.c_size_t()
    assert L.ffa_bwd_workspace_size(P(big), P(need)) == 0 and need.value > ffa.STATIC_SCRATCH_BYTES
    assert L.ffa_bwd_static_scratch(P(big), good, good, good, good, lse, good, meta, goodo, goodo, goodo,
                                    None) == 6
    assert L.ffa_bwd_static_scratch(P(_shape(d=96)), good, good, good, good, lse, good, meta, goodo,
                                    goodo, goodo, None) == 2
    assert L.ffa_bwd_static_scratch(None, good, good, good, good, lse, good, meta, goodo, goodo, goodo,
                                    None) == 1
    # metadata build: bad sizes, misaligned buffer, too-small buffer
    n = ctypes.c_size_t()
    assert L.ffa_block_meta_workspace_size(-1, 10, 10, 64, None, P(n)) == 1
    assert L.ffa_block_meta_workspace_size(1, 10, 10, 80, None, P(n)) == 2
    assert L.ffa_block_meta_workspace_size(1, 10, 10, 64, None, P(n)) == 0
    assert L.ffa_build_block_meta(0x1000, 1, 10, 10, 64, 0x10010, n.value, None) == 1
    assert L.ffa_build_block_meta(0x1000, 1, 10, 10, 64, 0x10000, 100, None) == 3
    assert L.ffa_build_block_meta(0, 1, 10, 10, 64, 0x10000, n.value, None) == 1


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_meta_workspace_bound_covers_actual_lists(idx):
    """The host-side size bound must hold the exact CSR lists of the oracle."""
    W = wl.workload(idx)
    for c in W.calls[:1]:
        host = torch.tensor(c.slices, dtype=torch.int32)
        nbytes = ffa.meta_workspace_size(len(c.slices), c.Tq, c.Tk, c.d, host)
        dense = ffa.meta_workspace_size(len(c.slices), c.Tq, c.Tk, c.d, None)
        assert nbytes <= dense
        qf = orc.block_meta(c.slices, c.Tq, c.Tk, 128, 64, "q2k")
        kb = orc.block_meta(c.slices, c.Tq, c.Tk, 64, 128, "k2q")
        entries = len(qf["full_block_idx"]) + len(qf["mask_block_idx"]) + \
            len(kb["full_block_idx"]) + len(kb["mask_block_idx"])
        nq = -(-c.Tq // 128)
        nslices_lists = sum((s[1] - 1) // 128 - s[0] // 128 + 1 for s in c.slices if s[1] > s[0])
        assert nbytes >= 4 * (entries + nslices_lists)


def test_source_digest_ignores_comments_only(tmp_path):
    """The digest that keys recorded hardware counters changes with the code
    of the HIP sources, not with their comments."""
    import bench
    d = tmp_path / "csrc"
    d.mkdir()
    (d / "a.hip").write_text("int f() {  // one\n  return 1;\n}\n")
    base = bench.source_code_digest(str(d))
    (d / "a.hip").write_text("// header\nint f() {  // two\n\n  return 1;   \n}\n")
    assert bench.source_code_digest(str(d)) == base
    (d / "a.hip").write_text("int f() {\n  return 2;\n}\n")
    assert bench.source_code_digest(str(d)) != base
