"""Flex-Flash-Attention for AMD Instinct MI355X: Python binding of libffa.

Argument marshalling only: every step runs in the HIP kernels of ``libffa.so``
(see ``include/ffa.h``).  PyTorch provides device memory and the stream.  If
the library is missing this module raises on first use; there is no fallback.

    meta = build_meta(slices, seqlen_q, seqlen_k, head_dim)   # once per mask
    o, lse = fwd(q, k, v, meta)
    dq, dk, dv = bwd(q, k, v, o, lse, do, meta)
    o = ffa_attention(q, k, v, meta)                          # autograd
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libffa.so")

FULL, CAUSAL, INV_CAUSAL, BI_CAUSAL = 0, 1, 2, 3
META_ERR_BOUNDS, META_ERR_TYPE, META_ERR_OVERLAP, META_ERR_CAPACITY = 1, 2, 4, 8

EXPORTED = (
    "ffa_block_meta_workspace_size", "ffa_build_block_meta", "ffa_block_meta_view", "ffa_fwd",
    "ffa_bwd_workspace_size", "ffa_bwd", "ffa_bwd_phases", "ffa_status_string", "ffa_abi_version",
    "ffa_fwd_ex", "ffa_bwd_ex", "ffa_chunk_areas", "ffa_dispatch_chunks", "ffa_rank_slices",
    "ffa_fwd_grouped", "ffa_bwd_grouped", "ffa_bwd_static_scratch",
)
MAX_MASK_GROUPS = 8             # FFA_MAX_MASK_GROUPS
BWD_PRE, BWD_DKDV, BWD_DQ, BWD_ALL = 1, 2, 4, 7
ACCUMULATE = 1                  # FFA_ACCUMULATE flag of ffa_fwd_ex / ffa_bwd_ex
STATIC_SCRATCH_BYTES = 64 << 20 # FFA_STATIC_SCRATCH_BYTES of ffa_bwd_static_scratch


class FFAError(RuntimeError):
    pass


class TensorIn(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("token_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64)]


class TensorOut(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("token_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64)]


class Shape(ctypes.Structure):
    _fields_ = [("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
                ("num_heads_q", ctypes.c_int32), ("num_heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class MetaView(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "bm_fwd", "bn_fwd", "bm_bwd", "bn_bwd", "num_qblocks_fwd", "num_kblocks_fwd",
        "num_qblocks_bwd", "num_kblocks_bwd")] + [("header_bytes", ctypes.c_int64)] + [
        (n, ctypes.c_void_p) for n in (
            "status", "area", "full_block_offset", "mask_block_offset", "k2q_full_block_offset",
            "k2q_mask_block_offset", "qblock_slice_offset", "schedule_fwd", "schedule_bwd",
            "index_base", "list_offsets", "block_records_fwd", "block_records_bwd")]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libffa.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise FFAError(f"{LIB_PATH} is missing: build it with `python -m flexible_mask_attention_amd._build`")
    L = ctypes.CDLL(LIB_PATH)
    st, i32, i64, vp, sz = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    L.ffa_block_meta_workspace_size.argtypes = [i32, i32, i32, i32, vp, ctypes.POINTER(sz)]
    L.ffa_block_meta_workspace_size.restype = st
    L.ffa_build_block_meta.argtypes = [vp, i32, i32, i32, i32, vp, sz, vp]
    L.ffa_build_block_meta.restype = st
    L.ffa_block_meta_view.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(MetaView)]
    L.ffa_block_meta_view.restype = st
    L.ffa_fwd.argtypes = [ctypes.POINTER(Shape), TensorIn, TensorIn, TensorIn, vp, TensorOut, vp, vp]
    L.ffa_fwd.restype = st
    L.ffa_bwd_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(sz)]
    L.ffa_bwd_workspace_size.restype = st
    L.ffa_bwd.argtypes = [ctypes.POINTER(Shape), TensorIn, TensorIn, TensorIn, TensorIn, vp, TensorIn,
                          vp, TensorOut, TensorOut, TensorOut, vp, sz, vp]
    L.ffa_bwd.restype = st
    L.ffa_bwd_phases.argtypes = L.ffa_bwd.argtypes[:-1] + [i32, vp]
    L.ffa_bwd_phases.restype = st
    L.ffa_fwd_ex.argtypes = L.ffa_fwd.argtypes[:-1] + [ctypes.c_uint32, vp]
    L.ffa_fwd_ex.restype = st
    L.ffa_bwd_ex.argtypes = L.ffa_bwd.argtypes[:-1] + [i32, ctypes.c_uint32, vp]
    L.ffa_bwd_ex.restype = st
    L.ffa_fwd_grouped.argtypes = [ctypes.POINTER(Shape), TensorIn, TensorIn, TensorIn, i32, vp, vp,
                                  TensorOut, vp, ctypes.c_uint32, vp]
    L.ffa_fwd_grouped.restype = st
    L.ffa_bwd_grouped.argtypes = [ctypes.POINTER(Shape), TensorIn, TensorIn, TensorIn, TensorIn, vp,
                                  TensorIn, i32, vp, vp, TensorOut, TensorOut, TensorOut, vp, sz, i32,
                                  ctypes.c_uint32, vp]
    L.ffa_bwd_grouped.restype = st
    L.ffa_bwd_static_scratch.argtypes = L.ffa_bwd.argtypes[:-3] + [vp]
    L.ffa_bwd_static_scratch.restype = st
    P32, P64 = ctypes.POINTER(i32), ctypes.POINTER(i64)
    L.ffa_chunk_areas.argtypes = [vp, i32, i32, i32, i32, vp]
    L.ffa_chunk_areas.restype = st
    L.ffa_dispatch_chunks.argtypes = [vp, i32, i32, vp]
    L.ffa_dispatch_chunks.restype = st
    L.ffa_rank_slices.argtypes = [vp, i32, i32, i32, i32, vp, i32, vp, i32, P32, vp, i32, P32]
    L.ffa_rank_slices.restype = st
    L.ffa_status_string.argtypes = [st]
    L.ffa_status_string.restype = ctypes.c_char_p
    L.ffa_abi_version.argtypes = []
    L.ffa_abi_version.restype = i32
    _lib_handle = L
    return L


def _check(code: int, what: str):
    if code != 0:
        raise FFAError(f"{what}: {lib().ffa_status_string(code).decode()} (status {code})")


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _tin(t: torch.Tensor) -> TensorIn:
    return TensorIn(t.data_ptr(), t.stride(0), t.stride(1))


def _tout(t: torch.Tensor) -> TensorOut:
    return TensorOut(t.data_ptr(), t.stride(0), t.stride(1))


def _check_thd(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 3 or not t.is_cuda:
        raise FFAError(f"{name} must be a 3-D bfloat16 CUDA tensor [tokens, heads, head_dim]")
    if t.stride(2) != 1:
        raise FFAError(f"{name}: the head_dim axis must be contiguous")


def _check_like(t: torch.Tensor, like: torch.Tensor, name: str, like_name: str):
    """``t`` (a caller-given output or a second input) must be a THD bf16 tensor
    of ``like``'s shape on ``like``'s device: the kernels write / read it with
    ``like``'s extents."""
    _check_thd(t, name)
    if tuple(t.shape) != tuple(like.shape) or t.device != like.device:
        raise FFAError(f"{name} must have the shape {tuple(like.shape)} and device of {like_name}, "
                       f"got {tuple(t.shape)} on {t.device}")


def _check_lse(lse: torch.Tensor, q: torch.Tensor, name: str = "lse"):
    """The LSE buffer: float32 [Hq, Tq], contiguous, on q's device."""
    want = (q.shape[1], q.shape[0])
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or tuple(lse.shape) != want
            or not lse.is_contiguous() or lse.device != q.device):
        got = (tuple(lse.shape), lse.dtype, lse.device) if isinstance(lse, torch.Tensor) else type(lse)
        raise FFAError(f"{name} must be a contiguous float32 tensor of shape {want} on {q.device}, got {got}")


def _check_inputs(q, k, v, extra=()):
    """q [Tq,Hq,d] and k, v [Tk,Hkv,d] on one device, plus (tensor, name) pairs
    shaped like q (o, do)."""
    _check_thd(q, "q")
    _check_thd(k, "k")
    _check_like(v, k, "v", "k")
    if k.device != q.device or k.shape[2] != q.shape[2]:
        raise FFAError("q and k must share the device and head_dim")
    for t, n in extra:
        _check_like(t, q, n, "q")


def _check_meta(meta, q, k, name="meta"):
    """The metadata must be built for this call's sequence lengths and head_dim
    (the kernels would otherwise write nothing) and live on q's device."""
    if not isinstance(meta, BlockMeta):
        raise FFAError(f"{name} must be a BlockMeta from build_meta")
    if (meta.seqlen_q, meta.seqlen_k, meta.head_dim) != (q.shape[0], k.shape[0], q.shape[2]):
        raise FFAError(f"{name} was built for seqlen_q={meta.seqlen_q}, seqlen_k={meta.seqlen_k}, "
                       f"head_dim={meta.head_dim}; the tensors have {q.shape[0]}, {k.shape[0]}, {q.shape[2]}")
    if meta.buf.device != q.device:
        raise FFAError(f"{name} lives on {meta.buf.device}, the tensors on {q.device}")


class BlockMeta:
    """Device block metadata of one slice table (q2k and k2q CSR lists)."""

    def __init__(self, buf: torch.Tensor, num_slices: int, seqlen_q: int, seqlen_k: int, head_dim: int):
        self.buf, self.num_slices = buf, num_slices
        self.seqlen_q, self.seqlen_k, self.head_dim = seqlen_q, seqlen_k, head_dim
        v = MetaView()
        _check(lib().ffa_block_meta_view(buf.data_ptr(), num_slices, seqlen_q, seqlen_k, head_dim,
                                         ctypes.byref(v)), "ffa_block_meta_view")
        self.view = v

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()

    def _read(self, addr: int, n: int, dtype) -> torch.Tensor:
        off = addr - self.buf.data_ptr()
        item = torch.empty((), dtype=dtype).element_size()
        return self.buf[off:off + n * item].view(dtype).cpu()

    def status(self) -> int:
        """Device status word (synchronising read)."""
        return int(self._read(self.view.status, 1, torch.int32)[0])

    def area(self) -> int:
        """Exact number of valid (query, key) pairs (synchronising read)."""
        return int(self._read(self.view.area, 1, torch.int64)[0])

    def csr(self) -> dict:
        """All CSR arrays as CPU int64 tensors (synchronising; for tests and tools)."""
        v = self.view
        nqf, nkb = v.num_qblocks_fwd, v.num_kblocks_bwd
        lo = self._read(v.list_offsets, 5, torch.int64).tolist()
        qf = self._read(v.full_block_offset, nqf + 1, torch.int32).long()
        qm = self._read(v.mask_block_offset, nqf + 1, torch.int32).long()
        kf = self._read(v.k2q_full_block_offset, nkb + 1, torch.int32).long()
        km = self._read(v.k2q_mask_block_offset, nkb + 1, torch.int32).long()
        qs = self._read(v.qblock_slice_offset, nqf + 1, torch.int32).long()
        base = v.index_base

        def lst(i, n):
            return self._read(base + 4 * lo[i], n, torch.int32).long() if n else torch.zeros(0, dtype=torch.long)

        return {
            "q2k": {"full_block_offset": qf, "full_block_idx": lst(0, int(qf[-1])),
                    "mask_block_offset": qm, "mask_block_idx": lst(1, int(qm[-1]))},
            "k2q": {"full_block_offset": kf, "full_block_idx": lst(2, int(kf[-1])),
                    "mask_block_offset": km, "mask_block_idx": lst(3, int(km[-1]))},
            "qblock_slice_offset": qs, "qblock_slice_idx": lst(4, int(qs[-1])),
            "schedule_fwd": self._read(v.schedule_fwd, nqf, torch.int32).long(),
            "schedule_bwd": self._read(v.schedule_bwd, nkb, torch.int32).long(),
            "records_fwd": self._read(v.block_records_fwd, 16 * nqf, torch.int32).long().view(nqf, 16),
            "records_bwd": self._read(v.block_records_bwd, 16 * nkb, torch.int32).long().view(nkb, 16),
            "tiles": (v.bm_fwd, v.bn_fwd, v.bm_bwd, v.bn_bwd),
        }


def meta_workspace_size(num_slices: int, seqlen_q: int, seqlen_k: int, head_dim: int,
                        host_slices: Optional[torch.Tensor] = None) -> int:
    n = ctypes.c_size_t()
    hp = None
    if host_slices is not None:
        host_slices = host_slices.to(torch.int32).contiguous().cpu()
        hp = host_slices.data_ptr()
    _check(lib().ffa_block_meta_workspace_size(num_slices, seqlen_q, seqlen_k, head_dim, hp,
                                               ctypes.byref(n)), "ffa_block_meta_workspace_size")
    return n.value


def build_meta(slices, seqlen_q: int, seqlen_k: int, head_dim: int, device=None,
               stream=None, out: Optional[torch.Tensor] = None, validate: bool = True) -> BlockMeta:
    """Build block metadata for a slice table.

    ``slices``: sequence of (q_start, q_end, k_start, k_end, mask_type) or an
    int32 tensor [S, 5] (host or device).  The buffer is sized from the host
    copy of the table when one is available; ``out`` (uint8, 256-byte aligned)
    is used as given, and the device status word reports a table that does
    not fit in it.

    ``validate`` (default): read the device status word once the build is done
    (a synchronising read, paid once per mask since the metadata is reused)
    and raise FFAError for a bad table, so that no forward or backward can run
    on metadata that makes the kernels write nothing.  Pass False where no
    synchronisation is allowed (e.g. under graph capture); the caller then
    checks ``status()`` itself."""
    if isinstance(slices, torch.Tensor):
        t = slices.to(torch.int32).reshape(-1, 5)
    else:
        t = torch.tensor([list(s) for s in slices], dtype=torch.int32).reshape(-1, 5)
    host = t.cpu() if not t.is_cuda else None
    dev = torch.device(device) if device is not None else (t.device if t.is_cuda else torch.device("cuda"))
    d_slices = t.to(dev).contiguous()
    S = d_slices.shape[0]
    if out is None:
        nbytes = meta_workspace_size(S, seqlen_q, seqlen_k, head_dim, host)
        out = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(lib().ffa_build_block_meta(d_slices.data_ptr() if S else None, S, seqlen_q, seqlen_k, head_dim,
                                      out.data_ptr(), out.numel(), _stream(stream)), "ffa_build_block_meta")
    m = BlockMeta(out, S, seqlen_q, seqlen_k, head_dim)
    m._slices = d_slices      # keep the device table alive with the metadata
    if validate:
        st = m.status()
        if st != 0:
            names = [n for f, n in ((META_ERR_BOUNDS, "range out of bounds"), (META_ERR_TYPE, "unknown mask type"),
                                    (META_ERR_OVERLAP, "overlapping slices"),
                                    (META_ERR_CAPACITY, "metadata buffer too small")) if st & f]
            raise FFAError(f"bad slice table (status {st}: {', '.join(names)})")
    return m


def _shape(q, k, scale) -> Shape:
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Shape(Tq, Tk, Hq, Hkv, d, float(scale))


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, meta: BlockMeta, scale: float = None,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None,
        accumulate: bool = False):
    """Forward.  q [Tq,Hq,d], k/v [Tk,Hkv,d] bf16 -> (o [Tq,Hq,d] bf16, lse [Hq,Tq] fp32).
    ``accumulate``: merge into the (out, lse) given (ffa_fwd_ex with FFA_ACCUMULATE)."""
    if accumulate and (out is None or lse is None):
        raise FFAError("accumulate needs the previous out and lse")
    _check_inputs(q, k, v)
    _check_meta(meta, q, k)
    sh = _shape(q, k, scale)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _check_like(out, q, "out", "q")
    if lse is None:
        lse = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=q.device)
    _check_lse(lse, q)
    _check(lib().ffa_fwd_ex(ctypes.byref(sh), _tin(q), _tin(k), _tin(v), meta.ptr, _tout(out),
                            lse.data_ptr(), ACCUMULATE if accumulate else 0, _stream(stream)),
           "ffa_fwd_ex")
    return out, lse


def _groups(metas, kv_head_end, q, k):
    if len(metas) != len(kv_head_end) or not 1 <= len(metas) <= MAX_MASK_GROUPS:
        raise FFAError("need 1..8 metadata buffers, one per kv-head group")
    for i, m in enumerate(metas):
        _check_meta(m, q, k, f"metas[{i}]")
    ptrs = (ctypes.c_void_p * len(metas))(*[m.ptr for m in metas])
    ends = (ctypes.c_int32 * len(metas))(*[int(e) for e in kv_head_end])
    return len(metas), ptrs, ends


def fwd_grouped(q, k, v, metas: Sequence[BlockMeta], kv_head_end: Sequence[int], scale: float = None,
                out=None, lse=None, stream=None, accumulate: bool = False):
    """Forward of several masks in one launch: kv heads [kv_head_end[g-1],
    kv_head_end[g]) and their query heads use metas[g] (ffa_fwd_grouped)."""
    if accumulate and (out is None or lse is None):
        raise FFAError("accumulate needs the previous out and lse")
    _check_inputs(q, k, v)
    sh = _shape(q, k, scale)
    ng, ptrs, ends = _groups(metas, kv_head_end, q, k)
    out = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    _check_like(out, q, "out", "q")
    if lse is None:
        lse = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=q.device)
    _check_lse(lse, q)
    _check(lib().ffa_fwd_grouped(ctypes.byref(sh), _tin(q), _tin(k), _tin(v), ng, ptrs, ends,
                                 _tout(out), lse.data_ptr(), ACCUMULATE if accumulate else 0,
                                 _stream(stream)), "ffa_fwd_grouped")
    return out, lse


def bwd_grouped(q, k, v, o, lse, do, metas: Sequence[BlockMeta], kv_head_end: Sequence[int],
                scale: float = None, dq=None, dk=None, dv=None, workspace=None, stream=None,
                phases: int = BWD_ALL, accumulate: bool = False):
    """Backward of a grouped forward (ffa_bwd_grouped) -> (dq, dk, dv)."""
    if accumulate and (dq is None or dk is None or dv is None):
        raise FFAError("accumulate needs the dq, dk, dv to add to")
    _check_inputs(q, k, v, ((o, "o"), (do, "do")))
    _check_lse(lse, q)
    sh = _shape(q, k, scale)
    ng, ptrs, ends = _groups(metas, kv_head_end, q, k)
    dq, dk, dv = _grad_buffers(q, k, v, dq, dk, dv)
    workspace = _workspace(q, k, scale, workspace)
    _check(lib().ffa_bwd_grouped(ctypes.byref(sh), _tin(q), _tin(k), _tin(v), _tin(o), lse.data_ptr(),
                                 _tin(do), ng, ptrs, ends, _tout(dq), _tout(dk), _tout(dv),
                                 workspace.data_ptr(), workspace.numel(), int(phases),
                                 ACCUMULATE if accumulate else 0, _stream(stream)), "ffa_bwd_grouped")
    return dq, dk, dv


# ------------------------------------------------------------------------
# Context-parallel dispatch (host only; see ffa.h)
# ------------------------------------------------------------------------

def _host_slices(slices) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(slices, dtype=np.int32).reshape(-1, 5))
    return a


def chunk_areas(slices, seqlen_q: int, seqlen_k: int, chunk_size: int) -> np.ndarray:
    """Valid (query, key) pairs of each query chunk of ``chunk_size`` tokens."""
    h = _host_slices(slices)
    n = -(-seqlen_q // chunk_size) if chunk_size > 0 else 0
    out = np.zeros(max(n, 1), dtype=np.int64)
    _check(lib().ffa_chunk_areas(h.ctypes.data if len(h) else None, len(h), seqlen_q, seqlen_k,
                                 chunk_size, out.ctypes.data), "ffa_chunk_areas")
    return out[:n]


def dispatch_chunks(areas, cp_size: int) -> np.ndarray:
    """Bucket (rank) of every chunk: equal chunk counts, greedy min-max area."""
    a = np.ascontiguousarray(np.asarray(areas, dtype=np.int64))
    out = np.zeros(len(a), dtype=np.int32)
    _check(lib().ffa_dispatch_chunks(a.ctypes.data, len(a), cp_size, out.ctypes.data),
           "ffa_dispatch_chunks")
    return out


def rank_slices(slices, seqlen_q: int, seqlen_k: int, chunk_size: int, chunks):
    """Local slice table of the share made of ``chunks`` (in that order) and the
    global key ranges it needs: (local_slices [S', 5], kv_ranges [R, 3] =
    (global_start, global_end, buffer_start), local seqlen_k)."""
    h = _host_slices(slices)
    c = np.ascontiguousarray(np.asarray(chunks, dtype=np.int32))
    nl, nk = ctypes.c_int32(), ctypes.c_int32()
    L = lib()
    args = (h.ctypes.data if len(h) else None, len(h), seqlen_q, seqlen_k, chunk_size,
            c.ctypes.data if len(c) else None, len(c))
    code = L.ffa_rank_slices(*args, None, 0, ctypes.byref(nl), None, 0, ctypes.byref(nk))
    if code not in (0, 3):
        _check(code, "ffa_rank_slices")
    loc = np.zeros((max(nl.value, 1), 5), dtype=np.int32)
    kv = np.zeros((max(nk.value, 1), 3), dtype=np.int32)
    _check(L.ffa_rank_slices(*args, loc.ctypes.data, nl.value, ctypes.byref(nl), kv.ctypes.data,
                             nk.value, ctypes.byref(nk)), "ffa_rank_slices")
    loc, kv = loc[: nl.value], kv[: nk.value]
    tk = int(kv[-1, 2] + kv[-1, 1] - kv[-1, 0]) if len(kv) else 0
    return loc, kv, tk


def bwd_workspace_size(q, k, scale=None) -> int:
    n = ctypes.c_size_t()
    sh = _shape(q, k, scale)
    _check(lib().ffa_bwd_workspace_size(ctypes.byref(sh), ctypes.byref(n)), "ffa_bwd_workspace_size")
    return n.value


def _grad_buffers(q, k, v, dq, dk, dv):
    """Caller-given gradient buffers (checked against q, k, v) or new ones."""
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    _check_like(dq, q, "dq", "q")
    _check_like(dk, k, "dk", "k")
    _check_like(dv, v, "dv", "v")
    return dq, dk, dv


def _workspace(q, k, scale, workspace):
    need = bwd_workspace_size(q, k, scale)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise FFAError(f"workspace must be a contiguous buffer on {q.device}")
    return workspace


def bwd(q, k, v, o, lse, do, meta: BlockMeta, scale: float = None, dq=None, dk=None, dv=None,
        workspace: Optional[torch.Tensor] = None, stream=None, phases: int = BWD_ALL,
        accumulate: bool = False):
    """Backward -> (dq, dk, dv), bf16, same shapes as q, k, v.  ``phases``
    selects a subset of the backward kernels (BWD_PRE | BWD_DKDV | BWD_DQ);
    ``accumulate`` adds to the dq, dk, dv given (ffa_bwd_ex with FFA_ACCUMULATE)."""
    if accumulate and (dq is None or dk is None or dv is None):
        raise FFAError("accumulate needs the dq, dk, dv to add to")
    _check_inputs(q, k, v, ((o, "o"), (do, "do")))
    _check_lse(lse, q)
    _check_meta(meta, q, k)
    sh = _shape(q, k, scale)
    dq, dk, dv = _grad_buffers(q, k, v, dq, dk, dv)
    workspace = _workspace(q, k, scale, workspace)
    _check(lib().ffa_bwd_ex(ctypes.byref(sh), _tin(q), _tin(k), _tin(v), _tin(o), lse.data_ptr(),
                            _tin(do), meta.ptr, _tout(dq), _tout(dk), _tout(dv), workspace.data_ptr(),
                            workspace.numel(), int(phases), ACCUMULATE if accumulate else 0,
                            _stream(stream)), "ffa_bwd_ex")
    return dq, dk, dv


def bwd_static_scratch(q, k, v, o, lse, do, meta: BlockMeta, scale: float = None, dq=None, dk=None,
                       dv=None, stream=None):
    """Backward with the library's static scratch array instead of a workspace
    (ffa_bwd_static_scratch): for callers that cannot allocate device memory,
    who pass dq, dk, dv.  Same results as ``bwd``; calls that may overlap on one
    GPU must be serialised."""
    _check_inputs(q, k, v, ((o, "o"), (do, "do")))
    _check_lse(lse, q)
    _check_meta(meta, q, k)
    sh = _shape(q, k, scale)
    dq, dk, dv = _grad_buffers(q, k, v, dq, dk, dv)
    _check(lib().ffa_bwd_static_scratch(ctypes.byref(sh), _tin(q), _tin(k), _tin(v), _tin(o),
                                        lse.data_ptr(), _tin(do), meta.ptr, _tout(dq), _tout(dk),
                                        _tout(dv), _stream(stream)), "ffa_bwd_static_scratch")
    return dq, dk, dv


class FFAFunction(torch.autograd.Function):
    """Autograd wrapper: ``meta`` is one BlockMeta, or a list of them with
    ``kv_head_end`` for several masks in one launch."""

    @staticmethod
    def forward(ctx, q, k, v, meta, scale, kv_head_end=None):
        if isinstance(meta, (list, tuple)):
            o, lse = fwd_grouped(q, k, v, meta, kv_head_end, scale)
        else:
            o, lse = fwd(q, k, v, meta, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.meta, ctx.scale, ctx.kv_head_end = meta, scale, kv_head_end
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        do = do.contiguous()
        if isinstance(ctx.meta, (list, tuple)):
            dq, dk, dv = bwd_grouped(q, k, v, o, lse, do, ctx.meta, ctx.kv_head_end, ctx.scale)
        else:
            dq, dk, dv = bwd(q, k, v, o, lse, do, ctx.meta, ctx.scale)
        return dq, dk, dv, None, None, None


def ffa_attention(q, k, v, meta, scale: float = None, kv_head_end=None) -> torch.Tensor:
    """Flex-Flash-Attention with autograd support (see FFAFunction)."""
    return FFAFunction.apply(q, k, v, meta, scale, kv_head_end)


__all__ = ["BWD_PRE", "BWD_DKDV", "BWD_DQ", "BWD_ALL", "ACCUMULATE", "build_meta", "fwd", "bwd", "ffa_attention", "FFAFunction", "BlockMeta", "lib",
           "bwd_static_scratch", "STATIC_SCRATCH_BYTES",
           "meta_workspace_size", "bwd_workspace_size", "chunk_areas", "dispatch_chunks",
           "fwd_grouped", "bwd_grouped", "MAX_MASK_GROUPS",
           "rank_slices", "FFAError", "FULL", "CAUSAL", "INV_CAUSAL",
           "BI_CAUSAL", "EXPORTED"]
