"""Python binding of libattnres (AttnRes depth aggregation on MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attnres.h``.  PyTorch supplies
device memory and the current stream.  There is no fallback: if the library
is not built, importing this module raises.

Layouts (see the header): ``hist [n_hist, T, d]`` (bf16 or fp32), pseudo-queries
``w [n_q, d]`` fp32 (row j is read ``q_begin + j``), ``out [n_q, T, d]``,
``lse [n_q, T]`` fp32.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import _build

LIBRARY = _build.LIBRARY

F32, BF16 = 0, 1
FULL, BLOCK = 0, 1

STATUS = {0: "ATTNRES_OK", 1: "ATTNRES_ERR_INVALID_ARG", 2: "ATTNRES_ERR_UNSUPPORTED",
          3: "ATTNRES_ERR_ALIGN", 4: "ATTNRES_ERR_WORKSPACE", 5: "ATTNRES_ERR_HIP"}

# every symbol include/attnres.h declares
EXPORTS = ["attnres_full_fwd", "attnres_full_fwd_q", "attnres_query_proj", "attnres_block_fwd",
           "attnres_block_fwd_q", "attnres_block_phase1", "attnres_block_phase2",
           "attnres_block_phase1_q", "attnres_block_phase2_q",
           "attnres_bwd", "attnres_bwd_noalloc", "attnres_bwd_noalloc_max_workspace",
           "attnres_bwd_workspace_bytes", "attnres_block_index_table",
           "attnres_status_string", "attnres_last_error"]

if not os.path.exists(LIBRARY):
    raise ImportError(f"libattnres.so is not built ({LIBRARY}); run __graft_entry__.build()")

_lib = ctypes.CDLL(LIBRARY)

_i64, _f32, _int, _vp, _sz = (ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
                              ctypes.c_size_t)
_lib.attnres_full_fwd.restype = _int
_lib.attnres_full_fwd.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _i64, _i64, _f32, _vp, _i64,
                                  _vp, _int, _vp, _vp, _vp, _vp, _vp]
_lib.attnres_block_fwd.restype = _int
_lib.attnres_block_fwd.argtypes = [_vp, _int, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _f32, _vp,
                                   _int, _vp, _vp, _vp]
_lib.attnres_full_fwd_q.restype = _int
_lib.attnres_full_fwd_q.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _i64, _i64, _f32, _vp, _i64,
                                    _vp, _int, _vp, _vp]
_lib.attnres_query_proj.restype = _int
_lib.attnres_query_proj.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _int, _vp, _vp]
_lib.attnres_block_phase1.restype = _int
_lib.attnres_block_phase1.argtypes = [_vp, _i64, _i64, _i64, _vp, _int, _vp, _vp, _i64, _f32, _vp,
                                      _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp]
_lib.attnres_block_phase2.restype = _int
_lib.attnres_block_phase2.argtypes = [_vp, _int, _i64, _i64, _vp, _int, _vp, _vp, _vp, _f32, _vp,
                                      _int, _vp, _vp, _vp, _vp]
_lib.attnres_block_fwd_q.restype = _int
_lib.attnres_block_fwd_q.argtypes = [_vp, _int, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _f32,
                                     _vp, _int, _vp, _vp]
_lib.attnres_block_phase1_q.restype = _int
_lib.attnres_block_phase1_q.argtypes = [_vp, _i64, _i64, _i64, _vp, _int, _vp, _vp, _i64, _f32,
                                        _vp, _vp, _vp, _vp, _int, _vp, _vp]
_lib.attnres_block_phase2_q.restype = _int
_lib.attnres_block_phase2_q.argtypes = [_vp, _int, _i64, _i64, _vp, _int, _vp, _vp, _vp, _f32,
                                        _vp, _int, _vp, _vp]
_lib.attnres_bwd.restype = _int
_lib.attnres_bwd.argtypes = [_int, _i64, _vp, _int, _i64, _i64, _i64, _vp, _i64, _i64, _f32,
                             _vp, _int, _vp, _int, _int, _vp, _vp, _sz, _vp]
_lib.attnres_bwd_noalloc.restype = _int
_lib.attnres_bwd_noalloc.argtypes = [_int, _i64, _vp, _int, _i64, _i64, _i64, _vp, _i64, _i64,
                                     _f32, _vp, _int, _vp, _int, _int, _vp, _vp]
_lib.attnres_bwd_noalloc_max_workspace.restype = _sz
_lib.attnres_bwd_noalloc_max_workspace.argtypes = []
_lib.attnres_bwd_workspace_bytes.restype = _sz
_lib.attnres_bwd_workspace_bytes.argtypes = [_int, _i64, _i64, _i64, _i64, _i64, _i64]
_lib.attnres_block_index_table.restype = _int
_lib.attnres_block_index_table.argtypes = [_i64, _i64, _i64, _i64, _vp]
_lib.attnres_status_string.restype = ctypes.c_char_p
_lib.attnres_status_string.argtypes = [_int]
_lib.attnres_last_error.restype = ctypes.c_char_p
_lib.attnres_last_error.argtypes = []


class AttnResError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def last_error() -> str:
    return _lib.attnres_last_error().decode()


def status_string(status: int) -> str:
    return _lib.attnres_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise AttnResError(status, last_error())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _torch_dtype(code: int):
    import torch
    return torch.float32 if code == F32 else torch.bfloat16


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _require(t, name, *, dtype=None, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def full_fwd(hist, w, *, q_begin: int = 0, n_q: int | None = None, eps: float = 1e-6,
             rinv=None, rinv_valid_rows: int = 0, out=None, out_dtype=None, lse=None,
             want_lse: bool = True, normed=None, norm_gain=None, alpha=None):
    """Full AttnRes reads q_begin .. q_begin+n_q-1.  Returns (out, lse).
    normed (same shape and dtype as out) receives the fused pre-norm
    norm_gain * h * r(h) when given (norm_gain [n_q, d] fp32 or None); alpha
    [n_q, n_hist, T] fp32 receives the softmax weights when given."""
    import torch
    _require(hist, "hist")
    n_hist, T, d = hist.shape
    n_q = n_hist - q_begin if n_q is None else n_q
    _require(w, "w", dtype=torch.float32, shape=(n_q, d))
    odt = _dtype_code(hist) if out_dtype is None else (F32 if out_dtype == torch.float32 else BF16)
    if out is None:
        out = torch.empty((n_q, T, d), dtype=_torch_dtype(odt), device=hist.device)
    else:
        _require(out, "out", shape=(n_q, T, d))
        odt = _dtype_code(out)
    if lse is None and want_lse:
        lse = torch.empty((n_q, T), dtype=torch.float32, device=hist.device)
    if lse is not None:
        _require(lse, "lse", dtype=torch.float32, shape=(n_q, T))
    if rinv is not None:
        _require(rinv, "rinv", dtype=torch.float32, shape=(n_hist, T))
    if normed is not None:
        _require(normed, "normed", dtype=out.dtype, shape=(n_q, T, d))
        if norm_gain is not None:
            _require(norm_gain, "norm_gain", dtype=torch.float32, shape=(n_q, d))
    if alpha is not None:
        _require(alpha, "alpha", dtype=torch.float32, shape=(n_q, n_hist, T))
    _check(_lib.attnres_full_fwd(_ptr(hist), _dtype_code(hist), n_hist, T, d, _ptr(w), q_begin,
                                 n_q, eps, _ptr(rinv), rinv_valid_rows, _ptr(out), odt, _ptr(lse),
                                 _ptr(norm_gain), _ptr(normed), _ptr(alpha), _stream(hist)))
    return out, lse


def query_proj(x, W, *, q=None):
    """Input-dependent queries q[j, t] = W[j] @ x[j, t] (bf16 x [n_q, T, d] and
    W [n_q, d, d]; fp32 q).  Returns q."""
    import torch
    _require(x, "x", dtype=torch.bfloat16)
    n_q, T, d = x.shape
    _require(W, "W", dtype=torch.bfloat16, shape=(n_q, d, d))
    if q is None:
        q = torch.empty((n_q, T, d), dtype=torch.float32, device=x.device)
    _require(q, "q", dtype=torch.float32, shape=(n_q, T, d))
    _check(_lib.attnres_query_proj(_ptr(x), BF16, n_q, T, d, _ptr(W), BF16, _ptr(q), _stream(x)))
    return q


def full_fwd_q(hist, q, *, q_begin: int = 0, eps: float = 1e-6, rinv=None,
               rinv_valid_rows: int = 0, out=None, out_dtype=None, lse=None, want_lse: bool = True):
    """Full AttnRes with a query per (read, token): q [n_q, T, d] fp32 for reads
    q_begin .. q_begin + n_q - 1.  Returns (out, lse)."""
    import torch
    _require(hist, "hist")
    n_hist, T, d = hist.shape
    n_q = q.shape[0]
    _require(q, "q", dtype=torch.float32, shape=(n_q, T, d))
    odt = _dtype_code(hist) if out_dtype is None else (F32 if out_dtype == torch.float32 else BF16)
    if out is None:
        out = torch.empty((n_q, T, d), dtype=_torch_dtype(odt), device=hist.device)
    else:
        _require(out, "out", shape=(n_q, T, d))
        odt = _dtype_code(out)
    if lse is None and want_lse:
        lse = torch.empty((n_q, T), dtype=torch.float32, device=hist.device)
    if lse is not None:
        _require(lse, "lse", dtype=torch.float32, shape=(n_q, T))
    if rinv is not None:
        _require(rinv, "rinv", dtype=torch.float32, shape=(n_hist, T))
    _check(_lib.attnres_full_fwd_q(_ptr(hist), _dtype_code(hist), n_hist, T, d, _ptr(q), q_begin,
                                   n_q, eps, _ptr(rinv), rinv_valid_rows, _ptr(out), odt,
                                   _ptr(lse), _stream(hist)))
    return out, lse


def block_fwd(hist, w, S: int, *, q_begin: int = 0, n_q: int | None = None, eps: float = 1e-6,
              out=None, out_dtype=None, lse=None, want_lse: bool = True, alpha=None):
    """Block AttnRes reads (block size S), two-phase.  Returns (out, lse)."""
    import torch
    _require(hist, "hist")
    n_hist, T, d = hist.shape
    n_q = n_hist - q_begin if n_q is None else n_q
    _require(w, "w", dtype=torch.float32, shape=(n_q, d))
    odt = _dtype_code(hist) if out_dtype is None else (F32 if out_dtype == torch.float32 else BF16)
    if out is None:
        out = torch.empty((n_q, T, d), dtype=_torch_dtype(odt), device=hist.device)
    else:
        _require(out, "out", shape=(n_q, T, d))
        odt = _dtype_code(out)
    if lse is None and want_lse:
        lse = torch.empty((n_q, T), dtype=torch.float32, device=hist.device)
    if lse is not None:
        _require(lse, "lse", dtype=torch.float32, shape=(n_q, T))
    if alpha is not None:
        _require(alpha, "alpha", dtype=torch.float32, shape=(n_q, n_hist, T))
    _check(_lib.attnres_block_fwd(_ptr(hist), _dtype_code(hist), n_hist, T, d, S, _ptr(w),
                                  q_begin, n_q, eps, _ptr(out), odt, _ptr(lse), _ptr(alpha),
                                  _stream(hist)))
    return out, lse


def block_fwd_q(hist, q, S: int, *, q_begin: int = 0, eps: float = 1e-6, out=None,
                out_dtype=None, lse=None, want_lse: bool = True):
    """Block AttnRes reads q_begin .. q_begin + n_q - 1 (block size S) with a
    query per (read, token): q [n_q, T, d] fp32.  Returns (out, lse)."""
    import torch
    _require(hist, "hist")
    n_hist, T, d = hist.shape
    n_q = q.shape[0]
    _require(q, "q", dtype=torch.float32, shape=(n_q, T, d))
    odt = _dtype_code(hist) if out_dtype is None else (F32 if out_dtype == torch.float32 else BF16)
    if out is None:
        out = torch.empty((n_q, T, d), dtype=_torch_dtype(odt), device=hist.device)
    else:
        _require(out, "out", shape=(n_q, T, d))
        odt = _dtype_code(out)
    if lse is None and want_lse:
        lse = torch.empty((n_q, T), dtype=torch.float32, device=hist.device)
    if lse is not None:
        _require(lse, "lse", dtype=torch.float32, shape=(n_q, T))
    _check(_lib.attnres_block_fwd_q(_ptr(hist), _dtype_code(hist), n_hist, T, d, S, _ptr(q),
                                    q_begin, n_q, eps, _ptr(out), odt, _ptr(lse), _stream(hist)))
    return out, lse


def block_phase1(blocks, n_src: int, v, w, *, partial=None, eps: float = 1e-6, rs=None, o=None,
                 lse1=None, out0=None, lse0=None, normed0=None, norm_gain0=None):
    """Model-order Block AttnRes, phase 1: close block n_src-1 into blocks[n_src-1]
    (= partial + v, fp32) and score the group's reads (queries w [n_reads, d])
    against blocks[0 .. n_src-1].  Returns (o, lse1); out0 / lse0 receive the
    group's first read if given."""
    import torch
    # shapes first: the kernel writes blocks[n_src - 1] and rs[n_src - 1], so a
    # wrong n_src or a short rs would write past the tensors
    if blocks.dim() != 3:
        raise ValueError(f"blocks must be [n_blocks, T, d], got shape {tuple(blocks.shape)}")
    n_blocks, T, d = blocks.shape
    if not 1 <= n_src <= n_blocks:
        raise ValueError(f"n_src = {n_src} outside 1 .. blocks.shape[0] = {n_blocks}")
    if rs is not None and (rs.dim() != 2 or rs.shape[0] < n_src or rs.shape[1] != T):
        raise ValueError(f"rs must be [>= n_src = {n_src}, T = {T}], got shape {tuple(rs.shape)}")
    _require(blocks, "blocks", dtype=torch.float32)
    _require(v, "v", shape=(T, d))
    n_reads = w.shape[0]
    _require(w, "w", dtype=torch.float32, shape=(n_reads, d))
    if partial is not None:
        _require(partial, "partial", dtype=torch.float32, shape=(T, d))
    if rs is not None:
        _require(rs, "rs", dtype=torch.float32)
    if o is None:
        o = torch.empty((n_reads, T, d), dtype=torch.float32, device=v.device)
    _require(o, "o", dtype=torch.float32, shape=(n_reads, T, d))
    if lse1 is None:
        lse1 = torch.empty((n_reads, T), dtype=torch.float32, device=v.device)
    _require(lse1, "lse1", dtype=torch.float32, shape=(n_reads, T))
    odt = F32
    if out0 is not None:
        _require(out0, "out0", shape=(T, d))
        odt = _dtype_code(out0)
    if lse0 is not None:
        _require(lse0, "lse0", dtype=torch.float32, shape=(T,))
    if normed0 is not None:
        _require(normed0, "normed0", shape=(T, d))
        if out0 is not None and normed0.dtype != out0.dtype:
            raise TypeError("normed0 must have the dtype of out0")
        odt = _dtype_code(normed0)
        if norm_gain0 is not None:
            _require(norm_gain0, "norm_gain0", dtype=torch.float32, shape=(d,))
    _check(_lib.attnres_block_phase1(_ptr(blocks), n_src, T, d, _ptr(v), _dtype_code(v),
                                     _ptr(partial), _ptr(w), n_reads, eps, _ptr(rs), _ptr(o),
                                     _ptr(lse1), _ptr(out0), odt, _ptr(lse0), _ptr(norm_gain0),
                                     _ptr(normed0), _stream(v)))
    return o, lse1


def block_phase2(v, partial, first_in_block: bool, w, o, lse1, *, eps: float = 1e-6, out=None,
                 out_dtype=None, lse=None, normed=None, norm_gain=None):
    """Model-order Block AttnRes, phase 2: partial += v (in place; = v when
    first_in_block), then merge the partial sum into the read's phase-1 result.
    Returns (out, lse)."""
    import torch
    _require(v, "v")
    T, d = v.shape
    _require(partial, "partial", dtype=torch.float32, shape=(T, d))
    _require(w, "w", dtype=torch.float32, shape=(d,))
    _require(o, "o", dtype=torch.float32, shape=(T, d))
    _require(lse1, "lse1", dtype=torch.float32, shape=(T,))
    odt = _dtype_code(v) if out_dtype is None else (F32 if out_dtype == torch.float32 else BF16)
    if out is None:
        out = torch.empty((T, d), dtype=_torch_dtype(odt), device=v.device)
    else:
        _require(out, "out", shape=(T, d))
        odt = _dtype_code(out)
    if lse is not None:
        _require(lse, "lse", dtype=torch.float32, shape=(T,))
    if normed is not None:
        _require(normed, "normed", dtype=out.dtype, shape=(T, d))
        if norm_gain is not None:
            _require(norm_gain, "norm_gain", dtype=torch.float32, shape=(d,))
    _check(_lib.attnres_block_phase2(_ptr(v), _dtype_code(v), T, d, _ptr(partial),
                                     1 if first_in_block else 0, _ptr(w), _ptr(o), _ptr(lse1), eps,
                                     _ptr(out), odt, _ptr(lse), _ptr(norm_gain), _ptr(normed),
                                     _stream(v)))
    return out, lse


def block_phase1_q(blocks, n_src: int, v, q, *, partial=None, eps: float = 1e-6, rs=None, o=None,
                   lse1=None, out0=None, lse0=None):
    """Model-order phase 1 with per-token queries q [n_reads, T, d] fp32.  With v
    (row closing block n_src-1) it closes the block as block_phase1 does; with
    v=None it only scores the frozen sources blocks[0 .. n_src-1] (no state is
    written).  Returns (o, lse1)."""
    import torch
    if blocks.dim() != 3:
        raise ValueError(f"blocks must be [n_blocks, T, d], got shape {tuple(blocks.shape)}")
    n_blocks, T, d = blocks.shape
    if not 1 <= n_src <= n_blocks:
        raise ValueError(f"n_src = {n_src} outside 1 .. blocks.shape[0] = {n_blocks}")
    if rs is not None and (rs.dim() != 2 or rs.shape[0] < n_src or rs.shape[1] != T):
        raise ValueError(f"rs must be [>= n_src = {n_src}, T = {T}], got shape {tuple(rs.shape)}")
    _require(blocks, "blocks", dtype=torch.float32)
    if v is not None:
        _require(v, "v", shape=(T, d))
    elif partial is not None:
        raise ValueError("partial needs the row v that closes the block")
    n_reads = q.shape[0]
    _require(q, "q", dtype=torch.float32, shape=(n_reads, T, d))
    if partial is not None:
        _require(partial, "partial", dtype=torch.float32, shape=(T, d))
    if rs is not None:
        _require(rs, "rs", dtype=torch.float32)
    dev = blocks.device
    if o is None:
        o = torch.empty((n_reads, T, d), dtype=torch.float32, device=dev)
    _require(o, "o", dtype=torch.float32, shape=(n_reads, T, d))
    if lse1 is None:
        lse1 = torch.empty((n_reads, T), dtype=torch.float32, device=dev)
    _require(lse1, "lse1", dtype=torch.float32, shape=(n_reads, T))
    odt = F32
    if out0 is not None:
        _require(out0, "out0", shape=(T, d))
        odt = _dtype_code(out0)
    if lse0 is not None:
        _require(lse0, "lse0", dtype=torch.float32, shape=(T,))
    _check(_lib.attnres_block_phase1_q(_ptr(blocks), n_src, T, d, _ptr(v),
                                       F32 if v is None else _dtype_code(v), _ptr(partial), _ptr(q),
                                       n_reads, eps, _ptr(rs), _ptr(o), _ptr(lse1), _ptr(out0), odt,
                                       _ptr(lse0), _stream(blocks)))
    return o, lse1


def block_phase2_q(v, partial, first_in_block: bool, q, o, lse1, *, eps: float = 1e-6, out=None,
                   out_dtype=None, lse=None):
    """Model-order phase 2 with a per-token query q [T, d] fp32.  Returns (out, lse)."""
    import torch
    _require(v, "v")
    T, d = v.shape
    _require(partial, "partial", dtype=torch.float32, shape=(T, d))
    _require(q, "q", dtype=torch.float32, shape=(T, d))
    _require(o, "o", dtype=torch.float32, shape=(T, d))
    _require(lse1, "lse1", dtype=torch.float32, shape=(T,))
    odt = _dtype_code(v) if out_dtype is None else (F32 if out_dtype == torch.float32 else BF16)
    if out is None:
        out = torch.empty((T, d), dtype=_torch_dtype(odt), device=v.device)
    else:
        _require(out, "out", shape=(T, d))
        odt = _dtype_code(out)
    if lse is not None:
        _require(lse, "lse", dtype=torch.float32, shape=(T,))
    _check(_lib.attnres_block_phase2_q(_ptr(v), _dtype_code(v), T, d, _ptr(partial),
                                       1 if first_in_block else 0, _ptr(q), _ptr(o), _ptr(lse1),
                                       eps, _ptr(out), odt, _ptr(lse), _stream(v)))
    return out, lse


def block_model_order(hist, w, S: int, *, eps: float = 1e-6, out=None, lse=None, state=None,
                      normed=None, norm_gain=None):
    """All reads of a Block AttnRes history in model order through the two
    phase entry points (one phase-1 call per block group, one phase-2 call per
    row inside a block), as a model's forward runs them.  `state` may carry
    preallocated buffers (dict with blocks, partial, rs, o, lse1).  Returns
    (out [n_hist, T, d], lse [n_hist, T]).  normed (like out) receives the
    fused pre-norm of every read when given (norm_gain [n_hist, d] or None)."""
    import torch
    _require(hist, "hist")
    n_hist, T, d = hist.shape
    _require(w, "w", dtype=torch.float32, shape=(n_hist, d))
    dev = hist.device
    n_blk = 1 + (n_hist - 1) // S
    st = state if state is not None else {}
    blocks = st.get("blocks")
    if blocks is None:
        blocks = torch.empty((n_blk, T, d), dtype=torch.float32, device=dev)
    partial = st.get("partial")
    if partial is None:
        partial = torch.empty((T, d), dtype=torch.float32, device=dev)
    rs = st.get("rs")
    if rs is None:
        rs = torch.empty((n_blk, T), dtype=torch.float32, device=dev)
    o = st.get("o")
    if o is None:
        o = torch.empty((S, T, d), dtype=torch.float32, device=dev)
    lse1 = st.get("lse1")
    if lse1 is None:
        lse1 = torch.empty((S, T), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty_like(hist)
    if lse is None:
        lse = torch.empty((n_hist, T), dtype=torch.float32, device=dev)
    for m in range(n_blk):
        l0 = m * S
        n_reads = min(S, n_hist - l0)
        ng = (lambda l: None) if norm_gain is None else (lambda l: norm_gain[l])
        nd = (lambda l: None) if normed is None else (lambda l: normed[l])
        block_phase1(blocks[: m + 1], m + 1, hist[l0], w[l0: l0 + n_reads],
                     partial=partial if (m > 0 and S > 1) else None, eps=eps, rs=rs[: m + 1],
                     o=o[:n_reads], lse1=lse1[:n_reads], out0=out[l0], lse0=lse[l0],
                     normed0=nd(l0), norm_gain0=ng(l0))
        for k in range(1, n_reads):
            block_phase2(hist[l0 + k], partial, k == 1, w[l0 + k], o[k], lse1[k], eps=eps,
                         out=out[l0 + k], lse=lse[l0 + k], normed=nd(l0 + k),
                         norm_gain=ng(l0 + k))
    return out, lse


def block_model_order_q(hist, W, S: int, *, eps: float = 1e-6, out=None, lse=None):
    """All reads of a Block AttnRes history in model order with the
    input-dependent query: read l projects the newest row, q_l = W[l] v_l
    (query_proj on the matrix cores), then runs one phase-1 call over the
    frozen sources (closing block l / S when l is a multiple of S) and, inside
    a block, one phase-2 call that adds row l to the partial sum and merges
    it.  hist bf16 [n_hist, T, d], W bf16 [n_hist, d, d].  Returns (out, lse)."""
    import torch
    _require(hist, "hist", dtype=torch.bfloat16)
    n_hist, T, d = hist.shape
    _require(W, "W", dtype=torch.bfloat16, shape=(n_hist, d, d))
    dev = hist.device
    n_blk = 1 + (n_hist - 1) // S
    blocks = torch.empty((n_blk, T, d), dtype=torch.float32, device=dev)
    partial = torch.empty((T, d), dtype=torch.float32, device=dev)
    rs = torch.empty((n_blk, T), dtype=torch.float32, device=dev)
    o = torch.empty((1, T, d), dtype=torch.float32, device=dev)
    lse1 = torch.empty((1, T), dtype=torch.float32, device=dev)
    q = torch.empty((1, T, d), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty_like(hist)
    if lse is None:
        lse = torch.empty((n_hist, T), dtype=torch.float32, device=dev)
    for l in range(n_hist):
        m, k = divmod(l, S)
        query_proj(hist[l:l + 1], W[l:l + 1], q=q)
        if k == 0:
            block_phase1_q(blocks[: m + 1], m + 1, hist[l], q,
                           partial=partial if (m > 0 and S > 1) else None, eps=eps,
                           rs=rs[: m + 1], o=o, lse1=lse1, out0=out[l], lse0=lse[l])
        else:
            block_phase1_q(blocks[: m + 1], m + 1, None, q, eps=eps, rs=rs[: m + 1], o=o,
                           lse1=lse1)
            block_phase2_q(hist[l], partial, k == 1, q[0], o[0], lse1[0], eps=eps, out=out[l],
                           lse=lse[l])
    return out, lse


def bwd_workspace_bytes(variant: int, S: int, n_hist: int, T: int, d: int, q_begin: int,
                        n_q: int) -> int:
    return int(_lib.attnres_bwd_workspace_bytes(variant, S, n_hist, T, d, q_begin, n_q))


def bwd(variant: int, hist, w, dout, *, S: int = 1, q_begin: int = 0, eps: float = 1e-6,
        dhist=None, dhist_dtype=None, dw=None, workspace=None, accumulate: bool = False):
    """Gradients of sum(out * dout) w.r.t. hist and w for the reads
    q_begin .. q_begin + n_q - 1 (n_q = dout.shape[0]).  Returns (dhist, dw).
    accumulate=True adds them into the given fp32 dhist and dw instead."""
    import torch
    if accumulate and (dhist is None or dw is None):
        raise ValueError("accumulate=True needs the dhist and dw to add into")
    _require(hist, "hist")
    n_hist, T, d = hist.shape
    n_q = dout.shape[0]
    _require(w, "w", dtype=torch.float32, shape=(n_q, d))
    _require(dout, "dout", shape=(n_q, T, d))
    ddt = _dtype_code(hist) if dhist_dtype is None else (F32 if dhist_dtype == torch.float32 else BF16)
    if dhist is None:
        dhist = torch.empty((n_hist, T, d), dtype=_torch_dtype(ddt), device=hist.device)
    else:
        _require(dhist, "dhist", shape=(n_hist, T, d))
        ddt = _dtype_code(dhist)
    if dw is None:
        dw = torch.empty((n_q, d), dtype=torch.float32, device=hist.device)
    _require(dw, "dw", dtype=torch.float32, shape=(n_q, d))
    need = bwd_workspace_bytes(variant, S, n_hist, T, d, q_begin, n_q)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=hist.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.attnres_bwd(variant, S, _ptr(hist), _dtype_code(hist), n_hist, T, d, _ptr(w),
                            q_begin, n_q, eps, _ptr(dout), _dtype_code(dout),
                            _ptr(dhist), ddt, 1 if accumulate else 0, _ptr(dw), _ptr(workspace),
                            ws_bytes, _stream(hist)))
    return dhist, dw


def bwd_noalloc(variant: int, hist, w, dout, dhist, dw, *, S: int = 1, q_begin: int = 0,
                eps: float = 1e-6, accumulate: bool = False):
    """attnres_bwd_noalloc: as bwd, into the caller's dhist and dw, with the
    library's static device workspace (no allocation, in the binding either).
    Returns (dhist, dw)."""
    import torch
    _require(hist, "hist")
    n_hist, T, d = hist.shape
    n_q = dout.shape[0]
    _require(w, "w", dtype=torch.float32, shape=(n_q, d))
    _require(dout, "dout", shape=(n_q, T, d))
    _require(dhist, "dhist", shape=(n_hist, T, d))
    _require(dw, "dw", dtype=torch.float32, shape=(n_q, d))
    _check(_lib.attnres_bwd_noalloc(variant, S, _ptr(hist), _dtype_code(hist), n_hist, T, d,
                                    _ptr(w), q_begin, n_q, eps, _ptr(dout), _dtype_code(dout),
                                    _ptr(dhist), _dtype_code(dhist), 1 if accumulate else 0,
                                    _ptr(dw), _stream(hist)))
    return dhist, dw


def bwd_noalloc_max_workspace() -> int:
    return int(_lib.attnres_bwd_noalloc_max_workspace())


def block_index_table(n_hist: int, S: int, q_begin: int = 0, n_q: int | None = None) -> np.ndarray:
    """[n_q, 3] int32: (completed blocks, partial begin row, partial end row)."""
    n_q = n_hist - q_begin if n_q is None else n_q
    out = np.zeros((max(n_q, 0), 3), dtype=np.int32)
    _check(_lib.attnres_block_index_table(n_hist, S, q_begin, n_q,
                                          out.ctypes.data_as(ctypes.c_void_p)))
    return out


def raw():
    """The ctypes handle of the C library (for tests of the raw ABI)."""
    return _lib
