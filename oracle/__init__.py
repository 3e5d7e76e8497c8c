"""fp64 CPU oracle for the AttnRes depth aggregation -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The GPU library never calls it, and it
shares no code with the GPU library: the arithmetic lives in
``attnres_oracle.c`` (plain C, double precision, one token per OpenMP
iteration), this file only marshals numpy arrays.

What the oracle computes, with citations of the pages, is stated in the header
of ``attnres_oracle.c``.  In short, for read ``l`` and token ``t``:
``h = sum_x softmax_x(r(x) * w_l.x) * x`` over the read's sources, with
``r(x) = 1/sqrt(mean(x^2) + eps)``.

Every function takes numpy arrays of any float dtype; values are upcast to
float64 exactly (bf16 and fp32 values are float64-representable).  Tensors use
the library's layouts: ``hist [n_hist, T, d]``, ``w [n_q, d]``,
``out [n_q, T, d]``, ``lse [n_q, T]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attnres_oracle.c")
LIBRARY = os.path.join(_HERE, "libattnres_oracle.so")

FULL = 0
BLOCK = 1

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-Wextra", "-shared",
           "-fPIC", "-o", LIBRARY + ".tmp", SOURCE, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        build()
    lib = ctypes.CDLL(LIBRARY)
    i64, dbl, ip = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    vp = ctypes.c_void_p
    lib.attnres_oracle_num_threads.restype = ip
    lib.attnres_oracle_num_threads.argtypes = []
    lib.attnres_oracle_set_num_threads.restype = None
    lib.attnres_oracle_set_num_threads.argtypes = [ip]
    lib.attnres_oracle_block_sources.restype = None
    lib.attnres_oracle_block_sources.argtypes = [i64, i64, ctypes.POINTER(i64),
                                                 ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.attnres_oracle_num_sources.restype = i64
    lib.attnres_oracle_num_sources.argtypes = [ip, i64, i64]
    lib.attnres_oracle_fwd.restype = ip
    lib.attnres_oracle_fwd.argtypes = [ip, i64, vp, i64, i64, i64, vp, i64, i64, dbl,
                                       vp, vp, vp]
    lib.attnres_oracle_block_fwd_twophase.restype = ip
    lib.attnres_oracle_block_fwd_twophase.argtypes = [i64, vp, i64, i64, i64, vp, i64,
                                                      i64, dbl, vp, vp]
    lib.attnres_oracle_fwd_tokq.restype = ip
    lib.attnres_oracle_fwd_tokq.argtypes = [ip, i64, vp, i64, i64, i64, vp, i64, i64, dbl, vp, vp]
    lib.attnres_oracle_query_proj.restype = ip
    lib.attnres_oracle_query_proj.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.attnres_oracle_prenorm.restype = ip
    lib.attnres_oracle_prenorm.argtypes = [vp, i64, i64, i64, vp, dbl, vp]
    lib.attnres_oracle_bwd.restype = ip
    lib.attnres_oracle_bwd.argtypes = [ip, i64, vp, i64, i64, i64, vp, i64, i64, dbl,
                                       vp, vp, vp]
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS or all cores)."""
    return int(_load().attnres_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the following oracle calls (used to time it on one core)."""
    _load().attnres_oracle_set_num_threads(int(n))


def block_sources(l: int, S: int) -> tuple[int, int, int]:
    """(completed blocks m, partial-sum rows [begin, end)) seen by read ``l``."""
    lib = _load()
    m, b, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    lib.attnres_oracle_block_sources(int(l), int(S), ctypes.byref(m), ctypes.byref(b),
                                     ctypes.byref(e))
    return m.value, b.value, e.value


def num_sources(variant: int, l: int, S: int = 1) -> int:
    return int(_load().attnres_oracle_num_sources(int(variant), int(l), int(S)))


def _check_shapes(hist, w, q_begin, n_q):
    if hist.ndim != 3 or w.ndim != 2:
        raise ValueError("hist must be [n_hist, T, d] and w [n_q, d]")
    n_hist, T, d = hist.shape
    if n_q is None:
        n_q = n_hist - q_begin
    if w.shape != (n_q, d):
        raise ValueError(f"w has shape {w.shape}, expected {(n_q, d)}")
    return n_hist, T, d, n_q


def fwd(variant: int, hist, w, *, S: int = 1, q_begin: int = 0, n_q: int | None = None,
        eps: float = 1e-6, want_alpha: bool = False):
    """Single-pass forward.  Returns (out, lse) or (out, lse, alpha)."""
    hist, w = _f64(hist), _f64(w)
    n_hist, T, d, n_q = _check_shapes(hist, w, q_begin, n_q)
    out = np.zeros((n_q, T, d), np.float64)
    lse = np.zeros((n_q, T), np.float64)
    alpha = np.zeros((n_q, T, n_hist), np.float64) if want_alpha else None
    rc = _load().attnres_oracle_fwd(variant, S, _ptr(hist), n_hist, T, d, _ptr(w), q_begin,
                                    n_q, float(eps), _ptr(out), _ptr(lse), _ptr(alpha))
    if rc != 0:
        raise ValueError("oracle fwd rejected its arguments")
    return (out, lse, alpha) if want_alpha else (out, lse)


def full_fwd(hist, w, **kw):
    return fwd(FULL, hist, w, **kw)


def block_fwd(hist, w, S: int, **kw):
    return fwd(BLOCK, hist, w, S=S, **kw)


def fwd_tokq(variant: int, hist, q, *, S: int = 1, q_begin: int = 0, eps: float = 1e-6):
    """Forward with a query per (read, token): q [n_q, T, d].  Returns (out, lse)."""
    hist, q = _f64(hist), _f64(q)
    n_hist, T, d = hist.shape
    n_q = q.shape[0]
    if q.shape != (n_q, T, d) or q_begin < 0 or q_begin + n_q > n_hist:
        raise ValueError("q must be [n_q, T, d] with q_begin + n_q <= n_hist")
    out = np.zeros((n_q, T, d), np.float64)
    lse = np.zeros((n_q, T), np.float64)
    rc = _load().attnres_oracle_fwd_tokq(variant, S, _ptr(hist), n_hist, T, d, _ptr(q), q_begin,
                                         n_q, float(eps), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle fwd_tokq rejected its arguments")
    return out, lse


def query_proj(x, W) -> np.ndarray:
    """q[j, t] = W[j] @ x[j, t] in fp64: x [n_q, T, d], W [n_q, d, d]."""
    x, W = _f64(x), _f64(W)
    n_q, T, d = x.shape
    if W.shape != (n_q, d, d):
        raise ValueError("W must be [n_q, d, d]")
    q = np.zeros_like(x)
    if _load().attnres_oracle_query_proj(_ptr(x), _ptr(W), n_q, T, d, _ptr(q)) != 0:
        raise ValueError("oracle query_proj rejected its arguments")
    return q


def prenorm(z, gain=None, eps: float = 1e-6) -> np.ndarray:
    """Pre-norm of read mixtures z [n_q, T, d]: gain[l] * z * r(z) with the
    keys' RMSNorm (gain [n_q, d] or None for unit gain), fp64."""
    z = _f64(z)
    n_q, T, d = z.shape
    g = None if gain is None else _f64(gain)
    if g is not None and g.shape != (n_q, d):
        raise ValueError("gain must be [n_q, d]")
    y = np.zeros_like(z)
    if _load().attnres_oracle_prenorm(_ptr(z), n_q, T, d, _ptr(g), float(eps), _ptr(y)) != 0:
        raise ValueError("oracle prenorm rejected its arguments")
    return y


def block_fwd_twophase(hist, w, S: int, *, q_begin: int = 0, n_q: int | None = None,
                       eps: float = 1e-6):
    """Two-phase Block forward (phase 1 over frozen sources, LSE merge of the
    partial sum).  Returns (out, lse)."""
    hist, w = _f64(hist), _f64(w)
    n_hist, T, d, n_q = _check_shapes(hist, w, q_begin, n_q)
    out = np.zeros((n_q, T, d), np.float64)
    lse = np.zeros((n_q, T), np.float64)
    rc = _load().attnres_oracle_block_fwd_twophase(S, _ptr(hist), n_hist, T, d, _ptr(w),
                                                   q_begin, n_q, float(eps), _ptr(out),
                                                   _ptr(lse))
    if rc != 0:
        raise ValueError("oracle two-phase fwd rejected its arguments")
    return out, lse


def bwd(variant: int, hist, w, dout, *, S: int = 1, q_begin: int = 0,
        eps: float = 1e-6):
    """Gradients (dhist [n_hist, T, d], dw [n_q, d]) of sum(out * dout)."""
    hist, w, dout = _f64(hist), _f64(w), _f64(dout)
    n_hist, T, d, n_q = _check_shapes(hist, w, q_begin, None if dout.ndim != 3 else dout.shape[0])
    if dout.shape != (n_q, T, d):
        raise ValueError("dout must be [n_q, T, d]")
    dhist = np.zeros((n_hist, T, d), np.float64)
    dw = np.zeros((n_q, d), np.float64)
    rc = _load().attnres_oracle_bwd(variant, S, _ptr(hist), n_hist, T, d, _ptr(w), q_begin,
                                    n_q, float(eps), _ptr(dout), _ptr(dhist), _ptr(dw))
    if rc != 0:
        raise ValueError("oracle bwd rejected its arguments")
    return dhist, dw


# ---------------------------------------------------------------------------
# Rounding of fp64 results to the library's output dtypes (for reporting the
# fraction of GPU outputs that equal the correctly rounded oracle value).

def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64.  Exact single rounding from float64 (no float32 intermediate)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    ax = np.abs(x[finite])
    m, e = np.frexp(ax)                     # ax = m * 2**e, m in [0.5, 1)
    # bf16 has 8 significant bits; below 2**-126 the spacing stays 2**-133
    e = np.maximum(e, -125)
    ulp = np.ldexp(1.0, e - 8)
    q = ax / ulp                            # exact: power-of-two scaling
    fl = np.floor(q)
    rem = q - fl
    up = (rem > 0.5) | ((rem == 0.5) & (np.fmod(fl, 2.0) == 1.0))
    r = (fl + up) * ulp
    r = np.where(r >= 2.0 ** 128, np.inf, r)  # overflow rounds to infinity
    out[finite] = np.copysign(r, x[finite])
    out[~finite] = x[~finite]
    return out


def ulp_bf16(x) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (one unit in the last place)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)
    e = np.maximum(e, -125)
    return np.ldexp(1.0, e - 8)
