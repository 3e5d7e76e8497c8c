"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects every invalid argument on the host before touching the GPU.
No compute call is made here (there is no GPU in this container)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnres.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIPERR = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1

# fake, well-aligned device addresses: validation never dereferences them
P = 1 << 20
P2 = 2 << 20
P3 = 3 << 20


@pytest.fixture(scope="module")
def ar():
    import depth_wise_attention_attnres_amd as ar
    return ar


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(attnres_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for name in ["attnres_full_fwd", "attnres_block_fwd", "attnres_bwd"]:
        assert name in syms


def test_library_exports_every_declared_symbol(ar):
    lib = ctypes.CDLL(ar.LIBRARY)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert sorted(ar.EXPORTS) == declared_symbols()


def _full(ar, hist=P, hdt=BF16, n_hist=4, T=16, d=64, w=P2, q_begin=0, n_q=4, eps=1e-6,
          rinv=None, rvalid=0, out=P3, odt=BF16, lse=None, gain=None, normed=None, alpha=None):
    return ar.raw().attnres_full_fwd(hist, hdt, n_hist, T, d, w, q_begin, n_q, eps, rinv, rvalid,
                                     out, odt, lse, gain, normed, alpha, None)


def test_full_fwd_validation(ar):
    assert _full(ar, d=12) == ALIGN
    assert "multiple of 8" in ar.last_error()
    assert _full(ar, d=0) == INVALID
    assert _full(ar, d=8192) == UNSUPPORTED
    assert _full(ar, n_hist=0) == INVALID
    assert _full(ar, T=-1) == INVALID
    assert _full(ar, q_begin=1, n_q=4) == INVALID
    assert "outside the history" in ar.last_error()
    assert _full(ar, q_begin=-1) == INVALID
    assert _full(ar, n_q=-1) == INVALID
    assert _full(ar, hdt=7) == INVALID
    assert _full(ar, odt=3) == INVALID
    assert _full(ar, hist=None) == INVALID
    assert _full(ar, w=None) == INVALID
    assert _full(ar, out=None) == INVALID
    assert _full(ar, hist=P + 8) == ALIGN
    assert _full(ar, w=P2 + 4) == ALIGN
    assert _full(ar, out=P3 + 2) == ALIGN
    assert _full(ar, lse=P + 2) == ALIGN
    assert _full(ar, rinv=P + 1, rvalid=0) == ALIGN
    assert _full(ar, rinv=None, rvalid=2) == INVALID
    assert _full(ar, rinv=P, rvalid=5) == INVALID
    assert _full(ar, eps=-1.0) == INVALID
    assert _full(ar, eps=float("inf")) == INVALID
    assert _full(ar, eps=float("nan")) == INVALID
    assert _full(ar, T=1 << 40) == UNSUPPORTED
    assert _full(ar, normed=P + 8) == ALIGN
    assert _full(ar, normed=P, gain=P2 + 4) == ALIGN
    assert _full(ar, alpha=P + 2) == ALIGN
    assert _full(ar, T=1 << 22, d=8, n_hist=1, n_q=1) == UNSUPPORTED
    assert "2^22" in ar.last_error()
    assert _full(ar, T=(1 << 22) - 1, d=8, n_hist=1, n_q=1, hist=None) == INVALID  # size accepted


def test_empty_calls_launch_nothing(ar):
    # T == 0 or n_q == 0: valid, returns before any HIP call
    assert _full(ar, T=0) == OK
    assert _full(ar, n_q=0) == OK
    assert _full(ar, T=0, hist=None, w=None, out=None) == OK
    assert ar.last_error() == ""
    assert ar.raw().attnres_block_fwd(P, BF16, 4, 0, 64, 2, P2, 0, 4, 1e-6, P3, BF16, None,
                                      None, None) == OK


def test_block_fwd_validation(ar):
    lib = ar.raw()
    assert lib.attnres_block_fwd(P, BF16, 9, 16, 64, 0, P2, 0, 9, 1e-6, P3, BF16, None, None, None) == INVALID
    assert "S must be" in ar.last_error()
    assert lib.attnres_block_fwd(P, BF16, 9, 16, 60, 2, P2, 0, 9, 1e-6, P3, BF16, None, None, None) == ALIGN
    assert lib.attnres_block_fwd(P, BF16, 9, 16, 64, 2, P2, 5, 9, 1e-6, P3, BF16, None, None, None) == INVALID
    assert lib.attnres_block_fwd(P, BF16, 9, 16, 64, 2, P2, 0, 9, 1e-6, None, BF16, None, None, None) == INVALID
    assert lib.attnres_block_fwd(P, BF16, 9, 16, 64, 2, P2, 0, 9, 1e-6, P3 + 4, BF16, None, None, None) == ALIGN


def test_status_strings(ar):
    for code, name in ar.STATUS.items():
        assert ar.status_string(code).startswith(name)
    assert "unknown" in ar.status_string(99)


def test_last_error_is_thread_local(ar):
    import threading
    assert _full(ar, d=12) == ALIGN
    seen = {}

    def other():
        seen["msg"] = ar.last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "multiple of 8" in ar.last_error()


# ---------------------------------------------------------------------------
# Block index table: bit-exact against the oracle's independent indexing

@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 8, 16, 64, 100])
def test_block_index_table_matches_oracle(ar, oracle, S):
    n_hist = 141
    tab = ar.block_index_table(n_hist, S)
    assert tab.dtype == np.int32 and tab.shape == (n_hist, 3)
    for l in range(n_hist):
        assert tuple(int(x) for x in tab[l]) == oracle.block_sources(l, S), (S, l)
    sub = ar.block_index_table(n_hist, S, q_begin=37, n_q=20)
    assert np.array_equal(sub, tab[37:57])


def test_block_index_table_validation(ar):
    lib = ar.raw()
    buf = (ctypes.c_int32 * 30)()
    assert lib.attnres_block_index_table(10, 0, 0, 10, buf) == INVALID
    assert lib.attnres_block_index_table(10, 2, 5, 6, buf) == INVALID
    assert lib.attnres_block_index_table(10, 2, 0, 10, None) == INVALID
    assert lib.attnres_block_index_table(10, 2, 0, 0, None) == OK


def _bwd(ar, variant=0, S=1, hist=P, hdt=BF16, n_hist=4, T=16, d=64, w=P2, q_begin=0, n_q=4,
         eps=1e-6, dout=P, gdt=BF16, dhist=P2, ddt=BF16, acc=0, dw=P3, ws=P, ws_bytes=1 << 40):
    return ar.raw().attnres_bwd(variant, S, hist, hdt, n_hist, T, d, w, q_begin, n_q, eps,
                                dout, gdt, dhist, ddt, acc, dw, ws, ws_bytes, None)


def test_bwd_validation(ar):
    assert _bwd(ar, variant=2) == INVALID
    assert _bwd(ar, variant=1, S=0) == INVALID
    assert _bwd(ar, d=12) == ALIGN
    assert _bwd(ar, q_begin=2) == INVALID
    assert _bwd(ar, dout=None) == INVALID
    assert "dout" in ar.last_error()
    assert _bwd(ar, dhist=None) == INVALID
    assert _bwd(ar, dw=None) == INVALID
    assert _bwd(ar, gdt=5) == INVALID
    assert _bwd(ar, ddt=5) == INVALID
    assert _bwd(ar, dhist=P2 + 8) == ALIGN
    assert _bwd(ar, ws=None) == WORKSPACE
    assert _bwd(ar, ws_bytes=16) == WORKSPACE
    assert "needed" in ar.last_error()
    assert _bwd(ar, ws=P + 64) == ALIGN
    assert _bwd(ar, T=0) == OK
    assert _bwd(ar, acc=2) == INVALID
    assert _bwd(ar, acc=1) == INVALID  # accumulating needs an fp32 dhist
    assert "fp32" in ar.last_error()
    assert _bwd(ar, acc=1, ddt=F32, T=0) == OK


def test_bwd_workspace_size(ar):
    lib = ar.raw()
    full = lib.attnres_bwd_workspace_bytes(0, 1, 49, 16384, 1024, 0, 49)
    block = lib.attnres_bwd_workspace_bytes(1, 4, 49, 16384, 1024, 0, 49)
    assert full > 0 and block > 0 and full % 256 == 0
    # Full ignores S; Block with S = 1 needs the same layout as Full
    assert lib.attnres_bwd_workspace_bytes(0, 7, 49, 16384, 1024, 0, 49) == full
    assert lib.attnres_bwd_workspace_bytes(1, 1, 49, 16384, 1024, 0, 49) == full
    assert lib.attnres_bwd_workspace_bytes(0, 1, 49, 16384, 1024, 10, 49) == 0  # reads past the history
    assert lib.attnres_bwd_workspace_bytes(2, 1, 49, 16384, 1024, 0, 49) == 0


def test_block_phase_validation(ar):
    lib = ar.raw()
    # blocks, n_src, T, d, v, v_dt, partial, w, n_reads, eps, rs, o, lse1, out0, out_dt, lse0, stream
    def ph1(blocks=P, n_src=3, T=16, d=64, v=P2, vdt=BF16, partial=None, w=P3, n_reads=4, eps=1e-6,
            rs=None, o=P, lse1=P2, out0=None, odt=BF16, lse0=None, g0=None, n0=None):
        return lib.attnres_block_phase1(blocks, n_src, T, d, v, vdt, partial, w, n_reads, eps, rs, o,
                                        lse1, out0, odt, lse0, g0, n0, None)
    assert ph1(n_src=0) == INVALID
    assert ph1(n_src=14) == UNSUPPORTED
    assert ph1(n_reads=0) == INVALID
    assert ph1(n_reads=65) == UNSUPPORTED
    assert ph1(d=12) == ALIGN
    assert ph1(blocks=None) == INVALID
    assert ph1(o=None) == INVALID
    assert ph1(lse1=None) == INVALID
    assert ph1(v=None) == INVALID
    assert ph1(w=None) == INVALID
    assert ph1(partial=P + 8) == ALIGN
    assert ph1(out0=P + 4) == ALIGN
    assert ph1(rs=P + 2) == ALIGN
    assert ph1(odt=9) == INVALID
    assert ph1(T=0) == OK
    assert ph1(n0=P + 4) == ALIGN

    def ph2(v=P, vdt=BF16, T=16, d=64, partial=P2, first=1, w=P3, o=P, lse1=P2, eps=1e-6, out=P3,
            odt=BF16, lse=None, g=None, nrm=None):
        return lib.attnres_block_phase2(v, vdt, T, d, partial, first, w, o, lse1, eps, out, odt, lse,
                                        g, nrm, None)
    assert ph2(first=2) == INVALID
    assert ph2(partial=None) == INVALID
    assert ph2(o=None) == INVALID
    assert ph2(lse1=None) == INVALID
    assert ph2(out=None) == INVALID
    assert ph2(out=P3 + 2) == ALIGN
    assert ph2(d=4) == ALIGN
    assert ph2(eps=float("nan")) == INVALID
    assert ph2(T=0) == OK
    assert ph2(nrm=P + 4) == ALIGN
    assert ph2(nrm=P, g=P2 + 8) == ALIGN


def test_query_proj_and_full_fwd_q_validation(ar):
    lib = ar.raw()
    # x, x_dt, n_q, T, d, W, w_dt, q, stream
    assert lib.attnres_query_proj(P, F32, 2, 16, 64, P2, BF16, P3, None) == UNSUPPORTED
    assert lib.attnres_query_proj(P, BF16, 2, 16, 64, P2, F32, P3, None) == UNSUPPORTED
    assert lib.attnres_query_proj(P, BF16, 2, 16, 60, P2, BF16, P3, None) == ALIGN
    assert lib.attnres_query_proj(P, BF16, 2, 16, 8192, P2, BF16, P3, None) == UNSUPPORTED
    assert lib.attnres_query_proj(P, BF16, 2, 16, 64, None, BF16, P3, None) == INVALID
    assert lib.attnres_query_proj(P, BF16, 2, 16, 64, P2, BF16, P3 + 4, None) == ALIGN
    assert lib.attnres_query_proj(P, BF16, 0, 16, 64, None, BF16, None, None) == OK
    assert lib.attnres_query_proj(P, 7, 2, 16, 64, P2, BF16, P3, None) == INVALID
    # one launch: at most 2^23 tiles of 256 x 256 (2^32 work-items), and T < 2^22
    assert lib.attnres_query_proj(P, BF16, 64, 1 << 21, 4096, P2, BF16, P3, None) == UNSUPPORTED
    assert "tiles" in ar.last_error()
    assert lib.attnres_query_proj(P, BF16, 1, 1 << 22, 64, P2, BF16, P3, None) == UNSUPPORTED
    assert "2^22" in ar.last_error()
    # hist, dt, n_hist, T, d, q, q_begin, n_q, eps, rinv, rvalid, out, out_dt, lse, stream
    assert lib.attnres_full_fwd_q(P, BF16, 4, 16, 64, None, 0, 4, 1e-6, None, 0, P3, BF16, None,
                                  None) == INVALID
    assert lib.attnres_full_fwd_q(P, BF16, 4, 16, 64, P2 + 4, 0, 4, 1e-6, None, 0, P3, BF16, None,
                                  None) == ALIGN
    assert lib.attnres_full_fwd_q(P, BF16, 4, 16, 64, P2, 1, 4, 1e-6, None, 0, P3, BF16, None,
                                  None) == INVALID
    assert lib.attnres_full_fwd_q(P, BF16, 4, 0, 64, P2, 0, 4, 1e-6, None, 0, P3, BF16, None,
                                  None) == OK


def test_package_fails_loudly_without_the_library(tmp_path):
    # a copy of the package without libattnres.so must refuse to import (there
    # is no CPU fallback)
    import shutil
    import subprocess
    import sys
    src = os.path.join(ROOT, "depth_wise_attention_attnres_amd")
    dst = tmp_path / "depth_wise_attention_attnres_amd"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.so", "csrc", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import depth_wise_attention_attnres_amd"],
                       cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "not built" in r.stderr


def test_block_phase1_binding_rejects_bad_n_src_and_rs(ar):
    # the kernel writes blocks[n_src - 1] and rs[n_src - 1]: the binding checks
    # both shapes before anything reaches the library (CPU tensors suffice,
    # the shape checks come before the device check)
    import torch
    blocks = torch.zeros((3, 4, 16))
    v = torch.zeros((4, 16))
    w = torch.zeros((2, 16))
    with pytest.raises(ValueError, match="n_src"):
        ar.block_phase1(blocks, 4, v, w)
    with pytest.raises(ValueError, match="n_src"):
        ar.block_phase1(blocks, 0, v, w)
    with pytest.raises(ValueError, match="rs"):
        ar.block_phase1(blocks, 3, v, w, rs=torch.zeros((2, 4)))
    with pytest.raises(ValueError, match="rs"):
        ar.block_phase1(blocks, 2, v, w, rs=torch.zeros((3, 5)))
    with pytest.raises(ValueError, match="blocks"):
        ar.block_phase1(torch.zeros((4, 16)), 1, v, w)
    # valid shapes get as far as the device check
    with pytest.raises(ValueError, match="GPU"):
        ar.block_phase1(blocks, 3, v, w, rs=torch.zeros((3, 4)))


def test_bwd_binding_accumulate_needs_targets(ar):
    import torch
    h = torch.zeros((3, 4, 16))
    with pytest.raises(ValueError, match="accumulate"):
        ar.bwd(ar.FULL, h, torch.zeros((3, 16)), torch.zeros((3, 4, 16)), accumulate=True)


def test_bwd_noalloc_validation(ar):
    lib = ar.raw()
    assert lib.attnres_bwd_noalloc_max_workspace() == 64 << 20

    def nb(n_hist=4, T=16, d=64, n_q=4, ddt=BF16, acc=0, dout=P, dw=P3):
        return lib.attnres_bwd_noalloc(0, 1, P, BF16, n_hist, T, d, P2, 0, n_q, 1e-6, dout, BF16,
                                       P2, ddt, acc, dw, None)
    assert nb(d=12) == ALIGN
    assert nb(dout=None) == INVALID
    assert nb(acc=1) == INVALID
    assert nb(T=0) == OK
    # a call whose workspace exceeds the static array is refused on the host
    need = lib.attnres_bwd_workspace_bytes(0, 1, 49, 4096, 1024, 0, 49)
    assert need > 64 << 20
    assert nb(n_hist=49, T=4096, d=1024, n_q=49) == UNSUPPORTED
    assert "static scratch" in ar.last_error()


def test_block_q_entry_points_validation(ar):
    lib = ar.raw()

    def bq(n_hist=9, T=16, d=64, S=4, q=P2, q_begin=0, n_q=9, out=P3):
        return lib.attnres_block_fwd_q(P, BF16, n_hist, T, d, S, q, q_begin, n_q, 1e-6, out, BF16,
                                       None, None)
    assert bq(d=12) == ALIGN
    assert bq(S=0) == INVALID
    assert bq(q=None) == INVALID
    assert bq(q=P2 + 4) == ALIGN
    assert bq(out=None) == INVALID
    assert bq(q_begin=3) == INVALID  # reads past the history
    assert bq(T=0) == OK

    def p1(v=P2, partial=None, q=P3, n_src=2, n_reads=1):
        return lib.attnres_block_phase1_q(P, n_src, 16, 64, v, BF16, partial, q, n_reads, 1e-6,
                                          None, P, P2, None, BF16, None, None)
    assert p1(q=None) == INVALID
    assert p1(v=None, partial=P) == INVALID  # a partial sum needs the row closing the block
    assert "partial" in ar.last_error()
    assert p1(n_src=0) == INVALID
    assert p1(n_reads=65) == UNSUPPORTED

    def p2(q=P3, first=1):
        return lib.attnres_block_phase2_q(P, BF16, 16, 64, P, first, q, P2, P3, 1e-6, P, BF16,
                                          None, None)
    assert p2(q=None) == INVALID
    assert p2(first=2) == INVALID
