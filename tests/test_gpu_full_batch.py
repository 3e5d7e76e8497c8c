"""GPU parity of the Full forward for calls with many reads (run on an MI355X).

A call with at least 16 reads is served by the kernel that stages each token's
rows in LDS once (full_batch.hip) when at least two thirds of the rows fit
(the rest are then read from global memory); the shapes below are chosen to
qualify (see ``_qualifies``), covering one to four 16-byte chunks per lane,
ragged last groups of reads (n_q not a multiple of 4), rows past the LDS,
reads that start past row 0, the RMS cache, the fused pre-norm and the weight
probe.  Every output is compared with the fp64 oracle; the full-size
workloads compare a token sample, which is exact per token because tokens are
independent."""
import numpy as np
import pytest
import torch

from parity import check_lse, check_out, check_rel, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LDS_BYTES = 160 * 1024  # LDS a workgroup may hold on this part


@pytest.fixture(scope="module")
def ar():
    import depth_wise_attention_attnres_amd as ar
    return ar


def _lds_rows(n_rows, d, dtype):
    """Rows the library stages in LDS: as many as fit next to the RMS scales,
    8 score tables of 4 floats per row and the group counter."""
    elem = 2 if dtype == "bf16" else 4
    n_pad = (n_rows + 3) // 4 * 4
    room = LDS_BYTES - (4 * n_pad + 8 * 16 * n_pad + 16)
    return min(n_rows, room // (d * elem))


def _qualifies(n_rows, n_q, d, dtype):
    """The rule the library applies: >= 16 reads, <= 4 (bf16) or 3 (fp32)
    chunks of 8 per lane, at least two thirds of the rows in LDS."""
    nch = (d // 8 + 63) // 64
    return (n_q >= 16 and nch <= (4 if dtype == "bf16" else 3)
            and 3 * _lds_rows(n_rows, d, dtype) >= 2 * n_rows)


def _inputs(n_hist, T, d, seed, dtype, w_sigma=0.3):
    rng = np.random.default_rng(seed)
    hist = rng.standard_normal((n_hist, T, d)).astype(np.float32)
    w = (rng.standard_normal((n_hist, d)) * w_sigma).astype(np.float32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    h = torch.from_numpy(hist).to(DEV).to(tdt)
    return h, torch.from_numpy(w).to(DEV), to_f64(h), w.astype(np.float64)


# (n_hist, T, d): chunks per lane 1 (d=64, 200), 2 (520, 896, 1024), 3 (1032), 4 (2048)
SHAPES = [(16, 37, 64), (19, 50, 200), (33, 70, 520), (21, 33, 1032), (18, 9, 2048),
          (65, 40, 896), (49, 24, 1024)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d", SHAPES)
def test_batch_all_reads(ar, oracle, dtype, n_hist, T, d):
    # fp32 at (18, 9, 2048) and (65, 40, 896) does not qualify (the rows do
    # not fit in LDS at 4 bytes): the streaming kernel serves those calls, and
    # they are checked against the oracle all the same
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=n_hist * 31 + d, dtype=dtype)
    out, lse = ar.full_fwd(h, w)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.full_fwd(h64, w64)
    check_out(to_f64(out), ref, dtype)
    check_lse(to_f64(lse), ref_lse)


@pytest.mark.parametrize("dtype,n_hist,T,d", [("bf16", 70, 19, 1536), ("f32", 40, 23, 1032)])
def test_batch_rows_past_lds(ar, oracle, dtype, n_hist, T, d):
    # more rows than LDS holds: the first are staged, the rest (seen only by
    # the last groups of reads) come from global memory in both passes
    n_lds = _lds_rows(n_hist, d, dtype)
    assert _qualifies(n_hist, n_hist, d, dtype) and n_lds < n_hist
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=n_hist + d, dtype=dtype, w_sigma=0.05)
    rinv = torch.empty((n_hist, T), device=DEV)
    normed = torch.empty(h.shape, dtype=h.dtype, device=DEV)
    out = torch.empty_like(normed)
    lse = torch.empty((n_hist, T), device=DEV)
    ar.full_fwd(h, w, out=out, lse=lse, rinv=rinv, normed=normed)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.full_fwd(h64, w64)
    check_out(to_f64(out), ref, dtype)
    check_lse(to_f64(lse), ref_lse)
    check_out(to_f64(normed), oracle.prenorm(ref, None), dtype, what="normed")
    r_ref = 1.0 / np.sqrt((h64 ** 2).mean(axis=2) + 1e-6)
    np.testing.assert_allclose(to_f64(rinv), r_ref, rtol=2e-6)


@pytest.mark.parametrize("hdt,odt", [("bf16", "f32"), ("f32", "bf16")])
def test_batch_mixed_dtypes(ar, oracle, hdt, odt):
    h, w, h64, w64 = _inputs(23, 45, 136, seed=8, dtype=hdt)
    out, _ = ar.full_fwd(h, w, out_dtype=torch.float32 if odt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    ref, _ = oracle.full_fwd(h64, w64)
    check_out(to_f64(out), ref, odt)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batch_q_begin_with_partly_valid_cache(ar, oracle, dtype):
    # reads 5..24 of a 27-row history; rows 0..4 of the RMS cache come from an
    # earlier call, rows 5..24 are formed and written by this one
    n_hist, T, d = 27, 41, 264
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=13, dtype=dtype)
    rinv = torch.full((n_hist, T), float("nan"), device=DEV)
    ar.full_fwd(h, w[:5], q_begin=0, n_q=5, rinv=rinv)
    out, lse = ar.full_fwd(h, w[5:25], q_begin=5, n_q=20, rinv=rinv, rinv_valid_rows=5)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.full_fwd(h64, w64[5:25], q_begin=5, n_q=20)
    check_out(to_f64(out), ref, dtype)
    check_lse(to_f64(lse), ref_lse)
    r = to_f64(rinv)
    assert np.isfinite(r[:25]).all() and np.isnan(r[25:]).all()  # rows past the last read untouched
    r_ref = 1.0 / np.sqrt((h64[:25] ** 2).mean(axis=2) + 1e-6)
    np.testing.assert_allclose(r[:25], r_ref, rtol=2e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_gain", [False, True])
def test_batch_prenorm(ar, oracle, dtype, with_gain):
    n_hist, T, d = 22, 29, 520
    h, w, hd, wd = _inputs(n_hist, T, d, seed=21, dtype=dtype)
    gain = torch.from_numpy(np.random.default_rng(3).uniform(0.5, 1.5, (n_hist, d)).astype(np.float32)).to(DEV) \
        if with_gain else None
    out = torch.empty(h.shape, dtype=h.dtype, device=DEV)
    normed = torch.empty_like(out)
    ar.full_fwd(h, w, out=out, normed=normed, norm_gain=gain)
    torch.cuda.synchronize()
    ref, _ = oracle.full_fwd(hd, wd)
    check_out(to_f64(out), ref, dtype)
    check_out(to_f64(normed), oracle.prenorm(ref, None if gain is None else to_f64(gain)), dtype, what="normed")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("q_begin", [0, 2])
def test_batch_alpha_probe(ar, oracle, dtype, q_begin):
    n_hist, T, d = 21, 31, 264
    h, w, hd, wd = _inputs(n_hist, T, d, seed=17 + q_begin, dtype=dtype, w_sigma=0.05)
    n_q = n_hist - q_begin
    w = w[q_begin:].contiguous()
    alpha = torch.full((n_q, n_hist, T), float("nan"), device=DEV)
    ar.full_fwd(h, w, q_begin=q_begin, alpha=alpha)
    torch.cuda.synchronize()
    _, _, ref = oracle.fwd(oracle.FULL, hd, wd[q_begin:], q_begin=q_begin, want_alpha=True)
    a = to_f64(alpha)
    check_rel(a, ref.transpose(0, 2, 1), 1e-5, "alpha")
    assert (a >= 0).all()
    np.testing.assert_allclose(a.sum(1), 1.0, atol=1e-5)
    for j in range(n_q):
        assert (a[j, q_begin + j + 1:] == 0).all()


def test_batch_agrees_with_model_order(ar, oracle):
    # the batched call and the read-by-read sweep (streaming kernel, RMS cache)
    # compute the same function: both within the bar of the oracle on one input
    n_hist, T, d = 40, 64, 896
    h, w, hd, wd = _inputs(n_hist, T, d, seed=2, dtype="bf16", w_sigma=0.05)
    ob, lb = ar.full_fwd(h, w)
    rinv = torch.empty((n_hist, T), device=DEV)
    om = torch.empty_like(h)
    lm = torch.empty((n_hist, T), device=DEV)
    for l in range(n_hist):
        ar.full_fwd(h, w[l:l + 1], q_begin=l, n_q=1, rinv=rinv, rinv_valid_rows=l,
                    out=om[l:l + 1], lse=lm[l:l + 1])
    torch.cuda.synchronize()
    ref, ref_lse = oracle.full_fwd(hd, wd)
    check_out(to_f64(ob), ref, "bf16")
    check_out(to_f64(om), ref, "bf16")
    check_lse(to_f64(lb), ref_lse)
    check_lse(to_f64(lm), ref_lse)


@pytest.mark.parametrize("name", ["full_L32_d896", "fwdbwd_L24_d1024"])
def test_batch_workload_sampled(ar, oracle, name):
    # the full-size history in one call with every read, a token sample checked
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs, token_sample
    wl = WORKLOADS[name]
    assert _qualifies(wl.n_hist, wl.n_hist, wl.d, wl.dtype)
    h, w, _ = device_inputs(wl, DEV)
    out, lse = ar.full_fwd(h, w)
    torch.cuda.synchronize()
    idx = token_sample(wl.T, 384, seed=wl.seed)
    ti = torch.from_numpy(idx).to(DEV)
    ref, ref_lse = oracle.full_fwd(to_f64(h.index_select(1, ti)), to_f64(w))
    stats = check_out(to_f64(out.index_select(1, ti)), ref, wl.dtype)
    check_lse(to_f64(lse.index_select(1, ti)), ref_lse)
    print(f"{name} batched: {stats}", flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d,q_begin", [(16, 1, 8, 0), (21, 2, 8, 5), (17, 1, 1024, 1)])
def test_batch_edges(ar, oracle, dtype, n_hist, T, d, q_begin):
    # one token, d = 8 (one chunk, 63 idle lanes), exactly 16 reads
    n_q = n_hist - q_begin
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=n_hist + T + d, dtype=dtype)
    out, lse = ar.full_fwd(h, w[q_begin:].contiguous(), q_begin=q_begin, n_q=n_q)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.full_fwd(h64, w64[q_begin:], q_begin=q_begin, n_q=n_q)
    check_out(to_f64(out), ref, dtype)
    check_lse(to_f64(lse), ref_lse)


# ---- the matrix-core kernel (full_batch_mfma.hip) ----------------------------
# bf16 rows and bf16 outputs, d a multiple of 32, at most 96 reads, at most
# 96 / 80 / 48 / 40 rows with 1 / 2 / 3 / 4 chunks of 8 per lane (a token's
# rows are prefetched in registers), no fused pre-norm, and everything in LDS:
# rows (d + 8 bf16 each), the weights' two bf16 parts per read (32 per started
# 32 rows, + 8), two tables of one float per read and row tile, the RMS scales.

def _mfma_lds(n_rows, n_q, d):
    nrb, nks = (n_rows + 15) // 16, (n_rows + 31) // 32
    return (n_rows * (d + 8) * 2 + 2 * n_q * (32 * nks + 8) * 2 + 2 * n_q * nrb * 4
            + (n_rows + 3) // 4 * 4 * 4)


def _mfma_qualifies(n_rows, n_q, d):
    nch = (d // 8 + 63) // 64
    max_rows = {1: 96, 2: 80, 3: 48, 4: 40}.get(nch, 0)
    return (n_q >= 16 and n_q <= 96 and d % 32 == 0 and n_rows <= max_rows
            and _mfma_lds(n_rows, n_q, d) <= LDS_BYTES)


# (n_hist, T, d, q_begin): chunks per lane 1 (d 32, 96), 2 (896), 3 (1536), 4 (2048);
# one read tile and two row tiles (17 rows, 16 reads); ragged read and row tiles
# (33 reads over 40 rows); the maximum of 96 rows and 96 reads; a read tile that
# starts past row 0 sees every row tile
MFMA_SHAPES = [(16, 37, 32, 0), (17, 20, 96, 1), (40, 23, 160, 7), (96, 5, 64, 0),
               (65, 9, 896, 0), (40, 7, 1536, 3), (30, 13, 2048, 0), (70, 6, 256, 38)]


@pytest.mark.parametrize("n_hist,T,d,q_begin", MFMA_SHAPES)
def test_batch_mfma_shapes(ar, oracle, n_hist, T, d, q_begin):
    n_q = n_hist - q_begin
    assert _mfma_qualifies(n_hist, n_q, d)
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=3 * n_hist + d + q_begin, dtype="bf16")
    out, lse = ar.full_fwd(h, w[q_begin:].contiguous(), q_begin=q_begin, n_q=n_q)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.full_fwd(h64, w64[q_begin:], q_begin=q_begin, n_q=n_q)
    stats = check_out(to_f64(out), ref, "bf16")
    check_lse(to_f64(lse), ref_lse)
    # one rounding of an fp32 result: nearly every output is RNE(ref) exactly
    assert stats["frac_equal_rne"] > 0.99, stats


def test_batch_mfma_rows_past_reads_and_cache(ar, oracle):
    # a history longer than the reads see (rows past the last read are never
    # staged); reads 5..36 with rows 0..4 of the RMS cache valid from an
    # earlier call, rows 5..36 formed and written by this one
    n_hist, T, d = 45, 19, 320
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=29, dtype="bf16")
    rinv = torch.full((n_hist, T), float("nan"), device=DEV)
    ar.full_fwd(h, w[:5], q_begin=0, n_q=5, rinv=rinv)
    assert _mfma_qualifies(37, 32, d)
    out, lse = ar.full_fwd(h, w[5:37], q_begin=5, n_q=32, rinv=rinv, rinv_valid_rows=5)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.full_fwd(h64, w64[5:37], q_begin=5, n_q=32)
    check_out(to_f64(out), ref, "bf16")
    check_lse(to_f64(lse), ref_lse)
    r = to_f64(rinv)
    assert np.isfinite(r[:37]).all() and np.isnan(r[37:]).all()
    np.testing.assert_allclose(r[:37], 1.0 / np.sqrt((h64[:37] ** 2).mean(axis=2) + 1e-6), rtol=2e-6)


@pytest.mark.parametrize("q_begin", [0, 3])
def test_batch_mfma_alpha_probe(ar, oracle, q_begin):
    # weights in fp32 from the matrix-core scores; zero past each read's row
    # and for history rows no read of the call sees
    n_hist, T, d = 41, 17, 128
    n_q = 35 - q_begin
    assert _mfma_qualifies(q_begin + n_q, n_q, d)
    h, w, hd, wd = _inputs(n_hist, T, d, seed=47 + q_begin, dtype="bf16", w_sigma=0.05)
    w = w[q_begin:q_begin + n_q].contiguous()
    alpha = torch.full((n_q, n_hist, T), float("nan"), device=DEV)
    out, _ = ar.full_fwd(h, w, q_begin=q_begin, n_q=n_q, alpha=alpha)
    torch.cuda.synchronize()
    ref_out, _, ref = oracle.fwd(oracle.FULL, hd, wd[q_begin:q_begin + n_q], q_begin=q_begin, n_q=n_q,
                                 want_alpha=True)
    a = to_f64(alpha)
    check_rel(a, ref.transpose(0, 2, 1), 1e-5, "alpha")
    np.testing.assert_allclose(a.sum(1), 1.0, atol=1e-5)
    for j in range(n_q):
        assert (a[j, q_begin + j + 1:] == 0).all()
    check_out(to_f64(out), ref_out, "bf16")


# A call with more history rows than the matrix-core kernel stages (80 at two
# chunks per lane): its leading reads go to that kernel, the rest to the
# vector kernel (or, for fewer than 16 remaining reads, the streaming kernel),
# which trusts the RMS cache rows the first part wrote.  Every
# output, lse, weight probe and cache row against the oracle, from read 0 and
# from a later first read, with and without an earlier valid cache prefix.
@pytest.mark.parametrize("n_hist,T,d,q_begin,valid", [(100, 23, 640, 0, 0), (100, 19, 640, 30, 7),
                                                      (141, 6, 640, 0, 0), (90, 17, 640, 0, 3)])
def test_batch_split_between_kernels(ar, oracle, n_hist, T, d, q_begin, valid):
    n_q = n_hist - q_begin
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=n_hist + q_begin, dtype="bf16", w_sigma=0.05)
    rinv = torch.full((n_hist, T), float("nan"), device=DEV)
    if valid:
        ar.full_fwd(h, w[:valid], q_begin=0, n_q=valid, rinv=rinv)
    alpha = torch.full((n_q, n_hist, T), float("nan"), device=DEV)
    out, lse = ar.full_fwd(h, w[q_begin:].contiguous(), q_begin=q_begin, n_q=n_q, rinv=rinv,
                           rinv_valid_rows=valid, alpha=alpha)
    torch.cuda.synchronize()
    ref, ref_lse, ref_a = oracle.fwd(oracle.FULL, h64, w64[q_begin:], q_begin=q_begin, n_q=n_q,
                                     want_alpha=True)
    check_out(to_f64(out), ref, "bf16")
    check_lse(to_f64(lse), ref_lse)
    check_rel(to_f64(alpha), ref_a.transpose(0, 2, 1), 1e-5, "alpha")
    r = to_f64(rinv)
    r_ref = 1.0 / np.sqrt((h64 ** 2).mean(axis=2) + 1e-6)
    np.testing.assert_allclose(r, r_ref, rtol=2e-6)
