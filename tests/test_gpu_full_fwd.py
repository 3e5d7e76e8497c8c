"""GPU parity of attnres_full_fwd against the fp64 oracle (run on an MI355X).

Small cases compare every element; the full-size workloads run in the
launch configuration the benchmark times (one call per read, with the
per-(row, token) RMS cache) and compare a sample of tokens, which is exact
per token because tokens are independent."""
import numpy as np
import pytest
import torch

from parity import check_lse, check_out, check_rel, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ar():
    import depth_wise_attention_attnres_amd as ar
    return ar


def _inputs(n_hist, T, d, seed, dtype, w_sigma=0.3, sigma_growth=False):
    rng = np.random.default_rng(seed)
    scale = np.linspace(1, 8, n_hist)[:, None, None] if sigma_growth else 1.0
    hist = (rng.standard_normal((n_hist, T, d)) * scale).astype(np.float32)
    w = (rng.standard_normal((n_hist, d)) * w_sigma).astype(np.float32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    h = torch.from_numpy(hist).to(DEV).to(tdt)
    return h, torch.from_numpy(w).to(DEV), to_f64(h), w.astype(np.float64)


SHAPES = [(1, 5, 8), (2, 3, 16), (9, 37, 64), (5, 300, 200), (17, 256, 256), (7, 129, 520),
          (4, 70, 1032), (6, 33, 2048), (3, 17, 4096), (12, 1, 896)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d", SHAPES)
def test_full_all_reads(ar, oracle, dtype, n_hist, T, d):
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=n_hist * 1000 + d, dtype=dtype)
    out, lse = ar.full_fwd(h, w)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.full_fwd(h64, w64)
    check_out(to_f64(out), ref, dtype)
    check_lse(to_f64(lse), ref_lse)


@pytest.mark.parametrize("hdt,odt", [("bf16", "f32"), ("f32", "bf16")])
def test_full_mixed_dtypes(ar, oracle, hdt, odt):
    h, w, h64, w64 = _inputs(11, 45, 136, seed=5, dtype=hdt)
    out, _ = ar.full_fwd(h, w, out_dtype=torch.float32 if odt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    ref, _ = oracle.full_fwd(h64, w64)
    check_out(to_f64(out), ref, odt)


def test_full_model_order_with_rinv_cache(ar, oracle):
    # the fp32 16-sublayer workload, called read by read as a model would
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, host_inputs
    wl = WORKLOADS["full_fp32_small"]
    hist, w, _ = host_inputs(wl)
    h = torch.from_numpy(hist).to(DEV)
    wd = torch.from_numpy(w).to(DEV)
    rinv = torch.full((wl.n_hist, wl.T), -1.0, device=DEV)
    outs, lses = [], []
    for l in range(wl.n_hist):
        o, ls = ar.full_fwd(h, wd[l:l + 1], q_begin=l, n_q=1, rinv=rinv, rinv_valid_rows=l)
        outs.append(o)
        lses.append(ls)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.full_fwd(hist, w)
    check_out(to_f64(torch.cat(outs)), ref, "f32")
    check_lse(to_f64(torch.cat(lses)), ref_lse)
    h64 = hist.astype(np.float64)
    expect_r = 1.0 / np.sqrt((h64 ** 2).mean(-1) + 1e-6)
    np.testing.assert_allclose(to_f64(rinv), expect_r, rtol=2e-6)
    # the batched call agrees with the read-by-read calls
    ob, _ = ar.full_fwd(h, wd)
    check_out(to_f64(ob), ref, "f32")


def test_full_rinv_partially_valid(ar, oracle):
    n_hist, T, d = 10, 50, 96
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=77, dtype="bf16")
    rinv = torch.full((n_hist, T), -7.0, device=DEV)
    ar.full_fwd(h, w[:3], q_begin=0, n_q=3, rinv=rinv)          # fills rows 0..2
    snap = rinv.clone()
    out, _ = ar.full_fwd(h, w[5:8], q_begin=5, n_q=3, rinv=rinv, rinv_valid_rows=3)
    torch.cuda.synchronize()
    ref, _ = oracle.full_fwd(h64, w64[5:8], q_begin=5, n_q=3)
    check_out(to_f64(out), ref, "bf16")
    expect_r = 1.0 / np.sqrt((h64 ** 2).mean(-1) + 1e-6)
    got = to_f64(rinv)
    np.testing.assert_allclose(got[:8], expect_r[:8], rtol=2e-6)
    assert torch.equal(rinv[:3], snap[:3])       # trusted rows untouched
    assert (got[8:] == -7.0).all()               # rows past the last read untouched


def test_full_single_row_is_exact(ar):
    h, w, _, _ = _inputs(1, 77, 264, seed=3, dtype="bf16")
    out, lse = ar.full_fwd(h, w)
    torch.cuda.synchronize()
    assert torch.equal(out, h)


def test_full_zero_queries_give_prefix_mean(ar, oracle):
    n_hist, T, d = 13, 40, 128
    h, _, h64, _ = _inputs(n_hist, T, d, seed=9, dtype="f32")
    w = torch.zeros((n_hist, d), device=DEV)
    out, lse = ar.full_fwd(h, w)
    torch.cuda.synchronize()
    ref = np.cumsum(h64, axis=0) / np.arange(1, n_hist + 1)[:, None, None]
    check_out(to_f64(out), ref, "f32")
    np.testing.assert_allclose(to_f64(lse), np.log(np.arange(1, n_hist + 1))[:, None]
                               * np.ones((1, T)), atol=2e-6)


def test_full_is_deterministic(ar):
    h, w, _, _ = _inputs(20, 500, 640, seed=11, dtype="bf16", sigma_growth=True)
    o1, l1 = ar.full_fwd(h, w)
    o2, l2 = ar.full_fwd(h, w)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _model_order_sweep(ar, h, w):
    n_hist, T, _ = h.shape
    rinv = torch.empty((n_hist, T), device=DEV)
    out = torch.empty_like(h)
    lse = torch.empty((n_hist, T), device=DEV)
    for l in range(n_hist):
        ar.full_fwd(h, w[l:l + 1], q_begin=l, n_q=1, rinv=rinv, rinv_valid_rows=l,
                    out=out[l:l + 1], lse=lse[l:l + 1])
    return out, lse


@pytest.mark.parametrize("name", ["full_L32_d896", "full_L70_d640"])
def test_full_workload_model_order_sampled(ar, oracle, name):
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs, token_sample
    wl = WORKLOADS[name]
    h, w, _ = device_inputs(wl, DEV)
    out, lse = _model_order_sweep(ar, h, w)
    torch.cuda.synchronize()
    idx = token_sample(wl.T, 384, seed=wl.seed)
    ti = torch.from_numpy(idx).to(DEV)
    h64 = to_f64(h.index_select(1, ti))
    ref, ref_lse = oracle.full_fwd(h64, to_f64(w))
    stats = check_out(to_f64(out.index_select(1, ti)), ref, wl.dtype)
    check_lse(to_f64(lse.index_select(1, ti)), ref_lse)
    print(f"{name}: {stats}", flush=True)


def test_full_workload_batched_l70_sampled(ar, oracle):
    # the L=70 / d=640 history in one call with all 141 reads: its 180 KB of
    # rows per token do not all fit in a workgroup's LDS, so the batched kernel
    # stages the first rows and reads the rest from global memory
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs, token_sample
    wl = WORKLOADS["full_L70_d640"]
    h, w, _ = device_inputs(wl, DEV)
    out, lse = ar.full_fwd(h, w)
    torch.cuda.synchronize()
    idx = token_sample(wl.T, 256, seed=wl.seed + 1)
    ti = torch.from_numpy(idx).to(DEV)
    ref, ref_lse = oracle.full_fwd(to_f64(h.index_select(1, ti)), to_f64(w))
    stats = check_out(to_f64(out.index_select(1, ti)), ref, wl.dtype)
    check_lse(to_f64(lse.index_select(1, ti)), ref_lse)
    print(f"{wl.name} batched: {stats}", flush=True)


# ---------------------------------------------------------------------------
# fused pre-norm of the output (the sublayer's branch input RMSNorm_pre,l(h_l))

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_gain", [False, True])
@pytest.mark.parametrize("n_hist,T,d", [(9, 37, 64), (7, 129, 520), (6, 33, 2048)])
def test_full_prenorm_matches_oracle(ar, oracle, dtype, with_gain, n_hist, T, d):
    h, w, hd, wd = _inputs(n_hist, T, d, seed=n_hist + d, dtype=dtype)
    gain = torch.from_numpy(np.random.default_rng(d).uniform(0.5, 1.5, (n_hist, d)).astype(np.float32)).to(DEV) \
        if with_gain else None
    out = torch.empty(h.shape, dtype=h.dtype, device=DEV)
    normed = torch.empty_like(out)
    ar.full_fwd(h, w, out=out, normed=normed, norm_gain=gain)
    torch.cuda.synchronize()
    ref, _ = oracle.full_fwd(hd, wd)
    ref_n = oracle.prenorm(ref, None if gain is None else to_f64(gain))
    check_out(to_f64(out), ref, dtype)
    check_out(to_f64(normed), ref_n, dtype, what="normed")


def test_full_prenorm_in_model_order(ar, oracle):
    # read by read with the RMS cache, as a model runs it; gain per read
    n_hist, T, d = 17, 48, 896
    h, w, hd, wd = _inputs(n_hist, T, d, seed=4, dtype="bf16")
    gain = torch.from_numpy(np.random.default_rng(5).uniform(0.5, 1.5, (n_hist, d)).astype(np.float32)).to(DEV)
    rinv = torch.empty((n_hist, T), device=DEV)
    normed = torch.empty_like(h)
    for l in range(n_hist):
        ar.full_fwd(h, w[l:l + 1], q_begin=l, n_q=1, rinv=rinv, rinv_valid_rows=l,
                    normed=normed[l:l + 1], norm_gain=gain[l:l + 1])
    torch.cuda.synchronize()
    ref, _ = oracle.full_fwd(hd, wd)
    check_out(to_f64(normed), oracle.prenorm(ref, to_f64(gain)), "bf16", what="normed")


# ---------------------------------------------------------------------------
# weight probe (softmax weights in source order, tokens fastest)

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d,q_begin", [(9, 37, 64, 0), (17, 40, 520, 3), (6, 33, 2048, 0)])
def test_full_alpha_probe(ar, oracle, dtype, n_hist, T, d, q_begin):
    h, w, hd, wd = _inputs(n_hist, T, d, seed=n_hist * 5 + d, dtype=dtype, w_sigma=0.05)
    n_q = n_hist - q_begin
    w = w[q_begin:].contiguous()
    alpha = torch.full((n_q, n_hist, T), float("nan"), device=DEV)
    ar.full_fwd(h, w, q_begin=q_begin, alpha=alpha)
    torch.cuda.synchronize()
    _, _, ref = oracle.fwd(oracle.FULL, hd, wd[q_begin:], q_begin=q_begin, want_alpha=True)
    ref = ref.transpose(0, 2, 1)  # [n_q][n_hist][T]
    a = to_f64(alpha)
    check_rel(a, ref, 1e-5, "alpha")
    assert (a >= 0).all()
    np.testing.assert_allclose(a.sum(1), 1.0, atol=1e-5)
    for j in range(n_q):  # exactly zero past the read's source count
        assert (a[j, q_begin + j + 1:] == 0).all()
