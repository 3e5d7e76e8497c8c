"""GPU parity of attnres_block_fwd (two-phase Block AttnRes) against the fp64
oracle: every element on small and ragged cases, sampled tokens at the full
sizes of the 128K-token S=8 and the L=24 S=4 workloads."""
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


def _inputs(n_hist, T, d, seed, dtype, w_sigma=0.3):
    rng = np.random.default_rng(seed)
    hist = rng.standard_normal((n_hist, T, d)).astype(np.float32)
    w = (rng.standard_normal((n_hist, d)) * w_sigma).astype(np.float32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    h = torch.from_numpy(hist).to(DEV).to(tdt)
    return h, torch.from_numpy(w).to(DEV), to_f64(h), w.astype(np.float64)


# (n_hist, T, d, S): register two-phase path unless the source count exceeds 13
CASES = [(1, 4, 8, 1), (2, 5, 16, 1), (9, 37, 64, 1), (9, 37, 64, 2), (13, 21, 136, 3),
         (17, 40, 256, 4), (17, 40, 256, 16), (17, 40, 256, 40), (25, 19, 520, 8),
         (33, 11, 1024, 4), (65, 6, 2048, 8), (12, 9, 4096, 5), (20, 13, 896, 7),
         (40, 7, 128, 2), (70, 5, 64, 1)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d,S", CASES)
def test_block_all_reads(ar, oracle, dtype, n_hist, T, d, S):
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=n_hist * 31 + d + S, dtype=dtype)
    out, lse = ar.block_fwd(h, w, S)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_fwd(h64, w64, S)
    check_out(to_f64(out), ref, dtype)
    check_lse(to_f64(lse), ref_lse)


@pytest.mark.parametrize("n_hist,S,q_begin,n_q", [(17, 4, 5, 7), (17, 4, 16, 1), (33, 8, 0, 1),
                                                  (33, 8, 9, 17), (40, 2, 30, 10), (9, 3, 3, 1)])
def test_block_read_subsets(ar, oracle, n_hist, S, q_begin, n_q):
    h, w, h64, w64 = _inputs(n_hist, 23, 264, seed=S * 100 + q_begin, dtype="bf16")
    out, lse = ar.block_fwd(h, w[q_begin:q_begin + n_q], S, q_begin=q_begin, n_q=n_q)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_fwd(h64, w64[q_begin:q_begin + n_q], S, q_begin=q_begin, n_q=n_q)
    check_out(to_f64(out), ref, "bf16")
    check_lse(to_f64(lse), ref_lse)


# Calls with >= 16 reads over a bf16 history and at most 13 sources are served by
# the kernel with one wave per block group (block_batch.hip): fp32 and bf16
# outputs, odd and even S, three chunks per lane, and read ranges that start
# inside a group (the partial sum is caught up from the group's first row).
@pytest.mark.parametrize("odt", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d,S,q_begin", [(24, 9, 264, 2, 0), (22, 11, 1032, 3, 0),
                                                  (31, 7, 520, 5, 3), (40, 5, 2048, 8, 13),
                                                  (49, 6, 1024, 4, 0)])
def test_block_group_kernel(ar, oracle, odt, n_hist, T, d, S, q_begin):
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=n_hist * 7 + S + q_begin, dtype="bf16", w_sigma=0.05)
    n_q = n_hist - q_begin
    assert n_q >= 16 and 1 + (n_hist - 1) // S <= 13
    out, lse = ar.block_fwd(h, w[q_begin:], S, q_begin=q_begin, n_q=n_q,
                            out_dtype=torch.float32 if odt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_fwd(h64, w64[q_begin:], S, q_begin=q_begin, n_q=n_q)
    check_out(to_f64(out), ref, odt)
    check_lse(to_f64(lse), ref_lse)


# The per-group Block kernel on many tokens (several hundred workgroups, ragged
# counts) at every element against the oracle: reads starting inside a group,
# four chunks per lane at the 128K workload's d and S; then four chunks per lane
# with more than nine sources (the 13-source instantiation).
@pytest.mark.parametrize("n_hist,T,d,S,q_begin", [(33, 805, 256, 4, 0), (49, 601, 1024, 4, 3),
                                                  (65, 700, 2048, 8, 0), (40, 523, 520, 5, 13)])
def test_block_group_kernel_many_tokens(ar, oracle, n_hist, T, d, S, q_begin):
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=T + d + S, dtype="bf16", w_sigma=0.05)
    n_q = n_hist - q_begin
    out, lse = ar.block_fwd(h, w[q_begin:].contiguous(), S, q_begin=q_begin, n_q=n_q)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_fwd(h64, w64[q_begin:], S, q_begin=q_begin, n_q=n_q)
    check_out(to_f64(out), ref, "bf16")
    check_lse(to_f64(lse), ref_lse)


@pytest.mark.parametrize("n_hist,T,d,S", [(65, 9, 2048, 6), (49, 5, 1600, 4)])
def test_block_group_kernel_four_chunks_many_sources(ar, oracle, n_hist, T, d, S):
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=T * 3 + S, dtype="bf16", w_sigma=0.05)
    assert 10 <= 1 + (n_hist - 1) // S <= 13
    out, lse = ar.block_fwd(h, w, S)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_fwd(h64, w64, S)
    check_out(to_f64(out), ref, "bf16")
    check_lse(to_f64(lse), ref_lse)


def test_block_S1_matches_full_kernel(ar):
    h, w, _, _ = _inputs(12, 300, 512, seed=4, dtype="f32")
    ob, lb = ar.block_fwd(h, w, 1)
    of, lf = ar.full_fwd(h, w)
    torch.cuda.synchronize()
    check_out(to_f64(ob), to_f64(of), "f32", what="block S=1 vs full")
    check_lse(to_f64(lb), to_f64(lf))


def test_block_is_deterministic(ar):
    h, w, _, _ = _inputs(33, 200, 1024, seed=8, dtype="bf16")
    o1, l1 = ar.block_fwd(h, w, 4)
    o2, l2 = ar.block_fwd(h, w, 4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_block_zero_queries_give_stream_over_source_count(ar):
    n_hist, T, d, S = 19, 30, 192, 4
    h, _, h64, _ = _inputs(n_hist, T, d, seed=12, dtype="f32")
    w = torch.zeros((n_hist, d), device=DEV)
    out, _ = ar.block_fwd(h, w, S)
    torch.cuda.synchronize()
    n_src = np.array([1 + l // S + (1 if l % S else 0) for l in range(n_hist)], dtype=np.float64)
    ref = np.cumsum(h64, axis=0) / n_src[:, None, None]
    check_out(to_f64(out), ref, "f32")


@pytest.mark.parametrize("name,S", [("block_S8_d2048_128k", 8), ("fwdbwd_L24_d1024", 4)])
def test_block_workload_sampled(ar, oracle, name, S):
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs, token_sample
    wl = WORKLOADS[name]
    h, w, _ = device_inputs(wl, DEV)
    out, lse = ar.block_fwd(h, w, S)
    torch.cuda.synchronize()
    idx = token_sample(wl.T, 256, seed=wl.seed)
    ti = torch.from_numpy(idx).to(DEV)
    ref, ref_lse = oracle.block_fwd(to_f64(h.index_select(1, ti)), to_f64(w), S)
    stats = check_out(to_f64(out.index_select(1, ti)), ref, wl.dtype)
    check_lse(to_f64(lse.index_select(1, ti)), ref_lse)
    print(f"{name}: {stats}", flush=True)
    del h, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d,S", [(17, 40, 256, 4), (13, 21, 136, 3), (65, 6, 2048, 8),
                                          (70, 5, 64, 1)])
def test_block_alpha_probe(ar, oracle, dtype, n_hist, T, d, S):
    # two-phase kernel (<= 13 sources) and the streaming fallback (S = 1, 70 rows)
    h, w, hd, wd = _inputs(n_hist, T, d, seed=n_hist * 3 + S, dtype=dtype, w_sigma=0.05)
    alpha = torch.full((n_hist, n_hist, T), float("nan"), device=DEV)
    ar.block_fwd(h, w, S, alpha=alpha)
    torch.cuda.synchronize()
    _, _, ref = oracle.fwd(oracle.BLOCK, hd, wd, S=S, want_alpha=True)
    ref = ref.transpose(0, 2, 1)
    a = to_f64(alpha)
    check_rel(a, ref, 1e-5, "alpha")
    assert (a >= 0).all()
    np.testing.assert_allclose(a.sum(1), 1.0, atol=1e-5)
    for l in range(n_hist):
        ns = oracle.num_sources(oracle.BLOCK, l, S)
        assert (a[l, ns:] == 0).all()


@pytest.mark.parametrize("n_hist,T,d,S,q_begin,n_q", [(16, 1, 64, 4, 0, 16), (20, 3, 136, 20, 0, 20),
                                                      (20, 3, 136, 25, 0, 20), (30, 2, 8, 6, 7, 16),
                                                      (26, 5, 512, 2, 10, 16)])
def test_block_group_kernel_edges(ar, oracle, n_hist, T, d, S, q_begin, n_q):
    # exactly 16 reads, S at or past the history (only v_0 and the partial
    # sum), one token, d = 8, and reads that start inside a group
    h, w, h64, w64 = _inputs(n_hist, T, d, seed=T * 11 + S + q_begin, dtype="bf16", w_sigma=0.1)
    alpha = torch.full((n_q, n_hist, T), float("nan"), device=DEV)
    out, lse = ar.block_fwd(h, w[q_begin:q_begin + n_q].contiguous(), S, q_begin=q_begin, n_q=n_q,
                            alpha=alpha)
    torch.cuda.synchronize()
    ref, ref_lse, ref_a = oracle.fwd(oracle.BLOCK, h64, w64[q_begin:q_begin + n_q], S=S,
                                     q_begin=q_begin, n_q=n_q, want_alpha=True)
    check_out(to_f64(out), ref, "bf16")
    check_lse(to_f64(lse), ref_lse)
    check_rel(to_f64(alpha), ref_a.transpose(0, 2, 1), 1e-5, "alpha")
