"""GPU parity of attnres_bwd (Full and Block) against the fp64 oracle's
backward, which is itself pinned by finite differences on the CPU."""
import numpy as np
import pytest
import torch

from parity import check_out, check_rel, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FULL, BLOCK = 0, 1


@pytest.fixture(scope="module")
def ar():
    import depth_wise_attention_attnres_amd as ar
    return ar


def _case(n_hist, T, d, seed, dtype, w_sigma=0.3, n_q=None, q_begin=0):
    rng = np.random.default_rng(seed)
    n_q = n_hist - q_begin if n_q is None else n_q
    hist = rng.standard_normal((n_hist, T, d)).astype(np.float32)
    w = (rng.standard_normal((n_q, d)) * w_sigma).astype(np.float32)
    dout = rng.standard_normal((n_q, T, d)).astype(np.float32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    h = torch.from_numpy(hist).to(DEV).to(tdt)
    g = torch.from_numpy(dout).to(DEV).to(tdt)
    return h, torch.from_numpy(w).to(DEV), g


def _run(ar, variant, S, h, w, g, q_begin=0, dhist_dtype=None):
    dh, dw = ar.bwd(variant, h, w, g, S=S, q_begin=q_begin, dhist_dtype=dhist_dtype)
    torch.cuda.synchronize()
    return dh, dw


def _check(ar, oracle, variant, S, h, w, g, dtype, q_begin=0, dhist_dtype=None):
    dh, dw = _run(ar, variant, S, h, w, g, q_begin=q_begin, dhist_dtype=dhist_dtype)
    ref_dh, ref_dw = oracle.bwd(variant, to_f64(h), to_f64(w), to_f64(g), S=S, q_begin=q_begin)
    out_dt = dtype if dhist_dtype is None else ("f32" if dhist_dtype == torch.float32 else "bf16")
    if out_dt == "f32":
        check_rel(to_f64(dh), ref_dh, 1e-5, "dhist")
    else:
        check_out(to_f64(dh)[None], ref_dh[None], "bf16", what="dhist")
    check_rel(to_f64(dw), ref_dw, 1e-5, "dw")


CASES = [(1, 3, 8, 1), (2, 5, 16, 1), (9, 37, 64, 1), (9, 37, 64, 2), (13, 21, 136, 3),
         (17, 40, 256, 4), (17, 20, 256, 40), (25, 19, 520, 8), (33, 11, 1024, 4),
         (20, 13, 896, 7), (70, 5, 64, 1), (70, 6, 72, 5), (7, 45, 2048, 3)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d,S", CASES)
def test_bwd_matches_oracle(ar, oracle, dtype, n_hist, T, d, S):
    h, w, g = _case(n_hist, T, d, seed=n_hist * 7 + d + S, dtype=dtype)
    variant = FULL if S == 1 else BLOCK
    _check(ar, oracle, variant, S, h, w, g, dtype)
    if S == 1:  # Block with S = 1 is Full
        _check(ar, oracle, BLOCK, 1, h, w, g, dtype)


@pytest.mark.parametrize("variant,S,n_hist,q_begin,n_q", [(FULL, 1, 12, 4, 5), (FULL, 1, 12, 11, 1),
                                                          (BLOCK, 3, 17, 5, 7), (BLOCK, 4, 17, 0, 3),
                                                          (BLOCK, 2, 30, 21, 9)])
def test_bwd_read_subsets(ar, oracle, variant, S, n_hist, q_begin, n_q):
    h, w, g = _case(n_hist, 9, 128, seed=q_begin * 3 + n_q, dtype="f32", n_q=n_q, q_begin=q_begin)
    _check(ar, oracle, variant, S, h, w, g, "f32", q_begin=q_begin)


def test_bwd_bf16_history_fp32_gradient(ar, oracle):
    h, w, g = _case(17, 23, 192, seed=5, dtype="bf16")
    _check(ar, oracle, BLOCK, 4, h, w, g, "bf16", dhist_dtype=torch.float32)


def test_bwd_is_deterministic(ar):
    h, w, g = _case(25, 300, 512, seed=6, dtype="bf16")
    a = _run(ar, BLOCK, 4, h, w, g)
    b = _run(ar, BLOCK, 4, h, w, g)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("variant,S", [(FULL, 1), (BLOCK, 4)])
def test_bwd_workload_sampled(ar, oracle, variant, S):
    # the 48-sublayer, d = 1024, 4 x 4096-token workload: dhist of sampled
    # tokens from the full-size call; dw from a call on a token subset
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs, token_sample
    wl = WORKLOADS["fwdbwd_L24_d1024"]
    h, w, g = device_inputs(wl, DEV)
    dh, dw = _run(ar, variant, S, h, w, g)
    idx = token_sample(wl.T, 128, seed=wl.seed)
    ti = torch.from_numpy(idx).to(DEV)
    hs, gs = h.index_select(1, ti).contiguous(), g.index_select(1, ti).contiguous()
    ref_dh, ref_dw = oracle.bwd(variant, to_f64(hs), to_f64(w), to_f64(gs), S=S)
    stats = check_out(to_f64(dh.index_select(1, ti))[None], ref_dh[None], "bf16", what="dhist")
    _, dw_sub = _run(ar, variant, S, hs, w, gs)
    check_rel(to_f64(dw_sub), ref_dw, 1e-5, "dw (token subset)")
    print(f"bwd {variant} S={S}: {stats}", flush=True)


@pytest.mark.parametrize("variant,S,n_hist,q_begin,n_q,d", [(FULL, 1, 12, 4, 5, 128), (FULL, 1, 49, 17, 32, 256),
                                                            (FULL, 1, 70, 40, 30, 64),
                                                            (FULL, 1, 40, 0, 40, 136),
                                                            (BLOCK, 4, 30, 9, 21, 128)])
def test_bwd_read_subsets_bf16(ar, oracle, variant, S, n_hist, q_begin, n_q, d):
    # bf16 history and dout: the matrix-core scores path (Full, <= 64 reads),
    # with reads that start past row 0 and row tiles the first read tile skips
    h, w, g = _case(n_hist, 11, d, seed=q_begin * 5 + n_q + d, dtype="bf16", n_q=n_q,
                    q_begin=q_begin)
    _check(ar, oracle, variant, S, h, w, g, "bf16", q_begin=q_begin)


@pytest.mark.parametrize("n_hist,T,d,S,q_begin", [(33, 9, 1024, 4, 0), (26, 7, 200, 3, 5)])
def test_bwd_group_kernel_fp32_dout(ar, oracle, n_hist, T, d, S, q_begin):
    # bf16 history with an fp32 upstream gradient, >= 16 reads: the per-read
    # coefficients come from the kernel with one wave per block group
    h, w, g = _case(n_hist, T, d, seed=n_hist + S, dtype="bf16", q_begin=q_begin)
    g = g.to(torch.float32)
    _check(ar, oracle, BLOCK, S, h, w, g, "bf16", q_begin=q_begin)


@pytest.mark.parametrize("n_hist,T,d,S,q_begin", [(16, 1, 64, 4, 0), (18, 3, 136, 18, 0), (22, 2, 8, 5, 6)])
def test_bwd_group_kernel_edges(ar, oracle, n_hist, T, d, S, q_begin):
    # exactly 16 reads, S at the history length, one token, d = 8
    h, w, g = _case(n_hist, T, d, seed=n_hist * 3 + T + S, dtype="bf16", q_begin=q_begin)
    _check(ar, oracle, BLOCK, S, h, w, g, "bf16", q_begin=q_begin)


@pytest.mark.parametrize("variant,S", [(FULL, 1), (BLOCK, 4)])
def test_bwd_workload_full_dw(ar, oracle, variant, S):
    # The 48-sublayer, d = 1024, 4 x 4096-token workload at its full size, in
    # the launch configuration the benchmark times: dw is a reduction over all
    # 16384 tokens (512 chunks of 32 tokens summed in 16 groups of 32), so the
    # oracle runs on every token, 2048 at a time, its chunk dw summed in fp64.
    # dhist is compared on every token too.
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs
    wl = WORKLOADS["fwdbwd_L24_d1024"]
    h, w, g = device_inputs(wl, DEV)
    dh, dw = _run(ar, variant, S, h, w, g)
    ref_dw = np.zeros(tuple(dw.shape), np.float64)
    step = 2048
    for t0 in range(0, wl.T, step):
        hs = to_f64(h[:, t0:t0 + step])
        gs = to_f64(g[:, t0:t0 + step])
        ref_dh, part_dw = oracle.bwd(variant, hs, to_f64(w), gs, S=S)
        ref_dw += part_dw
        check_out(to_f64(dh[:, t0:t0 + step])[None], ref_dh[None], "bf16",
                  what=f"dhist tokens {t0}..{t0 + step}")
    check_rel(to_f64(dw), ref_dw, 1e-5, "dw (all tokens)")


@pytest.mark.parametrize("variant,S,dtype", [(FULL, 1, "f32"), (FULL, 1, "bf16"),
                                             (BLOCK, 4, "f32"), (BLOCK, 4, "bf16")])
def test_bwd_dw_many_chunks_per_group(ar, oracle, variant, S, dtype):
    # 2080 tokens: 65 chunks of 32 (the last one ragged) in 16 reduction
    # groups of 5, so every group sums several chunks and the last group fewer
    h, w, g = _case(17, 2080, 64, seed=11 + S, dtype=dtype, w_sigma=0.2)
    _check(ar, oracle, variant, S, h, w, g, dtype)


@pytest.mark.parametrize("variant,S", [(FULL, 1), (BLOCK, 3)])
def test_bwd_accumulate(ar, oracle, variant, S):
    # accumulate=True: the gradients of two read ranges, added into the same
    # fp32 dhist (starting from non-zero values), equal the oracle's gradient
    # of all reads plus the start values; dw rows of the two ranges are
    # disjoint.  Then dw accumulated over two token halves equals dw of all
    # tokens.
    n_hist, T, d, k = 14, 40, 136, 6
    h, w, g = _case(n_hist, T, d, seed=21 + S, dtype="bf16")
    ref_dh, ref_dw = oracle.bwd(variant, to_f64(h), to_f64(w), to_f64(g), S=S)
    start = torch.randn((n_hist, T, d), generator=torch.Generator().manual_seed(3)).to(DEV)
    dh = start.clone()
    dw = torch.zeros((n_hist, d), dtype=torch.float32, device=DEV)
    ar.bwd(variant, h, w[:k].contiguous(), g[:k].contiguous(), S=S, q_begin=0, dhist=dh,
           dw=dw[:k], accumulate=True)
    ar.bwd(variant, h, w[k:].contiguous(), g[k:].contiguous(), S=S, q_begin=k, dhist=dh,
           dw=dw[k:], accumulate=True)
    torch.cuda.synchronize()
    check_rel(to_f64(dh) - to_f64(start), ref_dh, 1e-5, "dhist accumulated over read ranges")
    check_rel(to_f64(dw), ref_dw, 1e-5, "dw of two read ranges")

    half = T // 2
    dw2 = torch.full((n_hist, d), 0.25, dtype=torch.float32, device=DEV)
    for sl in (slice(0, half), slice(half, T)):
        hs, gs = h[:, sl].contiguous(), g[:, sl].contiguous()
        dhs = torch.zeros((n_hist, hs.shape[1], d), dtype=torch.float32, device=DEV)
        ar.bwd(variant, hs, w, gs, S=S, dhist=dhs, dw=dw2, accumulate=True)
    torch.cuda.synchronize()
    check_rel(to_f64(dw2) - 0.25, ref_dw, 1e-5, "dw accumulated over token halves")


def test_bwd_accumulate_rows_no_read_sees(ar, oracle):
    # reads 0..4 of a 12-row history: rows 5.. get no gradient, so an
    # accumulating call leaves them as they were
    h, w, g = _case(12, 9, 64, seed=31, dtype="f32", n_q=5)
    start = torch.randn((12, 9, 64), generator=torch.Generator().manual_seed(4)).to(DEV)
    dh = start.clone()
    dw = torch.zeros((5, 64), dtype=torch.float32, device=DEV)
    ar.bwd(FULL, h, w, g, dhist=dh, dw=dw, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dh[5:], start[5:])
    ref_dh, ref_dw = oracle.bwd(FULL, to_f64(h), to_f64(w), to_f64(g))
    check_rel(to_f64(dh) - to_f64(start), ref_dh, 1e-5, "dhist")
    check_rel(to_f64(dw), ref_dw, 1e-5, "dw")


def test_bwd_mfma_scores_beyond_64k_lds(ar, oracle):
    # Full, bf16, 64 reads from row 0: the matrix-core coefficient kernel
    # needs about 80 KB of LDS per workgroup, above the 64 KB default limit
    h, w, g = _case(64, 7, 128, seed=41, dtype="bf16", w_sigma=0.1)
    _check(ar, oracle, FULL, 1, h, w, g, "bf16")
