"""GPU parity of the input-dependent query ("Kimi K3 notes 2", sec. 6): the
matrix-core projection attnres_query_proj against the oracle's plain
product, and the Full aggregation with per-token queries (attnres_full_fwd_q)
against the oracle's per-token forward -- with queries the oracle computed,
and end to end from the projection."""
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


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)


# small and ragged shapes, then several 256-token tiles per read with (read,
# token tile) group counts that are not multiples of the 8 XCD rounds, ragged
# last token and output tiles, and d = 2048 (16 output tiles)
@pytest.mark.parametrize("n_q,T,d", [(1, 5, 8), (3, 70, 64), (2, 100, 136), (2, 33, 2048), (1, 129, 896),
                                     (9, 700, 136), (3, 1037, 896), (2, 513, 2048), (11, 256, 64)])
def test_query_proj_matches_oracle(ar, oracle, n_q, T, d):
    rng = np.random.default_rng(n_q * 7 + d)
    x = _bf16(rng.standard_normal((n_q, T, d)))
    W = _bf16(rng.standard_normal((n_q, d, d)) / np.sqrt(d))
    q = ar.query_proj(x, W)
    torch.cuda.synchronize()
    check_rel(to_f64(q), oracle.query_proj(to_f64(x), to_f64(W)), 1e-5, "q")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d", [(9, 37, 64), (7, 129, 520), (5, 17, 2048)])
def test_full_fwd_q_matches_oracle(ar, oracle, dtype, n_hist, T, d):
    rng = np.random.default_rng(n_hist + d)
    hist = rng.standard_normal((n_hist, T, d)).astype(np.float32)
    q = (rng.standard_normal((n_hist, T, d)) * 0.05).astype(np.float32)  # queries from the test
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    h = torch.from_numpy(hist).to(DEV).to(tdt)
    out, lse = ar.full_fwd_q(h, torch.from_numpy(q).to(DEV))
    torch.cuda.synchronize()
    ref, ref_lse = oracle.fwd_tokq(oracle.FULL, to_f64(h), q.astype(np.float64))
    check_out(to_f64(out), ref, dtype)
    check_lse(to_f64(lse), ref_lse)


def test_full_fwd_q_model_order_end_to_end(ar, oracle):
    # read by read, as a model runs it: read l projects the newest row v_l with
    # W_l, then aggregates rows 0..l with that per-token query (RMS cache on)
    n_hist, T, d = 13, 96, 256
    rng = np.random.default_rng(5)
    h = _bf16(rng.standard_normal((n_hist, T, d)))
    W = _bf16(rng.standard_normal((n_hist, d, d)) * 0.05 / np.sqrt(d))
    rinv = torch.empty((n_hist, T), device=DEV)
    out = torch.empty_like(h)
    lse = torch.empty((n_hist, T), device=DEV)
    for l in range(n_hist):
        q = ar.query_proj(h[l:l + 1], W[l:l + 1])
        ar.full_fwd_q(h, q, q_begin=l, rinv=rinv, rinv_valid_rows=l, out=out[l:l + 1],
                      lse=lse[l:l + 1])
    torch.cuda.synchronize()
    q_ref = oracle.query_proj(to_f64(h), to_f64(W))  # every read projects its own row
    ref, ref_lse = oracle.fwd_tokq(oracle.FULL, to_f64(h), q_ref)
    check_out(to_f64(out), ref, "bf16")
    check_lse(to_f64(lse), ref_lse)


# Block reads with a query per (read, token).  The shapes reach each Block
# kernel: the per-group kernel (bf16 history, >= 16 reads, S >= 2, <= 13
# sources), the two-phase register kernel (fp32 histories or few reads) and the
# streaming kernel (more than 13 sources).
BLOCK_Q_CASES = [
    # n_hist, T, d, S, q_begin, dtype
    (33, 20, 256, 4, 0, "bf16"),     # per-group kernel
    (65, 9, 2048, 8, 0, "bf16"),     # per-group kernel at the 128K shape's width
    (26, 11, 136, 3, 5, "bf16"),     # per-group kernel, reads from row 5, ragged d
    (17, 23, 520, 4, 0, "f32"),      # two-phase kernel
    (12, 30, 64, 5, 3, "bf16"),      # two-phase kernel (fewer than 16 reads)
    (40, 7, 64, 2, 0, "bf16"),       # streaming kernel (20 blocks)
]


@pytest.mark.parametrize("n_hist,T,d,S,q_begin,dtype", BLOCK_Q_CASES)
def test_block_fwd_q_matches_oracle(ar, oracle, n_hist, T, d, S, q_begin, dtype):
    rng = np.random.default_rng(n_hist * 3 + d + S)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    h = torch.from_numpy(rng.standard_normal((n_hist, T, d)).astype(np.float32)).to(DEV).to(tdt)
    n_q = n_hist - q_begin
    q = (rng.standard_normal((n_q, T, d)) * 0.05).astype(np.float32)
    out, lse = ar.block_fwd_q(h, torch.from_numpy(q).to(DEV), S, q_begin=q_begin)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.fwd_tokq(oracle.BLOCK, to_f64(h), q.astype(np.float64), S=S,
                                   q_begin=q_begin)
    check_out(to_f64(out), ref, dtype)
    check_lse(to_f64(lse), ref_lse)


@pytest.mark.parametrize("n_hist,T,d,S", [(19, 96, 256, 4), (13, 40, 128, 1), (14, 33, 136, 3)])
def test_block_fwd_q_model_order_end_to_end(ar, oracle, n_hist, T, d, S):
    # read by read, as a model runs it: read l projects the newest row v_l with
    # W_l, scores the frozen sources (closing a block at l mod S == 0) and
    # merges the partial sum -- against the oracle's Block read with the
    # oracle's own projections
    rng = np.random.default_rng(7 + S)
    h = _bf16(rng.standard_normal((n_hist, T, d)))
    W = _bf16(rng.standard_normal((n_hist, d, d)) * 0.05 / np.sqrt(d))
    out, lse = ar.block_model_order_q(h, W, S)
    torch.cuda.synchronize()
    q_ref = oracle.query_proj(to_f64(h), to_f64(W))
    ref, ref_lse = oracle.fwd_tokq(oracle.BLOCK, to_f64(h), q_ref, S=S)
    check_out(to_f64(out), ref, "bf16")
    check_lse(to_f64(lse), ref_lse)
    # the same reads in one call from the GPU's projections
    q_all = ar.query_proj(h, W)
    out1, _ = ar.block_fwd_q(h, q_all, S)
    torch.cuda.synchronize()
    check_out(to_f64(out1), ref, "bf16", what="single call")


def test_block_fwd_q_workload_sampled(ar, oracle):
    # the 128K-token, S = 8, d = 2048 history at full size with a query per
    # (read, token) ~ N(0, 0.05^2) (68.7 GB of fp32 queries), in one call;
    # sampled tokens against the oracle (tokens are independent)
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs, token_sample
    wl = WORKLOADS["block_S8_d2048_128k"]
    h, _, _ = device_inputs(wl, DEV)
    n, T, d = h.shape
    gen = torch.Generator(device=DEV).manual_seed(wl.seed + 77)
    q = torch.empty((n, T, d), dtype=torch.float32, device=DEV)
    for l in range(n):
        q[l].normal_(0.0, 0.05, generator=gen)
    out, lse = ar.block_fwd_q(h, q, wl.S)
    torch.cuda.synchronize()
    idx = torch.from_numpy(token_sample(T, 128, seed=wl.seed)).to(DEV)
    hs = to_f64(h.index_select(1, idx))
    qs = to_f64(q.index_select(1, idx))
    del q
    ref, ref_lse = oracle.fwd_tokq(oracle.BLOCK, hs, qs, S=wl.S)
    stats = check_out(to_f64(out.index_select(1, idx)), ref, "bf16")
    check_lse(to_f64(lse.index_select(1, idx)), ref_lse)
    print(f"block_fwd_q 128K sampled: {stats}", flush=True)


def test_query_proj_workload_sampled(ar, oracle):
    # the projection of all 65 reads of the L=32 / d=896 / 16384-token history
    # at full size (the launch bench.py times: 64 token tiles per read, a
    # ragged last output tile), W ~ N(0, 0.05^2 / d) as in the benchmark;
    # sampled tokens against the oracle (tokens are independent)
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs, token_sample
    wl = WORKLOADS["full_L32_d896"]
    h, _, _ = device_inputs(wl, DEV)
    n, T, d = h.shape
    gen = torch.Generator(device=DEV)
    gen.manual_seed(wl.seed + 101)
    W = (torch.randn((n, d, d), generator=gen, device=DEV) * (0.05 / d ** 0.5)).to(torch.bfloat16)
    q = ar.query_proj(h, W)
    torch.cuda.synchronize()
    idx = torch.from_numpy(token_sample(T, 96, seed=wl.seed)).to(DEV)
    ref = oracle.query_proj(to_f64(h.index_select(1, idx)), to_f64(W))
    check_rel(to_f64(q.index_select(1, idx)), ref, 1e-5, "q")
