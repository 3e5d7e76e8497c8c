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


@pytest.mark.parametrize("n_q,T,d", [(1, 5, 8), (3, 70, 64), (2, 100, 136), (2, 33, 2048), (1, 129, 896)])
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
