"""GPU parity of the model-order Block AttnRes entry points
(attnres_block_phase1 once per block group, attnres_block_phase2 once per row
inside a block) against the fp64 oracle: every read of small and ragged
histories, and sampled tokens of the 128K-token S=8 workload at full size."""
import numpy as np
import pytest
import torch

from parity import check_lse, check_out, to_f64

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
    return h, torch.from_numpy(w).to(DEV)


# (n_hist, T, d, S): block groups of every size up to 13 sources, a history
# that S does not divide (the last block stays partial), S = 1 (every row is a
# block), ragged T and d, one and several waves per token
CASES = [(1, 5, 8, 1), (2, 7, 16, 1), (9, 37, 64, 2), (13, 21, 136, 3), (17, 40, 256, 4),
         (17, 9, 72, 5), (25, 19, 520, 8), (33, 11, 1024, 4), (65, 6, 2048, 8), (12, 9, 4096, 5),
         (13, 10, 200, 1), (20, 13, 896, 7)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d,S", CASES)
def test_model_order_matches_oracle(ar, oracle, dtype, n_hist, T, d, S):
    h, w = _inputs(n_hist, T, d, seed=n_hist * 11 + d + S, dtype=dtype)
    out, lse = ar.block_model_order(h, w, S)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_fwd(to_f64(h), to_f64(w), S)
    check_out(to_f64(out), ref, dtype)
    check_lse(to_f64(lse), ref_lse)


def test_model_order_fp32_output_of_bf16_history(ar, oracle):
    h, w = _inputs(17, 23, 192, seed=3, dtype="bf16")
    out = torch.empty(h.shape, dtype=torch.float32, device=DEV)
    out, lse = ar.block_model_order(h, w, 4, out=out)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_fwd(to_f64(h), to_f64(w), 4)
    check_out(to_f64(out), ref, "f32")


def test_block_state_holds_the_block_sums(ar):
    # after the sweep, blocks[c] is the fp32 sum of block c's rows (blocks[0] = v_0)
    n_hist, T, d, S = 17, 9, 64, 4
    h, w = _inputs(n_hist, T, d, seed=8, dtype="f32")
    n_blk = 1 + (n_hist - 1) // S
    st = {"blocks": torch.empty((n_blk, T, d), device=DEV)}
    ar.block_model_order(h, w, S, state=st)
    torch.cuda.synchronize()
    hd = to_f64(h)
    b = to_f64(st["blocks"])
    assert np.array_equal(b[0], hd[0])
    for c in range(1, n_blk):
        np.testing.assert_allclose(b[c], hd[(c - 1) * S + 1: c * S + 1].sum(0), rtol=0, atol=1e-5)


def test_rms_cache_is_bitwise_neutral(ar):
    # phase 1 with the RMS-scale cache gives exactly what recomputing gives
    n_hist, T, d, S = 25, 30, 320, 4
    h, w = _inputs(n_hist, T, d, seed=9, dtype="bf16")
    n_blk = 1 + (n_hist - 1) // S
    blocks = torch.empty((n_blk, T, d), device=DEV)
    rs = torch.empty((n_blk, T), device=DEV)
    partial = torch.empty((T, d), device=DEV)
    for m in range(n_blk):
        l0 = m * S
        n_reads = min(S, n_hist - l0)
        prt = partial if m > 0 else None
        o1, l1 = ar.block_phase1(blocks[: m + 1], m + 1, h[l0], w[l0: l0 + n_reads], partial=prt,
                                 rs=rs[: m + 1])
        blocks_copy = blocks.clone()
        o2, l2 = ar.block_phase1(blocks_copy[: m + 1], m + 1, h[l0], w[l0: l0 + n_reads],
                                 partial=prt, rs=None)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), m
        for k in range(1, n_reads):
            ar.block_phase2(h[l0 + k], partial, k == 1, w[l0 + k], o1[k], l1[k])


def test_model_order_agrees_with_single_call(ar):
    n_hist, T, d, S = 33, 64, 512, 8
    h, w = _inputs(n_hist, T, d, seed=12, dtype="f32")
    a, la = ar.block_model_order(h, w, S)
    b, lb = ar.block_fwd(h, w, S)
    torch.cuda.synchronize()
    scale = b.abs().amax().item()
    assert (a - b).abs().amax().item() <= 1e-5 * scale
    assert (la - lb).abs().amax().item() <= 1e-5 * (1 + lb.abs().amax().item())


def test_model_order_workload_sampled(ar, oracle):
    # the 128K-token, 64-sublayer, S = 8 prefill in model order (the schedule
    # bench.py times), checked on sampled tokens
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs, token_sample
    wl = WORKLOADS["block_S8_d2048_128k"]
    h, w, _ = device_inputs(wl, DEV)
    out, lse = ar.block_model_order(h, w, wl.S)
    torch.cuda.synchronize()
    idx = token_sample(wl.T, 256, seed=wl.seed + 1)
    ti = torch.from_numpy(idx).to(DEV)
    ref, ref_lse = oracle.block_fwd(to_f64(h.index_select(1, ti)), to_f64(w), wl.S)
    stats = check_out(to_f64(out.index_select(1, ti)), ref, wl.dtype)
    check_lse(to_f64(lse.index_select(1, ti)), ref_lse)
    print(f"model order {wl.name}: {stats}", flush=True)
    del h, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_hist,T,d,S", [(17, 40, 256, 4), (13, 21, 136, 3), (12, 9, 2048, 5)])
def test_model_order_prenorm_matches_oracle(ar, oracle, dtype, n_hist, T, d, S):
    h, w = _inputs(n_hist, T, d, seed=n_hist + S, dtype=dtype)
    gain = torch.from_numpy(np.random.default_rng(d + S).uniform(0.5, 1.5, (n_hist, d))
                            .astype(np.float32)).to(DEV)
    normed = torch.empty_like(h)
    out, _ = ar.block_model_order(h, w, S, normed=normed, norm_gain=gain)
    torch.cuda.synchronize()
    ref, _ = oracle.block_fwd(to_f64(h), to_f64(w), S)
    check_out(to_f64(out), ref, dtype)
    check_out(to_f64(normed), oracle.prenorm(ref, to_f64(gain)), dtype, what="normed")
