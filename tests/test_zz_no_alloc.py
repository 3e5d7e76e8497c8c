"""attnres_bwd_noalloc (the backward with the library's static device
workspace, for callers that cannot allocate) against attnres_bwd with a
caller workspace: the same kernels, so the results must be bitwise equal.
Two calls in a row, the second smaller, so stale contents of the shared
static array from the first call would show in the second."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FULL, BLOCK = 0, 1


@pytest.fixture(scope="module")
def ar():
    import depth_wise_attention_attnres_amd as ar
    return ar


def _case(n_hist, T, d, seed, dtype, n_q=None, q_begin=0):
    rng = np.random.default_rng(seed)
    n_q = n_hist - q_begin if n_q is None else n_q
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    h = torch.from_numpy(rng.standard_normal((n_hist, T, d)).astype(np.float32)).to(DEV).to(tdt)
    w = torch.from_numpy((rng.standard_normal((n_q, d)) * 0.3).astype(np.float32)).to(DEV)
    g = torch.from_numpy(rng.standard_normal((n_q, T, d)).astype(np.float32)).to(DEV).to(tdt)
    return h, w, g


def _both(ar, variant, S, h, w, g, q_begin=0):
    dh_ref, dw_ref = ar.bwd(variant, h, w, g, S=S, q_begin=q_begin)
    dh = torch.full_like(dh_ref, float("nan"))
    dw = torch.full_like(dw_ref, float("nan"))
    ar.bwd_noalloc(variant, h, w, g, dh, dw, S=S, q_begin=q_begin)
    torch.cuda.synchronize()
    return (dh, dw), (dh_ref, dw_ref)


def test_noalloc_matches_bwd_two_calls_second_smaller(ar):
    # first call: Block S=4, bf16, 300 tokens, d = 512 (about 13 MB of workspace)
    h, w, g = _case(25, 300, 512, seed=1, dtype="bf16")
    (dh, dw), (dh_ref, dw_ref) = _both(ar, BLOCK, 4, h, w, g)
    assert torch.equal(dh, dh_ref) and torch.equal(dw, dw_ref)
    # second call: Full, fp32, fewer rows, tokens and columns, reads from row 3
    h, w, g = _case(9, 37, 64, seed=2, dtype="f32", q_begin=3)
    (dh, dw), (dh_ref, dw_ref) = _both(ar, FULL, 1, h, w, g, q_begin=3)
    assert torch.equal(dh, dh_ref) and torch.equal(dw, dw_ref)


def test_noalloc_accumulate(ar):
    h, w, g = _case(13, 50, 136, seed=3, dtype="bf16")
    dh_ref, dw_ref = ar.bwd(BLOCK, h, w, g, S=3, dhist_dtype=torch.float32)
    start_h = torch.randn(dh_ref.shape, generator=torch.Generator().manual_seed(5)).to(DEV)
    start_w = torch.randn(dw_ref.shape, generator=torch.Generator().manual_seed(6)).to(DEV)
    dh, dw = start_h.clone(), start_w.clone()
    ar.bwd_noalloc(BLOCK, h, w, g, dh, dw, S=3, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dh, start_h + dh_ref) and torch.equal(dw, start_w + dw_ref)


def test_noalloc_rejects_calls_beyond_the_static_workspace(ar):
    need = ar.bwd_workspace_bytes(FULL, 1, 49, 4096, 1024, 0, 49)
    assert need > ar.bwd_noalloc_max_workspace()
    h = torch.zeros((49, 4096, 1024), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((49, 1024), dtype=torch.float32, device=DEV)
    dh = torch.empty_like(h)
    dw = torch.empty_like(w)
    with pytest.raises(ar.AttnResError, match="static scratch"):
        ar.bwd_noalloc(FULL, h, w, h, dh, dw)
