"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test names the property it checks and where it comes from.  None of them
retypes the oracle's formula: they use hand-derived closed forms, limits,
invariances, the pages' FLOP counts, brute-force enumeration and finite
differences.  Page short names: DepthBench reading notes ("DB"), the wln20
LLMRes post ("LR"), the jaimeyzzz Kimi K3 notes ("K3N"), the DataCamp
explainer ("DC").
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


# ---------------------------------------------------------------------------
# worked examples (tests/golden/worked_examples.json, hand-derived closed forms)

def test_worked_examples(oracle):
    spec = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))
    for ex in spec["examples"]:
        hist = np.array(ex["hist"], dtype=np.float64)
        w = np.array(ex["w"], dtype=np.float64)
        variant = oracle.FULL if ex["variant"] == "full" else oracle.BLOCK
        out, lse, alpha = oracle.fwd(variant, hist, w, S=ex["S"], q_begin=ex.get("q_begin", 0),
                                     eps=ex["eps"], want_alpha=True)
        np.testing.assert_allclose(out, np.array(ex["out"]), rtol=0, atol=1e-14, err_msg=ex["name"])
        np.testing.assert_allclose(lse, np.array(ex["lse"]), rtol=0, atol=1e-14, err_msg=ex["name"])
        np.testing.assert_allclose(alpha, np.array(ex["alpha"]), rtol=0, atol=1e-14,
                                   err_msg=ex["name"])


# ---------------------------------------------------------------------------
# w = 0: uniform average over the sources (K3N sec. 5: w_l = 0 reduces to a
# uniform mean; LR "Kimi AttnRes": zero-initialised queries give equal weights,
# like the standard residual).  Full: (l+1) h_l is the Pre-LN residual stream
# v_0 + ... + v_l (LR, the unrolled PreNorm recurrence).

def test_zero_query_full_is_prefix_mean(oracle):
    n_hist, T, d = 7, 5, 12
    hist = _rand((n_hist, T, d), 1)
    w = np.zeros((n_hist, d))
    out, lse = oracle.full_fwd(hist, w)
    stream = np.cumsum(hist, axis=0)          # Pre-LN residual stream after each row
    for l in range(n_hist):
        np.testing.assert_allclose((l + 1) * out[l], stream[l], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[l], math.log(l + 1), atol=1e-14)


def test_zero_query_block_is_stream_over_source_count(oracle):
    # The sources of a Block read partition rows 0..l (embedding, whole blocks,
    # the partial), so at w = 0 the read is the residual stream divided by the
    # number of sources: 1 + floor(l/S) + [l mod S != 0].
    n_hist, T, d = 12, 3, 8
    hist = _rand((n_hist, T, d), 2)
    w = np.zeros((n_hist, d))
    stream = np.cumsum(hist, axis=0)
    for S in (1, 2, 3, 4, 11, 20):
        out, _ = oracle.block_fwd(hist, w, S)
        for l in range(n_hist):
            n_src = 1 + l // S + (1 if l % S else 0)
            np.testing.assert_allclose(n_src * out[l], stream[l], rtol=1e-13, atol=1e-13,
                                       err_msg=f"S={S} l={l}")


# ---------------------------------------------------------------------------
# weights are non-negative and sum to one (DB sec. 2.3; LR "Kimi AttnRes")

@pytest.mark.parametrize("variant,S", [(0, 1), (1, 1), (1, 3), (1, 4)])
def test_alpha_on_simplex(oracle, variant, S):
    n_hist, T, d = 10, 6, 16
    hist = _rand((n_hist, T, d), 3) * np.linspace(1, 8, n_hist)[:, None, None]
    w = _rand((n_hist, d), 4, sigma=0.5)
    _, _, alpha = oracle.fwd(variant, hist, w, S=S, want_alpha=True)
    assert (alpha >= 0).all()
    np.testing.assert_allclose(alpha.sum(-1), 1.0, atol=1e-12)
    for l in range(n_hist):
        n_src = oracle.num_sources(variant, l, S)
        assert (alpha[l, :, n_src:] == 0).all()


# ---------------------------------------------------------------------------
# a read with one source returns it (DB sec. 2.3: the first sublayer reads the
# embedding directly)

def test_single_source_read_is_identity(oracle):
    T, d = 4, 9
    hist = _rand((1, T, d), 5)
    w = _rand((1, d), 6)
    out, lse = oracle.full_fwd(hist, w)
    assert np.array_equal(out[0], hist[0])
    # lse of a single source is its own score r(v) (w.v); with v a +-a vector
    # r(v) = 1/|a| when eps = 0
    a = 3.0
    v = a * np.array([1, -1, 1, 1, -1, 1, 1, 1, -1], dtype=np.float64)
    out, lse = oracle.full_fwd(v[None, None, :], w, eps=0.0)
    assert np.array_equal(out[0, 0], v)
    np.testing.assert_allclose(lse[0, 0], w[0] @ (v / a), atol=1e-14)


def test_eps_sits_inside_the_root(oracle):
    # RMSNorm(v) = v / sqrt(mean(v^2) + eps): for a +-a vector the key scale is
    # 1/sqrt(a^2 + eps); with a = 1, eps = 3 it is exactly 1/2.
    d = 8
    v = np.array([1, -1, -1, 1, 1, 1, -1, 1], dtype=np.float64)
    w = _rand((1, d), 61)
    _, lse = oracle.full_fwd(v[None, None, :], w, eps=3.0)
    np.testing.assert_allclose(lse[0, 0], 0.5 * (w[0] @ v), rtol=1e-15)


# ---------------------------------------------------------------------------
# two sources: the softmax is a logistic function of the score difference.
# Sources are scaled +-1 vectors, whose RMSNorm is the +-1 vector itself
# (eps = 0), so the scores are plain dot products; the scales a, b must not
# matter (RMSNorm on the key, DC: large layers must not dominate by scale).

@pytest.mark.parametrize("a,b", [(1.0, 1.0), (0.25, 7.0), (5.0, 0.01)])
def test_two_sources_logistic_and_scale_free(oracle, a, b):
    d = 16
    rng = np.random.default_rng(7)
    u0 = rng.choice([-1.0, 1.0], size=d)
    u1 = rng.choice([-1.0, 1.0], size=d)
    w = rng.standard_normal((1, d)) * 0.3
    hist = np.stack([a * u0, b * u1])[:, None, :]
    out, _ = oracle.full_fwd(hist, w, q_begin=1, n_q=1, eps=0.0)
    s0, s1 = w[0] @ u0, w[0] @ u1
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    expect = sig(s1 - s0) * hist[1, 0] + sig(s0 - s1) * hist[0, 0]
    np.testing.assert_allclose(out[0, 0], expect, rtol=1e-13, atol=1e-13)


def test_identical_sources_return_that_source(oracle):
    n_hist, T, d = 6, 3, 10
    row = _rand((1, T, d), 8)
    hist = np.repeat(row, n_hist, axis=0)
    w = _rand((n_hist, d), 9)
    out, _ = oracle.full_fwd(hist, w)
    for l in range(n_hist):
        np.testing.assert_allclose(out[l], row[0], rtol=1e-14, atol=1e-14)


def test_key_scale_invariance(oracle):
    # v_i -> c_i v_i (c_i > 0) leaves the weights unchanged when eps = 0
    n_hist, T, d = 8, 4, 16
    hist = _rand((n_hist, T, d), 10)
    w = _rand((n_hist, d), 11, sigma=0.3)
    c = np.exp(_rand((n_hist, T, 1), 12))
    _, _, a1 = oracle.full_fwd(hist, w, eps=0.0, want_alpha=True)
    _, _, a2 = oracle.full_fwd(hist * c, w, eps=0.0, want_alpha=True)
    np.testing.assert_allclose(a1, a2, rtol=1e-12, atol=1e-15)
    # with eps = 1e-6 the change is O(eps / mean square)
    _, _, a3 = oracle.full_fwd(hist * c, w, eps=1e-6, want_alpha=True)
    assert np.abs(a3 - a1).max() < 1e-4


def test_hard_selection_limit(oracle):
    # w -> lambda w, lambda -> infinity: the read selects the top-scoring source
    n_hist, T, d = 6, 5, 12
    hist = _rand((n_hist, T, d), 13)
    w = _rand((n_hist, d), 14)
    _, _, a1 = oracle.full_fwd(hist, w, want_alpha=True)
    out, _ = oracle.full_fwd(hist, 1e5 * w)
    for l in range(1, n_hist):
        for t in range(T):
            top = np.sort(a1[l, t, : l + 1])
            if top[-1] - top[-2] < 1e-3:
                continue
            i = int(np.argmax(a1[l, t]))
            np.testing.assert_allclose(out[l, t], hist[i, t], atol=1e-10)


# ---------------------------------------------------------------------------
# Block reading

def test_block_sources_match_model_order_process(oracle):
    # Brute force: run the model in order, appending sublayer outputs; every S
    # outputs freeze the running block into a summary (DB sec. 2.5, DC block
    # section).  Read l happens after output l is appended.
    for S in (1, 2, 3, 4, 8, 50):
        frozen, partial = [], []
        for l in range(0, 66):
            if l >= 1:
                partial.append(l)
                if len(partial) == S:
                    frozen.append(tuple(partial))
                    partial = []
            m, b, e = oracle.block_sources(l, S)
            assert m == len(frozen), (S, l)
            assert list(range(b, e)) == partial, (S, l)
            for c, rows in enumerate(frozen, start=1):
                assert rows == tuple(range((c - 1) * S + 1, c * S + 1))
            assert oracle.num_sources(1, l, S) == 1 + len(frozen) + (1 if partial else 0)


def test_block_S1_equals_full(oracle):
    n_hist, T, d = 9, 4, 16
    hist = _rand((n_hist, T, d), 15) * np.linspace(1, 8, n_hist)[:, None, None]
    w = _rand((n_hist, d), 16, sigma=0.4)
    o_full, l_full = oracle.full_fwd(hist, w)
    o_blk, l_blk = oracle.block_fwd(hist, w, 1)
    np.testing.assert_allclose(o_blk, o_full, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l_blk, l_full, rtol=1e-13, atol=1e-13)


def test_block_whole_history_one_block(oracle):
    # S >= number of sublayer outputs: every read sees {v_0, p_l}; with +-1
    # construction the two-source logistic closed form applies.
    n_hist, d = 6, 16
    rng = np.random.default_rng(17)
    u = rng.choice([-1.0, 1.0], size=(n_hist, d))
    hist = u[:, None, :].copy()
    w = rng.standard_normal((n_hist, d)) * 0.3
    out, _ = oracle.block_fwd(hist, w, S=n_hist + 3, eps=0.0)
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    for l in range(1, n_hist):
        p = hist[1 : l + 1, 0].sum(0)
        rp = 1.0 / math.sqrt((p * p).mean())
        s0, sp = w[l] @ u[0], rp * (w[l] @ p)
        expect = sig(sp - s0) * p + sig(s0 - sp) * hist[0, 0]
        np.testing.assert_allclose(out[l, 0], expect, rtol=1e-12, atol=1e-12)


def test_block_boundary_reads_equal_full_over_summaries(oracle):
    # At l = mS the partial is empty: the Block read is the Full read over the
    # compressed history [v_0, b_1, ..., b_m].
    S, n_blocks, T, d = 3, 4, 5, 8
    n_hist = 1 + S * n_blocks
    hist = _rand((n_hist, T, d), 18)
    w = _rand((n_hist, d), 19, sigma=0.5)
    out, lse = oracle.block_fwd(hist, w, S)
    comp = np.concatenate([hist[:1]] + [hist[1 + c * S : 1 + (c + 1) * S].sum(0, keepdims=True)
                                        for c in range(n_blocks)])
    for m in range(n_blocks + 1):
        l = m * S
        o2, l2 = oracle.full_fwd(comp[: m + 1], w[l : l + 1], q_begin=m, n_q=1)
        np.testing.assert_allclose(out[l], o2[0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[l], l2[0], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("S", [1, 2, 3, 4, 8])
def test_two_phase_equals_single_pass(oracle, S):
    # DC "两阶段计算": phase 1 over frozen sources + online-softmax merge of the
    # partial sum gives the same read as one softmax over all sources.
    n_hist, T, d = 19, 5, 24
    hist = _rand((n_hist, T, d), 20 + S)
    w = _rand((n_hist, d), 30 + S, sigma=0.5)
    o1, l1 = oracle.block_fwd(hist, w, S)
    o2, l2 = oracle.block_fwd_twophase(hist, w, S)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# the read is a softmax over a set: permuting its sources changes nothing

def test_permutation_invariance_full(oracle):
    n_hist, T, d = 8, 4, 12
    hist = _rand((n_hist, T, d), 40)
    w = _rand((1, d), 41, sigma=0.5)
    perm = np.random.default_rng(42).permutation(n_hist)
    o1, l1 = oracle.full_fwd(hist, w, q_begin=n_hist - 1, n_q=1)
    o2, l2 = oracle.full_fwd(hist[perm], w, q_begin=n_hist - 1, n_q=1)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


def test_permutation_invariance_block(oracle):
    S, T, d = 3, 4, 8
    n_hist = 1 + 3 * S + 2        # three whole blocks and a partial of two
    hist = _rand((n_hist, T, d), 43)
    w = _rand((n_hist, d), 44, sigma=0.5)
    o1, _ = oracle.block_fwd(hist, w, S)
    # (a) permute the rows inside block 2 (rows 4..6): reads from l = 6 on are unchanged
    h2 = hist.copy()
    h2[4:7] = hist[[6, 4, 5]]
    o2, _ = oracle.block_fwd(h2, w, S)
    np.testing.assert_allclose(o2[6:], o1[6:], rtol=1e-13, atol=1e-13)
    # (b) swap whole blocks 1 and 3: reads from l = 9 on are unchanged
    h3 = hist.copy()
    h3[1:4], h3[7:10] = hist[7:10], hist[1:4]
    o3, _ = oracle.block_fwd(h3, w, S)
    np.testing.assert_allclose(o3[9:], o1[9:], rtol=1e-13, atol=1e-13)
    # sanity: a read that does see the difference changes
    assert np.abs(o3[4] - o1[4]).max() > 1e-6


# ---------------------------------------------------------------------------
# backward: central finite differences of L = sum(out * dout) in fp64

def _loss(oracle, variant, S, hist, w, dout, eps):
    out, _ = oracle.fwd(variant, hist, w, S=S, eps=eps)
    return float((out * dout).sum())


@pytest.mark.parametrize("variant,S,n_hist,T,d", [
    (0, 1, 5, 2, 5), (0, 1, 6, 3, 4), (1, 2, 6, 2, 5), (1, 3, 6, 3, 4), (1, 1, 4, 2, 3),
    (1, 5, 6, 2, 4)])
def test_backward_matches_finite_differences(oracle, variant, S, n_hist, T, d):
    rng = np.random.default_rng(100 + 7 * n_hist + d + S)
    hist = rng.standard_normal((n_hist, T, d)) * np.linspace(1, 3, n_hist)[:, None, None]
    w = rng.standard_normal((n_hist, d)) * 0.7
    dout = rng.standard_normal((n_hist, T, d))
    eps = 1e-6
    dhist, dw = oracle.bwd(variant, hist, w, dout, S=S, eps=eps)
    h = 1e-6
    num_h = np.zeros_like(hist)
    for idx in np.ndindex(hist.shape):
        hp, hm = hist.copy(), hist.copy()
        hp[idx] += h
        hm[idx] -= h
        num_h[idx] = (_loss(oracle, variant, S, hp, w, dout, eps)
                      - _loss(oracle, variant, S, hm, w, dout, eps)) / (2 * h)
    num_w = np.zeros_like(w)
    for idx in np.ndindex(w.shape):
        wp, wm = w.copy(), w.copy()
        wp[idx] += h
        wm[idx] -= h
        num_w[idx] = (_loss(oracle, variant, S, hist, wp, dout, eps)
                      - _loss(oracle, variant, S, hist, wm, dout, eps)) / (2 * h)
    scale_h = np.abs(num_h).max()
    scale_w = np.abs(num_w).max()
    assert np.abs(dhist - num_h).max() <= 1e-6 * scale_h
    assert np.abs(dw - num_w).max() <= 1e-6 * scale_w


def test_backward_zero_query_closed_form(oracle):
    # At w = 0 every read is the uniform mean of its sources and the score
    # path vanishes, so each row i gets sum over reads l >= i of g_l / n_src(l)
    # (Full: n_src = l + 1).
    n_hist, T, d = 9, 3, 8
    hist = _rand((n_hist, T, d), 50)
    dout = _rand((n_hist, T, d), 51)
    w = np.zeros((n_hist, d))
    for variant, S in ((0, 1), (1, 2), (1, 4)):
        dhist, _ = oracle.bwd(variant, hist, w, dout, S=S)
        for i in range(n_hist):
            expect = sum(dout[l] / oracle.num_sources(variant, l, S) for l in range(i, n_hist))
            np.testing.assert_allclose(dhist[i], expect, rtol=1e-13, atol=1e-13)
        if variant == 0:
            for i in range(n_hist):
                expect = sum(dout[l] / (l + 1) for l in range(i, n_hist))
                np.testing.assert_allclose(dhist[i], expect, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# Source-read counts vs the FLOP accounting of DB Appendix D (sec. 4.7):
#   Delta F_Full  = 4 T d L (2L + 3)
#   Delta F_Block = 4 T d [ sum_{k=1}^{2L-1} (2 + floor(k/b)) + 9 ],  b = 2L/8
# (4 T d FLOPs per source read: 2d for the score, 2d for the weighted sum).
# Reads 1..2L are counted (read 0 copies the embedding).  The page counts a
# partial sum for every sublayer; at the 7 interior block boundaries the
# partial is empty in our reading, so ours is the page's count minus 7.

@pytest.mark.parametrize("L", [16, 20, 24, 28, 32])
def test_source_reads_match_appendix_d(oracle, L):
    T, d = 1, 1
    full = sum(oracle.num_sources(0, l) for l in range(1, 2 * L + 1))
    assert 4 * T * d * full == 4 * T * d * L * (2 * L + 3)
    b = 2 * L // 8
    page_block = sum(2 + k // b for k in range(1, 2 * L)) + 9
    ours = sum(oracle.num_sources(1, l, b) for l in range(1, 2 * L + 1))
    assert ours == page_block - 7


# ---------------------------------------------------------------------------
# helpers used by the parity tests

def test_round_to_bf16_matches_torch(oracle):
    import torch
    x = np.random.default_rng(60).standard_normal(100000).astype(np.float32) * 50
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3e38, 1e-40])])
    mine = oracle.round_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(mine, ref)
    assert (oracle.ulp_bf16(np.array([1.0, 1.5, 8.0, 15.9]))
            == np.array([2 ** -7, 2 ** -7, 2 ** -4, 2 ** -4])).all()


# ---------------------------------------------------------------------------
# pre-norm of the mixture (the branch input RMSNorm_pre,l(z_l))

def test_prenorm_worked_example(oracle):
    spec = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))
    for ex in spec["prenorm_examples"]:
        y = oracle.prenorm(np.array(ex["z"]), np.array(ex["gain"]), eps=ex["eps"])
        np.testing.assert_allclose(y, np.array(ex["y"]), rtol=1e-15, atol=0, err_msg=ex["name"])


def test_prenorm_unit_rms_and_scale_free(oracle):
    rng = np.random.default_rng(21)
    z = rng.standard_normal((3, 5, 48)) * rng.uniform(0.1, 9.0, (3, 5, 1))
    y = oracle.prenorm(z, eps=0.0)
    np.testing.assert_allclose((y * y).mean(-1), 1.0, rtol=1e-13)  # unit gain: RMS 1
    np.testing.assert_allclose(oracle.prenorm(7.5 * z, eps=0.0), y, rtol=1e-13)  # scale-free
    np.testing.assert_allclose(oracle.prenorm(-z, eps=0.0), -y, rtol=0, atol=0)  # odd
    # the direction is kept: y is a positive multiple of z
    cos = (y * z).sum(-1) / np.sqrt((y * y).sum(-1) * (z * z).sum(-1))
    np.testing.assert_allclose(cos, 1.0, rtol=1e-13)


def test_prenorm_gain_is_elementwise(oracle):
    rng = np.random.default_rng(22)
    z = rng.standard_normal((2, 4, 16))
    g = rng.standard_normal((2, 16))
    y1 = oracle.prenorm(z, eps=1e-6)
    yg = oracle.prenorm(z, g, eps=1e-6)
    np.testing.assert_allclose(yg, g[:, None, :] * y1, rtol=1e-14, atol=1e-15)


def test_prenorm_eps_inside_the_root(oracle):
    # a constant vector c: y = c / sqrt(c^2 + eps); the zero vector stays zero
    c, eps = 0.01, 1e-4
    y = oracle.prenorm(np.full((1, 1, 8), c), eps=eps)
    np.testing.assert_allclose(y, c / np.sqrt(c * c + eps), rtol=1e-14)
    assert np.array_equal(oracle.prenorm(np.zeros((1, 2, 8)), eps=eps), np.zeros((1, 2, 8)))


# ---------------------------------------------------------------------------
# input-dependent query (projection of the current hidden state)

def test_query_proj_worked_example(oracle):
    spec = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))
    for ex in spec["query_proj_examples"]:
        q = oracle.query_proj(np.array(ex["x"]), np.array(ex["W"]))
        np.testing.assert_array_equal(q, np.array(ex["q"]), err_msg=ex["name"])


@pytest.mark.parametrize("variant,S", [(0, 1), (1, 3)])
def test_tokq_zero_projection_is_the_zero_query(oracle, variant, S):
    rng = np.random.default_rng(31)
    hist = rng.standard_normal((8, 5, 16))
    q = np.zeros((8, 5, 16))
    out, lse = oracle.fwd_tokq(variant, hist, q, S=S)
    ref, ref_lse = oracle.fwd(variant, hist, np.zeros((8, 16)), S=S)
    np.testing.assert_allclose(out, ref, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-15)


@pytest.mark.parametrize("variant,S", [(0, 1), (1, 2)])
def test_tokq_shared_state_equals_fixed_query(oracle, variant, S):
    # every token has the same current state x_l, so q_l = W_l x_l is one query
    # per read: the per-token path must equal the pinned fixed-query forward
    rng = np.random.default_rng(32)
    n, T, d = 7, 6, 12
    hist = rng.standard_normal((n, T, d))
    W = rng.standard_normal((n, d, d)) * 0.1
    xs = rng.standard_normal((n, 1, d))
    q = oracle.query_proj(np.repeat(xs, T, axis=1), W)
    out, lse = oracle.fwd_tokq(variant, hist, q, S=S)
    ref, ref_lse = oracle.fwd(variant, hist, q[:, 0, :], S=S)
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-14)


def test_tokq_follows_its_token(oracle):
    # permuting the tokens of the history and of the queries permutes the outputs
    rng = np.random.default_rng(33)
    n, T, d = 6, 9, 8
    hist = rng.standard_normal((n, T, d))
    q = rng.standard_normal((n, T, d)) * 0.4
    perm = rng.permutation(T)
    out, _ = oracle.fwd_tokq(0, hist, q)
    out_p, _ = oracle.fwd_tokq(0, hist[:, perm], q[:, perm])
    np.testing.assert_allclose(out_p, out[:, perm], rtol=0, atol=0)
    # and a per-token query is really used: two tokens with equal histories but
    # different queries read differently
    hist2 = np.repeat(hist[:, :1], 2, axis=1)
    q2 = np.stack([q[:, 0], -q[:, 0]], axis=1)
    out2, _ = oracle.fwd_tokq(0, hist2, q2)
    assert np.abs(out2[-1, 0] - out2[-1, 1]).max() > 1e-3
