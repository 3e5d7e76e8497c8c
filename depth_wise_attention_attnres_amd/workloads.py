"""Synthetic workloads for the AttnRes depth aggregation.

Shapes and seeded input draws only -- this module holds none of the method's
arithmetic.  Both the GPU path (tests, benchmark) and the CPU oracle consume
the tensors made here; the oracle always reads back the exact bits the GPU
consumed, so the two never depend on two generators agreeing.

The five workloads mirror the model shapes of the pages:
  * ``full_fp32_small``   -- Full, fp32, 16 sublayers, d=256, 256 tokens.
  * ``full_L32_d896``     -- Full, bf16, the DepthBench 400M deep shape
    (32 Transformer blocks = 64 sublayers + embedding, d=896; "DepthBench"
    reading notes, Table 3), 8 x 2048 tokens (context 2048, sec. 3.2).
  * ``full_L70_d640``     -- Full, bf16, the deepest Table 3 shape (70 blocks,
    140 sublayers, d=640), 16384 tokens.
  * ``block_S8_d2048_128k`` -- Block, S=8 (64 sublayers in 8 blocks, DepthBench
    sec. 2.5), d=2048 (the 1.6B shape), one 128K-token prefill (DataCamp
    explainer, memory-efficient prefill bullet).
  * ``fwdbwd_L24_d1024``  -- Full and Block (S=4) forward + backward,
    48 sublayers + embedding, d=1024 (the 24-layer Table 3 shape), 4 x 4096.

Distributions: history rows are N(0, sigma_i^2) with sigma_i = 1 unless the
workload asks for a per-layer scale growing linearly from 1 to 8; pseudo-queries
are N(0, w_sigma^2); workloads ``full_fp32_small`` and ``full_L70_d640`` set
their last pseudo-query (the LM-head read) to zero; upstream gradients are
N(0, 1).  Every draw is seeded.
"""
from __future__ import annotations

import dataclasses

import numpy as np

# tensor ids mixed into the seed so each tensor has its own stream
HIST, W, DOUT = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    variant: str            # "full", "block" or "full+block"
    dtype: str              # "f32" or "bf16": history / output / dout dtype
    n_hist: int             # embedding + sublayer outputs
    T: int                  # tokens (batch x sequence, flattened)
    d: int                  # model width
    S: int = 1              # block size in sublayer outputs (Block only)
    w_sigma: float = 0.02
    zero_last_w: bool = False
    sigma_growth: bool = False   # per-layer scale growing linearly 1 -> 8
    backward: bool = False
    seed: int = 0

    @property
    def n_q(self) -> int:
        return self.n_hist

    def hist_sigma(self) -> np.ndarray:
        if not self.sigma_growth or self.n_hist == 1:
            return np.ones(self.n_hist)
        return 1.0 + 7.0 * np.arange(self.n_hist) / (self.n_hist - 1)

    def scaled(self, T: int) -> "Workload":
        """The same workload with another token count (tokens are independent)."""
        return dataclasses.replace(self, T=T)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("full_fp32_small", "full", "f32", n_hist=17, T=256, d=256,
                 w_sigma=0.02, zero_last_w=True, seed=0),
        Workload("full_L32_d896", "full", "bf16", n_hist=65, T=16384, d=896,
                 w_sigma=0.02, sigma_growth=True, seed=1),
        Workload("full_L70_d640", "full", "bf16", n_hist=141, T=16384, d=640,
                 w_sigma=0.02, zero_last_w=True, seed=2),
        Workload("block_S8_d2048_128k", "block", "bf16", n_hist=65, T=131072, d=2048,
                 S=8, w_sigma=0.05, seed=3),
        Workload("fwdbwd_L24_d1024", "full+block", "bf16", n_hist=49, T=16384, d=1024,
                 S=4, w_sigma=0.02, backward=True, seed=4),
    ]
}


# ---------------------------------------------------------------------------
# host (numpy) draws: small cases and CPU-only tests

def _rng(seed: int, tensor: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tensor, sub])


def host_normal(shape, *, seed: int, tensor: int, sigma=1.0, sub: int = 0) -> np.ndarray:
    """Seeded N(0, sigma^2) float64 draw (PCG64 stream keyed by seed/tensor/sub)."""
    return _rng(seed, tensor, sub).standard_normal(shape) * sigma


def host_inputs(wl: Workload, *, T: int | None = None):
    """(hist [n_hist,T,d], w [n_q,d], dout or None) as float32 numpy arrays,
    with history / dout values already rounded to the workload dtype."""
    import torch  # rounding to bf16 is done by torch's exact conversion

    T = wl.T if T is None else T
    sig = wl.hist_sigma()
    hist = np.stack([host_normal((T, wl.d), seed=wl.seed, tensor=HIST, sub=i, sigma=sig[i])
                     for i in range(wl.n_hist)]).astype(np.float32)
    w = host_normal((wl.n_q, wl.d), seed=wl.seed, tensor=W, sigma=wl.w_sigma).astype(np.float32)
    if wl.zero_last_w:
        w[-1] = 0.0
    dout = None
    if wl.backward:
        dout = host_normal((wl.n_q, T, wl.d), seed=wl.seed, tensor=DOUT).astype(np.float32)
    if wl.dtype == "bf16":
        hist = torch.from_numpy(hist).to(torch.bfloat16).float().numpy()
        if dout is not None:
            dout = torch.from_numpy(dout).to(torch.bfloat16).float().numpy()
    return hist, w, dout


# ---------------------------------------------------------------------------
# device (torch) draws: the full-size workloads are generated in place on the
# GPU, one history row at a time, so no float32 copy of the whole tensor exists

def torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def device_inputs(wl: Workload, device="cuda", *, T: int | None = None):
    """(hist, w, dout or None) as torch tensors on ``device``; hist and dout in
    the workload dtype, w in float32.  Seeded torch generator on the device."""
    import torch

    T = wl.T if T is None else T
    dt = torch_dtype(wl.dtype)
    gen = torch.Generator(device=device)
    sig = wl.hist_sigma()
    hist = torch.empty((wl.n_hist, T, wl.d), dtype=dt, device=device)
    for i in range(wl.n_hist):
        gen.manual_seed(wl.seed * 1_000_003 + HIST * 10_007 + i)
        row = torch.randn((T, wl.d), generator=gen, device=device, dtype=torch.float32)
        hist[i].copy_(row.mul_(float(sig[i])))
        del row
    gen.manual_seed(wl.seed * 1_000_003 + W * 10_007)
    w = torch.randn((wl.n_q, wl.d), generator=gen, device=device, dtype=torch.float32)
    w.mul_(wl.w_sigma)
    if wl.zero_last_w:
        w[-1].zero_()
    dout = None
    if wl.backward:
        dout = torch.empty((wl.n_q, T, wl.d), dtype=dt, device=device)
        for j in range(wl.n_q):
            gen.manual_seed(wl.seed * 1_000_003 + DOUT * 10_007 + j)
            dout[j].copy_(torch.randn((T, wl.d), generator=gen, device=device,
                                      dtype=torch.float32))
    return hist, w, dout


def token_sample(T: int, n: int, seed: int = 12345) -> np.ndarray:
    """Sorted token indices: the first and last 256 tokens plus a seeded
    uniform sample, ``n`` in total (all tokens when n >= T)."""
    if n >= T:
        return np.arange(T)
    edge = min(256, n // 4)
    head = np.arange(edge)
    tail = np.arange(T - edge, T)
    middle = np.setdiff1d(np.arange(T), np.concatenate([head, tail]))
    rng = np.random.default_rng(seed)
    pick = rng.choice(middle, size=n - 2 * edge, replace=False)
    return np.sort(np.concatenate([head, pick, tail]))
