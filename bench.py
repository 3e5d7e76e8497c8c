"""Benchmark of the AttnRes depth aggregation on one MI355X.

One step = the whole Full AttnRes forward of the DepthBench 400M deep shape
(L = 32 Transformer blocks: 64 sublayers + embedding, d = 896, 8 x 2048 tokens,
bf16 history, fp32 accumulation), executed the way a model executes it: one
library call per read l = 0..64 (each call streams history rows 0..l and
reuses the per-(row, token) RMS-scale cache).  Inputs are synthetic, seeded
and already resident in HBM when the timed region starts.

Printed: ONE JSON line with the throughput (tokens/s), a roofline object for
the dominant kernel (mean algorithmic bytes per launch / mean launch duration,
the latter from HIP events over the timed region, which holds only that
kernel's launches; against 8 TB/s), and the fp64 CPU oracle timed on a bounded
token sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
WORKLOAD = "full_L32_d896"
KERNEL_SOURCES = ["depth_wise_attention_attnres_amd/csrc/full_fwd.hip",
                  "depth_wise_attention_attnres_amd/csrc/device_common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "full_fwd_stream_L32_d896_traffic.json")


def read_bytes_per_token(l: int, d: int) -> int:
    """Algorithmic HBM bytes of read l for one token: rows 0..l (bf16), the
    output row (bf16), l cached RMS scales read, one written, the lse."""
    return (l + 1) * 2 * d + 2 * d + 4 * l + 4 + 4


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken
    on the current kernel source (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, hist, w, target_s: float = 15.0):
    """Time the fp64 oracle on a bounded token sample of the same workload."""
    import numpy as np
    import torch
    import oracle
    from depth_wise_attention_attnres_amd.workloads import token_sample

    def run(n):
        idx = torch.from_numpy(token_sample(wl.T, n, seed=99)).to(hist.device)
        h64 = hist.index_select(1, idx).to(torch.float64).cpu().numpy()
        w64 = w.to(torch.float64).cpu().numpy()
        t0 = time.perf_counter()
        oracle.full_fwd(h64, w64)
        return time.perf_counter() - t0

    def sized(target):
        probe_n = 128
        t_probe = run(probe_n)
        n = int(min(wl.T, max(probe_n, probe_n * target / max(t_probe, 1e-3))))
        n = max(probe_n, (n // 64) * 64)
        return n, run(n)

    cores = oracle.num_threads()
    n, t = sized(target_s)
    # the same oracle on one core, on a smaller sample (per-token cost is uniform)
    oracle.set_num_threads(1)
    try:
        n1, t1 = sized(target_s / 3)
    finally:
        oracle.set_num_threads(cores)
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {
        "value": n / t,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{n} of {wl.T} tokens of {wl.name} (all {wl.n_hist} reads per token, fp64, "
                  f"{t:.1f} s)",
        "single_core": {"value": n1 / t1, "unit": "tokens/s", "cores": 1,
                        "sample": f"{n1} tokens, {t1:.1f} s"},
        "cpu_model": cpu_model,
    }


PROFILE_WORKLOADS = {
    "block_S8_d2048_128k": "Block AttnRes two-phase forward, all 65 reads in one call, S=8",
    "bwd_L24_d1024_full": "Full AttnRes backward, 48 sublayers + embedding, d=1024, 16384 tokens",
    "bwd_L24_d1024_block_S4": "Block AttnRes (S=4) backward, 48 sublayers + embedding, d=1024, 16384 tokens",
    "block_S8_d2048_128k_model_order": "Block AttnRes S=8 in model order (phase 1 per group, phase 2 per row)",
    "full_L32_d896_batched": "Full AttnRes forward, all 65 reads in one call (rows staged in LDS)",
    "proj_L32_d896": "input-dependent query q_l = W_l v_l of all 65 reads, d=896, 16384 tokens",
    "full_L70_d640_batched": "Full AttnRes forward, all 141 reads in one call, d=640, 16384 tokens",
}


def profile_run(name):
    """One history copy (calibration), then the workload twice, for counters."""
    import torch
    import depth_wise_attention_attnres_amd as ar
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs
    dev = torch.device("cuda:0")
    if name.startswith("bwd_"):
        wl = WORKLOADS["fwdbwd_L24_d1024"]
        h, w, g = device_inputs(wl, dev)
        n, T, d = h.shape
        dst = torch.empty_like(h)
        dst.copy_(h)
        del dst
        variant, S = (ar.FULL, 1) if name.endswith("_full") else (ar.BLOCK, wl.S)
        ws = torch.empty(ar.bwd_workspace_bytes(variant, S, n, T, d, 0, n), dtype=torch.uint8,
                         device=dev)
        dh = torch.empty_like(h)
        dw = torch.empty((n, d), dtype=torch.float32, device=dev)
        for _ in range(2):
            ar.bwd(variant, h, w, g, S=S, dhist=dh, dw=dw, workspace=ws)
        torch.cuda.synchronize()
        print(f"profile run done: {name} ({PROFILE_WORKLOADS[name]}), history copy "
              f"{h.numel() * h.element_size()} bytes", flush=True)
        return
    if name == "proj_L32_d896":
        wl = WORKLOADS["full_L32_d896"]
        h, _, _ = device_inputs(wl, dev)
        n, T, d = h.shape
        dst = torch.empty_like(h)
        dst.copy_(h)
        del dst
        gen = torch.Generator(device=dev)
        gen.manual_seed(wl.seed + 101)
        W = (torch.randn((n, d, d), generator=gen, device=dev) * (0.05 / d ** 0.5)).to(torch.bfloat16)
        q = torch.empty((n, T, d), dtype=torch.float32, device=dev)
        for _ in range(2):
            ar.query_proj(h, W, q=q)
        torch.cuda.synchronize()
        print(f"profile run done: {name} ({PROFILE_WORKLOADS[name]}), history copy "
              f"{h.numel() * h.element_size()} bytes", flush=True)
        return
    wl = WORKLOADS[{"full_L32_d896_batched": "full_L32_d896",
                    "full_L70_d640_batched": "full_L70_d640"}.get(name, "block_S8_d2048_128k")]
    h, w, _ = device_inputs(wl, dev)
    n, T, d = h.shape
    dst = torch.empty_like(h)
    dst.copy_(h)
    del dst
    out = torch.empty_like(h)
    lse = torch.empty((n, T), dtype=torch.float32, device=dev)
    if name in ("full_L32_d896_batched", "full_L70_d640_batched"):
        fn = lambda: ar.full_fwd(h, w, out=out, lse=lse)
    elif name == "block_S8_d2048_128k":
        fn = lambda: ar.block_fwd(h, w, wl.S, out=out, lse=lse)
    else:
        S = wl.S
        n_blk = 1 + (n - 1) // S
        st = {"blocks": torch.empty((n_blk, T, d), dtype=torch.float32, device=dev),
              "partial": torch.empty((T, d), dtype=torch.float32, device=dev),
              "rs": torch.empty((n_blk, T), dtype=torch.float32, device=dev),
              "o": torch.empty((S, T, d), dtype=torch.float32, device=dev),
              "lse1": torch.empty((S, T), dtype=torch.float32, device=dev)}
        fn = lambda: ar.block_model_order(h, w, S, out=out, lse=lse, state=st)
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    print(f"profile run done: {name} ({PROFILE_WORKLOADS[name]}), history copy "
          f"{h.numel() * h.element_size()} bytes", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the Block 128K and forward+backward measurements")
    ap.add_argument("--profile", choices=sorted(PROFILE_WORKLOADS),
                    help="for rocprofv3: copy the workload's history once (a transfer of known "
                         "size that calibrates the HBM counters), run the workload twice, exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the AttnRes aggregation "
              "is per-token independent and the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import depth_wise_attention_attnres_amd as ar
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs

    if args.profile:
        profile_run(args.profile)
        return

    wl = WORKLOADS[WORKLOAD]
    dev = torch.device("cuda:0")
    hist, w, _ = device_inputs(wl, dev)
    n, T, d = hist.shape
    rinv = torch.empty((n, T), dtype=torch.float32, device=dev)
    out = torch.empty_like(hist)
    lse = torch.empty((n, T), dtype=torch.float32, device=dev)
    w_rows = [w[l:l + 1] for l in range(n)]
    out_rows = [out[l:l + 1] for l in range(n)]
    lse_rows = [lse[l:l + 1] for l in range(n)]

    def step():
        for l in range(n):
            ar.full_fwd(hist, w_rows[l], q_begin=l, n_q=1, rinv=rinv, rinv_valid_rows=l,
                        out=out_rows[l], lse=lse_rows[l])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # The step is nothing but the n launches of the dominant kernel, back to
    # back on the library's stream (the rocprofv3 trace of this command shows
    # about 1.2 us between launches, 0.7% of the step), so its mean launch
    # duration is taken as the timed region over the launches it holds: HIP
    # events on that stream, over the timed region (the gaps count against it).
    bytes_per_launch = [read_bytes_per_token(l, d) * T for l in range(n)]
    mean_bytes = sum(bytes_per_launch) / n
    mean_ms = ms_per_step / n
    achieved = mean_bytes / (mean_ms * 1e-3) / 1e9

    # diagnostic: the rate of single launches of a few lengths, from HIP events
    # around each launch (these intervals include the launch gaps, so they are
    # a lower bound of each kernel's own rate)
    probe = [0, 8, 16, 32, n - 1]
    ev = {l: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for l in probe}
    torch.cuda.synchronize()
    for l in range(n):
        if l in ev:
            ev[l][0].record(stream)
        ar.full_fwd(hist, w_rows[l], q_begin=l, n_q=1, rinv=rinv, rinv_valid_rows=l,
                    out=out_rows[l], lse=lse_rows[l])
        if l in ev:
            ev[l][1].record(stream)
    torch.cuda.synchronize()
    launch_gbs = {str(l): bytes_per_launch[l] / (ev[l][0].elapsed_time(ev[l][1]) * 1e-3) / 1e9
                  for l in probe}

    # diagnostic (with the extras): the same launches with a 1 GiB fill before
    # each one, which leaves the caches full of dirty lines as a model's
    # sublayer between two reads would; HIP events around each launch only (the
    # fill lies outside them), the best of three sweeps per launch
    cache_cleared = None
    if not args.no_extra:
        junk = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cleared = [float("inf")] * n
        for _ in range(3):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
            for l in range(n):
                junk.fill_(float(l))
                evs[l][0].record(stream)
                ar.full_fwd(hist, w_rows[l], q_begin=l, n_q=1, rinv=rinv, rinv_valid_rows=l,
                            out=out_rows[l], lse=lse_rows[l])
                evs[l][1].record(stream)
            torch.cuda.synchronize()
            cleared = [min(c, a.elapsed_time(b)) for c, (a, b) in zip(cleared, evs)]
        del junk
        cleared_ms = sum(cleared)
        cleared_gbs = sum(bytes_per_launch) / (cleared_ms * 1e-3) / 1e9
        cache_cleared = {
            "what": "kernel time of one step's 65 launches, each after a 1 GiB fill (caches dirty)",
            "kernel_ms_per_step": cleared_ms,
            "achieved_GBps": cleared_gbs,
            "frac": cleared_gbs / HBM_PEAK_GBS,
        }

    # context: a plain device-to-device copy of the same size as one step's
    # history (read + write), the achievable streaming rate of this device
    src = hist.view(-1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * src.element_size() * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del dst

    traffic = load_traffic()
    result = {
        "metric": "AttnRes aggregation tokens/s + achieved HBM GB/s (% of MI355X peak)",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, sigma_i^2) history, sigma growing 1..8; w ~ N(0, 0.02^2))",
        "config": {
            "workload": f"{WORKLOAD}: Full AttnRes forward, read by read (65 calls per step)",
            "n_hist": n, "tokens": T, "d": d, "reads_per_step": n,
            "accumulate": "fp32",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": "full_fwd_stream_kernel<bf16,bf16,16,7,1>",
            "mean_launch_ms": mean_ms,
            "mean_algorithmic_bytes_per_launch": mean_bytes,
            "launch_GBps_by_read": launch_gbs,
        },
        "step_gbs": sum(bytes_per_launch) / (ms_per_step * 1e-3) / 1e9,
        "copy_gbs": copy_gbs,
        "wall_s_timed": wall,
        "device": torch.cuda.get_device_name(dev),
    }
    if cache_cleared is not None:
        result["cache_cleared"] = cache_cleared
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, hist, w)
    if not args.no_extra:
        del hist, out, rinv, lse, src
        torch.cuda.empty_cache()
        result["extra"] = extra_measurements(dev)
    print(json.dumps(result), flush=True)


def _time(fn, stream, reps, warm):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps




def bwd_fmas_per_token(n_hist, n_q, S):
    """Multiply-adds per token and per column of d for one backward: for each
    read, the score and gradient dots of its sources (two per source), the
    value and query paths into every history row it sees (two per row) and
    the dw product (one per row); once per row, the squared norm of the
    source it closes and the coupling term."""
    total = 2 * n_hist
    for l in range(n_q):
        m = l // S
        n_src = m + 1 + (1 if l % S else 0)
        total += 2 * n_src + 3 * (l + 1)
    return total


def full_fwd_fmas_per_token(n_hist, n_q):
    """Multiply-adds per token and per column of d of a Full forward with reads
    0..n_q-1: a score dot and a weighted-sum term per (read, row), and one
    squared norm per row."""
    return n_hist + sum(2 * (l + 1) for l in range(n_q))


def model_order_bytes_per_token(n, d, S, vb=2, ob=2):
    """HBM bytes per token of one model-order Block sweep (phase 1 per group:
    frozen fp32 sources read, new row and partial sum read, new block written,
    the group's fp32 phase-1 sums and log-sum-exps written, the first read's
    output; phase 2 per row: row, partial sum and phase-1 sum read, partial sum
    and output written).  Queries come from L2 and are not counted."""
    total = 0
    n_blk = 1 + (n - 1) // S
    for m in range(n_blk):
        n_reads = min(S, n - m * S)
        total += 4 * d * m + vb * d + (4 * d if (m > 0 and S > 1) else 0) + 4 * d
        total += n_reads * (4 * d + 4) + ob * d + 4 + 4 * (m + 1)
        for k in range(1, n_reads):
            total += vb * d + (4 * d if k > 1 else 0) + 4 * d + 4 + 4 * d + ob * d + 4
    return total


def extra_measurements(dev):
    """The other rows of the hot path at their workload sizes: the Block
    two-phase forward over a 128K-token S=8 history (one call, and in model
    order), the Full forward with all reads in one call (L=32 / d=896 and
    L=70 / d=640) and the L=70 model-order sweep, the input-dependent query,
    and the Full and Block (S=4) forward + backward of the L=24 / d=1024
    workload."""
    import torch
    import depth_wise_attention_attnres_amd as ar
    from depth_wise_attention_attnres_amd.workloads import WORKLOADS, device_inputs

    stream = torch.cuda.current_stream(dev)
    res = {}
    wl = WORKLOADS["block_S8_d2048_128k"]
    h, w, _ = device_inputs(wl, dev)
    n, T, d = h.shape
    out = torch.empty_like(h)
    lse = torch.empty((n, T), dtype=torch.float32, device=dev)
    ms = _time(lambda: ar.block_fwd(h, w, wl.S, out=out, lse=lse), stream, 5, 2)
    nbytes = (n * T * d * 2) * 2 + n * T * 4
    res[wl.name] = {"what": "Block AttnRes two-phase forward, all 65 reads in one call, S=8",
                    "ms": ms, "tokens_per_s": T / (ms * 1e-3),
                    "algorithmic_GBps": nbytes / (ms * 1e-3) / 1e9,
                    "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "algorithmic_bytes": nbytes}
    # the same prefill in model order: one phase-1 call per block group, one
    # phase-2 call per row inside a block (state: fp32 block sums, partial sum,
    # RMS-scale cache, the group's phase-1 results)
    S = wl.S
    n_blk = 1 + (n - 1) // S
    st = {"blocks": torch.empty((n_blk, T, d), dtype=torch.float32, device=dev),
          "partial": torch.empty((T, d), dtype=torch.float32, device=dev),
          "rs": torch.empty((n_blk, T), dtype=torch.float32, device=dev),
          "o": torch.empty((S, T, d), dtype=torch.float32, device=dev),
          "lse1": torch.empty((S, T), dtype=torch.float32, device=dev)}
    ms = _time(lambda: ar.block_model_order(h, w, S, out=out, lse=lse, state=st), stream, 3, 1)
    nbytes = model_order_bytes_per_token(n, d, S) * T
    res[wl.name + "_model_order"] = {
        "what": "Block AttnRes S=8 in model order: attnres_block_phase1 per group + attnres_block_phase2 per row",
        "ms": ms, "tokens_per_s": T / (ms * 1e-3),
        "algorithmic_GBps": nbytes / (ms * 1e-3) / 1e9,
        "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes": nbytes}
    del h, w, out, lse, st
    torch.cuda.empty_cache()

    # Full forward with every read in one call (the rows are shared by the
    # reads, so the call is bound by its arithmetic, not by HBM), and the
    # deep-narrow L=70 / d=640 history in model order and in one call
    for name, model_order in [("full_L32_d896", False), ("full_L70_d640", True),
                              ("full_L70_d640", False)]:
        wl = WORKLOADS[name]
        h, w, _ = device_inputs(wl, dev)
        n, T, d = h.shape
        out = torch.empty_like(h)
        lse = torch.empty((n, T), dtype=torch.float32, device=dev)
        if model_order:
            rinv = torch.empty((n, T), dtype=torch.float32, device=dev)

            def sweep():
                for l in range(n):
                    ar.full_fwd(h, w[l:l + 1], q_begin=l, n_q=1, rinv=rinv, rinv_valid_rows=l,
                                out=out[l:l + 1], lse=lse[l:l + 1])
            ms = _time(sweep, stream, 5, 2)
            nbytes = sum(read_bytes_per_token(l, d) for l in range(n)) * T
            res[name + "_model_order"] = {
                "what": f"Full AttnRes forward in model order ({n} calls, one read each, RMS cache)",
                "ms": ms, "tokens_per_s": T / (ms * 1e-3),
                "algorithmic_GBps": nbytes / (ms * 1e-3) / 1e9,
                "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "algorithmic_bytes": nbytes}
            del rinv
        else:
            ms = _time(lambda: ar.full_fwd(h, w, out=out, lse=lse), stream, 5, 2)
            flops = 2.0 * full_fwd_fmas_per_token(n, n) * d * T
            nbytes = 2 * n * T * d * 2 + n * T * 4
            # bf16 rows and outputs: both contractions on the bf16 matrix cores
            # (split fp32 operands), the softmax and the operand splits on the
            # vector ALU; the useful arithmetic rate and the HBM fraction of the
            # algorithmic bytes (each row read once, each output written once)
            res[name + "_batched"] = {
                "what": f"Full AttnRes forward, all {n} reads in one call",
                "ms": ms, "tokens_per_s": T / (ms * 1e-3),
                "algorithmic_GBps": nbytes / (ms * 1e-3) / 1e9,
                "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "algorithmic_TFLOPs": flops / (ms * 1e-3) / 1e12}
        del h, w, out, lse
        torch.cuda.empty_cache()

    # input-dependent query on the L=32 / d=896 history: the projection of every
    # read's newest row (one call, all reads) and the model-order sweep with a
    # projection per read (synthetic W ~ N(0, 0.05^2 / d), bf16)
    wl = WORKLOADS["full_L32_d896"]
    h, _, _ = device_inputs(wl, dev)
    n, T, d = h.shape
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed + 101)
    W = (torch.randn((n, d, d), generator=gen, device=dev) * (0.05 / d ** 0.5)).to(torch.bfloat16)
    q_all = torch.empty((n, T, d), dtype=torch.float32, device=dev)
    ms_p = _time(lambda: ar.query_proj(h, W, q=q_all), stream, 3, 1)
    flops = 2.0 * n * T * d * d
    q1 = torch.empty((1, T, d), dtype=torch.float32, device=dev)
    rinv = torch.empty((n, T), dtype=torch.float32, device=dev)
    out = torch.empty_like(h)

    def sweep():
        for l in range(n):
            ar.query_proj(h[l:l + 1], W[l:l + 1], q=q1)
            ar.full_fwd_q(h, q1, q_begin=l, rinv=rinv, rinv_valid_rows=l, out=out[l:l + 1],
                          want_lse=False)
    ms_s = _time(sweep, stream, 3, 1)
    res[wl.name + "_input_dependent_query"] = {
        "what": "q_l = W_l v_l (d x d, bf16 matrix cores) + Full AttnRes with per-token queries",
        "proj_all_reads_ms": ms_p, "proj_TFLOPs": flops / (ms_p * 1e-3) / 1e12,
        "proj_frac_of_bf16_dense_peak": flops / (ms_p * 1e-3) / 1e12 / 2500.0,
        "model_order_ms": ms_s, "model_order_tokens_per_s": T / (ms_s * 1e-3)}
    del h, W, q_all, q1, rinv, out
    torch.cuda.empty_cache()

    wl = WORKLOADS["fwdbwd_L24_d1024"]
    h, w, g = device_inputs(wl, dev)
    n, T, d = h.shape
    out = torch.empty_like(h)
    lse = torch.empty((n, T), dtype=torch.float32, device=dev)
    dh = torch.empty_like(h)
    dw = torch.empty((n, d), dtype=torch.float32, device=dev)
    for name, variant, S in [("full", ar.FULL, 1), ("block_S4", ar.BLOCK, wl.S)]:
        ws = torch.empty(ar.bwd_workspace_bytes(variant, S, n, T, d, 0, n), dtype=torch.uint8,
                         device=dev)
        if variant == ar.FULL:
            fwd = lambda: ar.full_fwd(h, w, out=out, lse=lse)
        else:
            fwd = lambda: ar.block_fwd(h, w, S, out=out, lse=lse)
        bwd = lambda: ar.bwd(variant, h, w, g, S=S, dhist=dh, dw=dw, workspace=ws)
        # ten calls after three warm-up calls each (a few ms per call)
        ms_f = _time(fwd, stream, 10, 3)
        ms_b = _time(bwd, stream, 10, 3)
        res[f"{wl.name}_{name}"] = {
            "what": f"{name} forward (all reads, one call) + backward, bf16 in/out, fp32 dw",
            "fwd_ms": ms_f, "bwd_ms": ms_b,
            "fwd_bwd_tokens_per_s": T / ((ms_f + ms_b) * 1e-3),
            "fwd_algorithmic_GBps": (2 * n * T * d * 2) / (ms_f * 1e-3) / 1e9,
            "fwd_frac_of_hbm_peak": (2 * n * T * d * 2) / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS,
            **({"fwd_algorithmic_TFLOPs": 2 * full_fwd_fmas_per_token(n, n) * d * T / (ms_f * 1e-3) / 1e12}
               if variant == ar.FULL else {}),
            # compulsory traffic of the backward: history and dout read, dhist written
            "bwd_algorithmic_GBps": (3 * n * T * d * 2) / (ms_b * 1e-3) / 1e9,
            "bwd_frac_of_hbm_peak": (3 * n * T * d * 2) / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS,
            # useful arithmetic rate (the contractions run on the bf16 matrix
            # cores with split fp32 operands, the per-read softmax work on the
            # vector ALU; each kernel's own roofline is in its profile summary)
            "bwd_algorithmic_TFLOPs": 2 * bwd_fmas_per_token(n, n, S) * d * T / (ms_b * 1e-3) / 1e12,
        }
        del ws
    return res


if __name__ == "__main__":
    main()
