"""The benchmark's algorithmic byte and FMA counts (host logic, no GPU).

bench.py divides these counts by measured time to report GB/s and TFLOP/s, so
a wrong count would misstate every roofline figure.  Each is checked against
the total derived independently from the workload definition: per read l of
a Full model-order sweep, rows 0..l in (bf16), one output row out, the cached
RMS scales of l rows read and one written, the log-sum-exp; per (read, row)
pair a score dot and a weighted-sum term of d multiply-adds each, plus one
squared norm per row; the Block single call reads and writes every row once.
"""
import pytest

import bench

T_16K, T_128K = 16384, 131072


def test_full_model_order_bytes():
    # L=32 / d=896: 65 reads; L=70 / d=640: 141 reads
    b32 = sum(bench.read_bytes_per_token(l, 896) for l in range(65)) * T_16K
    b70 = sum(bench.read_bytes_per_token(l, 640) for l in range(141)) * T_16K
    assert b32 == pytest.approx(65.03e9, rel=2e-4)
    assert b70 == pytest.approx(213.57e9, rel=2e-4)
    # closed form of the same sum: rows sum to n(n+1)/2, scale reads to n(n-1)/2
    n, d = 65, 896
    closed = (2 * d * n * (n + 1) // 2 + 2 * d * n + 4 * n * (n - 1) // 2 + 8 * n) * T_16K
    assert b32 == closed


def test_full_forward_fmas():
    # F = 2 FLOP x FMAs: 127.9 GFLOP at L=32 / d=896, 422.8 at L=70 / d=640
    f32 = 2 * bench.full_fwd_fmas_per_token(65, 65) * 896 * T_16K
    f70 = 2 * bench.full_fwd_fmas_per_token(141, 141) * 640 * T_16K
    assert f32 == pytest.approx(127.86e9, rel=1e-4)
    assert f70 == pytest.approx(422.85e9, rel=1e-4)
    assert bench.full_fwd_fmas_per_token(1, 1) == 3  # one row: a norm, a dot, a term


def test_block_model_order_bytes_exceed_single_call():
    # the model-order Block sweep moves fp32 state between calls: several
    # times the single call's 2 x 65 bf16 rows per token, never less
    n, d, S = 65, 2048, 8
    single = 2 * n * 2 * d
    mo = bench.model_order_bytes_per_token(n, d, S)
    assert single * T_128K == pytest.approx(69.79e9, rel=2e-4)
    assert 4 * single < mo < 6 * single


def test_backward_fmas_full_equals_block_of_one():
    # Full is Block with S = 1, so both formulas agree there
    n = 49
    per_read = sum(2 * (l + 1) + 3 * (l + 1) for l in range(n))
    assert bench.bwd_fmas_per_token(n, n, 1) == 2 * n + per_read


def test_bench_refuses_more_than_one_gpu():
    # the benchmark measures one GPU; --gpus N > 1 exits with a message before
    # touching any device
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU only" in res.stdout + res.stderr
