"""Pins of the roofline accounting used by the benchmark."""
import os

from linear_attention_kda_amd import perfmodel

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "cost_model_example.txt")


def test_cost_model_matches_the_pages_worked_example():
    """The page prints about 1e11 FLOPs for T=1e6, d=128, C=64 (one head); the
    formula gives 1.27e11, i.e. the same order the page rounds to."""
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    T, d, C, printed = int(rows[0][0]), int(rows[0][1]), int(rows[0][2]), float(rows[0][3])
    f = perfmodel.flops_per_head(T, d, C)
    assert f == 6 * T * d * d + 3 * T * C * d + T * C * C
    assert 0.9 * printed <= f <= 1.5 * printed


def test_bytes_per_token_head():
    # q, k, v, o bf16 + g fp32 + beta fp32
    assert perfmodel.bytes_per_token_head() == 1540
    # scalar gate: one fp32 per token and head instead of 128
    assert perfmodel.bytes_per_token_head(scalar_gate=True) == 1032


def test_varlen_workload_bytes():
    # 65536 tokens, 32 heads, bf16 states in and out for 16 sequences
    b = perfmodel.workload_bytes(65536, 32, 16, 2, 2)
    assert b == 65536 * 32 * 1540 + 2 * 16 * 32 * 128 * 128 * 2


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 (or a multi-rank launch) exits with
    status 2 and says so, before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args],
                           capture_output=True, text=True, env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2, (args, env, r.stderr[-300:])
        assert "one GPU" in r.stderr
