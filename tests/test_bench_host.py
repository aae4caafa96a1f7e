"""Host-side logic of bench.py, on the CPU: the algorithmic FLOP counts that
every roofline figure divides by, the one-GPU refusal, and the rule that the
traffic figure is only read from a byte-counter summary taken on the current
kernel source."""
import hashlib
import os

import numpy as np
import pytest

import bench


def test_forward_flops_match_the_closed_form():
    # d * sum_i (i + 1) * (10 + 6 T) per head: 4d moment scan, 6d per CG
    # iteration, 6d output scan per causal pair
    n, d, T, heads = 4096, 128, 16, 32
    iters = np.full((4, 8, n), T, dtype=np.int32)
    pairs = n * (n + 1) // 2
    assert bench.algorithmic_flops(n, d, iters) == d * pairs * (10 + 6 * T) * heads
    assert bench.algorithmic_flops(n, d, iters) == 3_643_021_459_456
    assert bench.cg_flops(n, d, iters) == d * pairs * 6 * T * heads
    assert bench.backward_flops(n, d, iters) == d * pairs * (36 + 6 * T) * heads
    # without the score products re-formed in each sweep: 8d + 4d per iteration
    assert bench.min_flops(n, d, iters) == d * pairs * (8 + 4 * T) * heads


def test_flops_count_each_query_with_its_own_iterations():
    n, d = 5, 16
    iters = np.array([[[0, 1, 2, 3, 4]]], dtype=np.int32)
    expect = d * sum((i + 1) * (10 + 6 * t) for i, t in enumerate(range(5)))
    assert bench.algorithmic_flops(n, d, iters) == expect
    assert bench.cg_flops(n, d, iters) == d * sum((i + 1) * 6 * t for i, t in enumerate(range(5)))


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("current", [True, False])
def test_traffic_only_from_a_summary_of_the_current_kernel(tmp_path, current):
    src = os.path.join(bench.ROOT, "local_linear_attention_flashlla_amd", "csrc", "lla_mfma.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest() if current else "0" * 64
    p = tmp_path / "summary.txt"
    p.write_text(f"lla_mfma.hip sha256: {sha}\n\nbytes_per_launch cg_kernel: 1.2345e+09\n")
    got = bench.measured_traffic(str(p))
    assert got == (1.2345e9 if current else None)
    assert bench.measured_traffic(str(tmp_path / "missing.txt")) is None
