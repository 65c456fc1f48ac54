"""CPU checks of the bench's accounting: FLOP counts and the HBM traffic
models it prints next to the measured traffic."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synthetic  # noqa: E402


def test_flops_of_the_throughput_workload():
    # 4 N^2 d per head, halved for the causal mask: 4.398e12 at B8 H32 N8192 d128
    assert bench.attention_flops(8, 32, 8192, 128, True) == 2 * 8192 ** 2 * 128 * 8 * 32
    assert bench.attention_flops(1, 1, 10, 4, False) == 4 * 100 * 4


def test_causal_row_flops_counts_visible_keys():
    assert bench.causal_row_flops([0, 1, 9], 4) == 4 * 4 * (1 + 2 + 10)


def test_traffic_models_of_the_throughput_workload():
    m = bench.traffic_models(synthetic.WORKLOADS[3], 128)
    # compulsory: Q, K, V read and O written once (8 N d bytes per head) plus L (4 N)
    assert m["compulsory"] == 256 * (8 * 8192 * 128 + 4 * 8192) == 2155872256
    # Theta(N^2 d^2 / M), M = 160 KB of bf16 = 81920 elements, in bytes
    assert m["theta_N2d2_over_M"] == round(256 * 8192 ** 2 * 128 ** 2 * 2 / 81920)
    # no reuse: block i of 128 rows re-reads the K/V rows 0 .. 128(i + 1) - 1
    kv_rows = sum(128 * (i + 1) for i in range(64))
    assert m["no_reuse_per_query_block"] == 256 * (2 * 2 * 128 * kv_rows + 2 * 8192 * 128 * 2 + 4 * 8192)
    assert 34e9 < m["no_reuse_per_query_block"] < 37e9


def test_traffic_models_non_causal_and_ragged():
    w = synthetic.Workload(0, "", 1, 1, 300, 64, "bf16", False)
    m = bench.traffic_models(w, 128)
    assert m["no_reuse_per_query_block"] == 2 * 2 * 64 * 3 * 300 + 2 * 300 * 64 * 2 + 4 * 300
