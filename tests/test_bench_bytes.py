"""CPU: the byte counts behind every GB/s figure bench.py reports.

The unfused and fused element counts are pinned to the figures printed in
"CMU 15-779 Lecture 8: ML Compilers Part 1, Tile-based DSLs", section 3, for
the 1823 x 781 softmax (tests/golden/cmu15779_l8_softmax_counts.txt): five
separate kernels read 7,122,461 and write 4,274,935 elements, the fused
kernel reads and writes 1,423,763 each, about 4x less traffic. The fused
count is "Stax (4): GPU Codegen and Dynamic Shapes", 9.5's lower bound (each
element read once and written once), which is what bench.py's softmax_bytes
charges per fp32 element.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_unfused_and_fused_softmax_counts_match_the_lecture(golden):
    g = golden("cmu15779_l8_softmax_counts.txt")
    M, N = int(g["M"]), int(g["N"])
    reads, writes = bench.unfused_softmax_elements(M, N)
    assert reads == g["unfused_read"] and writes == g["unfused_write"]
    fused = g["fused_read"] + g["fused_write"]
    assert M * N == g["fused_read"] == g["fused_write"]
    assert bench.softmax_bytes(M, N) == 4 * fused  # fp32: 4 bytes per element moved
    assert round((reads + writes) / fused, 2) == g["ratio"]


def test_ragged_softmax_bytes_count_only_valid_prefixes():
    # lengths are clamped to [0, cols]; the padded tail is never moved; the
    # length array is read and the argmax written once per row
    L = np.array([-3, 0, 5, 781, 900], dtype=np.int32)
    valid = 0 + 0 + 5 + 781 + 781
    assert bench.softmax_bytes(5, 781, lengths=L) == 8 * valid + 5 * 4
    assert bench.softmax_bytes(5, 781, lengths=L, argmax=True) == 8 * valid + 5 * 4 + 5 * 4


def test_workload_bytes_per_launch():
    # each input read once and each output written once
    assert bench.sum_relu_add_bytes(64, 128) == 65_792
    assert bench.softmax_bytes(4096, 1024) == 33_554_432
    assert bench.layernorm_bytes(2048, 32768) == 268_566_528  # x, y and gamma, beta once
    assert bench.sumsq_bytes(1 << 28) == 1_073_741_828
