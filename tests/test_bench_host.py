"""Host-side arithmetic of bench.py (no GPU): the work counts its roofline and throughput figures
divide by, checked against the oracle's dense definitions and the byte count of the scan's
inputs and outputs."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from workloads import PREFILL_BF16, TINY_FP32, TRAIN_BF16

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("lens,P,layer,L,mode", [
    ([40], 4, 0, 0, "train"),
    ([37, 1, 20], 3, 2, 5, "test"),
    ([50, 0, 33], 5, 1, 7, "train"),
    ([64, 64], 8, 3, 64, "test"),
    ([29], 1, 0, 0, "test"),
    ([45, 12], 128, 0, 3, "train"),
])
def test_attention_pairs_equals_dense_mask(lens, P, layer, L, mode):
    """The visible-pair count behind the attention FLOP figure equals the number of true entries
    of the oracle's explicit mask (pith.science, Eq. 5 / Eq. 7 with the window of Eq. 8)."""
    seq_cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    chunk_cu, token_chunk, is_end = oracle.segment(seq_cu, P, layer)
    got = bench.attention_pairs(seq_cu, chunk_cu, token_chunk, L, mode == "train")
    want = 0
    for s in range(len(lens)):
        a, b = int(seq_cu[s]), int(seq_cu[s + 1])
        if b > a:
            m = oracle.dense_mask(token_chunk[a:b], is_end[a:b], L, mode)
            want += int(m.sum())
    assert got == want


def test_attention_pairs_closed_form():
    """M_train, L = 0, offset 0, P dividing n: n (n / P + P) / 2 pairs per sequence."""
    n, P = 96, 8
    seq_cu = np.array([0, n, 2 * n], np.int32)
    chunk_cu, token_chunk, _ = oracle.segment(seq_cu, P, 0)
    assert bench.attention_pairs(seq_cu, chunk_cu, token_chunk, 0, True) == 2 * n * (n // P + P) // 2


def test_scan_algorithmic_bytes():
    """x once, dt_K, dt_V, Bm/Cm of both SSMs, y_K, y_V: 2 (5 d + 4 N) bytes per token at bf16."""
    assert bench.scan_algorithmic_bytes(PREFILL_BF16) == 16384 * 2 * (5 * 2048 + 4 * 16) == 337_641_472
    assert bench.scan_algorithmic_bytes(TRAIN_BF16) == 8192 * 2 * (5 * 1024 + 4 * 16)
    assert bench.scan_algorithmic_bytes(TINY_FP32) == 256 * 4 * (5 * 64 + 4 * 16)


@pytest.mark.parametrize("P,o", [(4, 0), (4, 3), (8, 5), (1, 0), (3, 1)])
def test_decode_ends_before(P, o):
    """Chunk ends at positions below x under the positional rule (j + 1 - o) mod P == 0, which
    the decode bench uses to count the keys a step reads."""
    for x in range(0, 40):
        brute = sum(1 for j in range(x) if (j + 1 - o) % P == 0 and j + 1 - o >= 0)
        assert bench.att_ends_before(x, P, o) == brute, (x, P, o)


def test_multi_gpu_request_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_probe_per_simd_groups_waves_by_simd():
    """The issue-rate probe's host arithmetic: waves are grouped by (XCC, HW_ID bits 4..15), only
    SIMDs holding exactly W overlapping waves count, and a SIMD's clocks per instruction is its
    busy span over the instructions its waves issued."""
    W, ops = 2, 1000
    rows = []
    # SIMD A (xcc 0, simd 1): two overlapping waves spanning 100..4500 -> 4400 / 2000 = 2.2
    rows += [[100, 4300, 0, 10, (1 << 4) | 3, 0], [200, 4500, 1, 11, (1 << 4) | 5, 0]]
    # SIMD B (xcc 1, same HW_ID fields): overlapping, span 0..8000 -> 4.0
    rows += [[0, 8000, 0, 10, 1 << 4, 1], [10, 7990, 0, 10, 1 << 4, 1]]
    # SIMD C: two waves one after the other (not side by side) -> ignored
    rows += [[0, 100, 0, 1, 2 << 4, 0], [200, 300, 2, 3, 2 << 4, 0]]
    # SIMD D: a single wave -> ignored
    rows += [[0, 100, 0, 1, 3 << 4, 0]]
    r = bench.probe_per_simd(np.array(rows), ops, W)
    assert r["simds_used"] == 2
    assert r["clocks_per_instr_per_simd"] == pytest.approx((2.2 + 4.0) / 2)
    assert r["waves_per_simd_histogram"] == {"1": 1, "2": 3}
