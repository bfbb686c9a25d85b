"""Pins of the oracle's segmentation against closed forms, invariants and the pages' counts.

Sources: pith.science review of "Attamba: Attending To Multi-Token States" — "What carries
the argument" (chunks of P tokens, cyclic offset by layer index), "If this is right"
(variable-length boundaries via cu_seqlens), "Assumptions & free parameters" (offset =
layer index); rohan-paul.com "Key Insights" (cyclic chunking, randomized boundaries).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import decode_state_from_prefix, segment, uniform_chunk_starts
from workloads import PREFILL_CONFIGS, draw_chunk_lengths


GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def closed_form_count(n: int, P: int, o: int) -> int:
    """Chunks of one sequence: ceil(n/P) at o = 0; 1 + ceil((n-o)/P) for 0 < o < n; one
    chunk if n <= o (and none for an empty sequence)."""
    if n == 0:
        return 0
    if o == 0:
        return -(-n // P)
    if n <= o:
        return 1
    return 1 + -(-(n - o) // P)


@pytest.mark.parametrize("P", range(1, 9))
def test_count_closed_form(P):
    for n in range(0, 60):
        for layer in range(0, 2 * P + 1):
            starts = uniform_chunk_starts(n, P, layer)
            assert len(starts) == closed_form_count(n, P, layer % P), (n, P, layer)


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 8])
def test_chunk_lengths_shape(P):
    """First chunk has length o (if o > 0), then P, the last one may be partial."""
    for n in range(1, 50):
        for o in range(P):
            starts = uniform_chunk_starts(n, P, o) + [n]
            lens = np.diff(starts)
            assert lens.sum() == n and (lens >= 1).all()
            inner = lens[1:-1] if o > 0 else lens[:-1]
            if o > 0 and n > o:
                assert lens[0] == o
            assert (inner == P).all(), (n, P, o, lens)
            assert 1 <= lens[-1] <= P


def test_cyclic_offset_by_layer():
    """Layer l and l + P chunk identically; layer l's starts are layer 0's shifted by
    l mod P (plus the sequence start)."""
    n = 97
    for P in (2, 3, 4, 8):
        base = set(uniform_chunk_starts(n, P, 0))
        for layer in range(3 * P):
            s = uniform_chunk_starts(n, P, layer)
            assert s == uniform_chunk_starts(n, P, layer + P)
            shifted = {0} | {t + layer % P for t in base if t + layer % P < n}
            assert set(s) == shifted


def test_segment_packed_batch():
    seq_cu = [0, 5, 5, 17, 18]          # includes an empty and a 1-token sequence
    chunk_cu, tc, ie = segment(seq_cu, P=4, layer_idx=1)
    lens = [5, 0, 12, 1]
    assert len(chunk_cu) - 1 == sum(closed_form_count(n, 4, 1) for n in lens)
    for s in range(4):
        a, b = seq_cu[s], seq_cu[s + 1]
        if a < b:
            assert a in chunk_cu and ie[b - 1] == 1      # sequence start/end are chunk edges
    assert (np.diff(tc) >= 0).all() and ie.sum() == len(chunk_cu) - 1
    for t in range(seq_cu[-1]):
        assert chunk_cu[tc[t]] <= t < chunk_cu[tc[t] + 1]


def test_explicit_lengths_are_cu_seqlens():
    rng = np.random.default_rng(11)
    seq_cu = [0, 40, 41, 100]
    lens = []
    for a, b in zip(seq_cu[:-1], seq_cu[1:]):
        lens += draw_chunk_lengths(rng, b - a, 2, 16)
    chunk_cu, tc, ie = segment(seq_cu, chunk_lens=lens)
    assert list(chunk_cu) == list(np.concatenate([[0], np.cumsum(lens)]))
    with pytest.raises(ValueError):
        segment(seq_cu, chunk_lens=lens[:-1])
    with pytest.raises(ValueError):
        segment([0, 10], chunk_lens=[4, 7])


def test_config_chunk_counts():
    """Counts of the named workloads (closed form above)."""
    c = PREFILL_CONFIGS["train_bf16"]          # n=2048, P=8, layer 3 -> o=3
    chunk_cu, _, _ = segment(np.arange(c.B + 1) * c.n, c.P, c.layer_idx)
    assert len(chunk_cu) - 1 == c.B * (1 + math.ceil((c.n - 3) / 8)) == 1028
    c = PREFILL_CONFIGS["prefill_bf16"]
    chunk_cu, _, _ = segment(np.arange(c.B + 1) * c.n, c.P, c.layer_idx)
    assert len(chunk_cu) - 1 == c.B * c.n // c.P == 2048


def test_pages_footprint_example():
    """n/P + L cached states at n=1024, P=4, L=32 is 288; 36x the 8-token baseline window."""
    g = json.load(open(os.path.join(GOLDEN, "footprint_example.json")))
    n, P, L, E = g["n"], g["P"], g["L"], g["E"]
    y = np.zeros((n, E))
    st = decode_state_from_prefix(y, y, np.zeros(1), np.zeros(1), n, H=1, hd=E, P=P, layer_idx=0, L=L)
    assert len(st.bounds) + len(st.recent) == g["kv_states"]
    assert L // P == g["baseline_window"]
    assert (len(st.bounds) + len(st.recent)) / g["baseline_window"] == g["map_ratio"]


def test_pages_compression_ratios():
    g = json.load(open(os.path.join(GOLDEN, "compression_claims.json")))
    for c in g["cases"]:
        n, P, L = c["n"], c["P"], c["L"]
        y = np.zeros((n, 1))
        st = decode_state_from_prefix(y, y, np.zeros(1), np.zeros(1), n, H=1, hd=1, P=P, layer_idx=0, L=L)
        ratio = n / (len(st.bounds) + len(st.recent))
        assert round(ratio) == c["claimed_ratio"] and ratio < P
