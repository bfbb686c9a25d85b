"""Footprint accounting of the decode cache against the pages' worked example and the
allocation a DecodeCache actually makes (host side; the cache is allocated on the CPU, no
kernel runs)."""
import json
import os

import torch

import ssm_compressed_chunked_amd as att
from ssm_compressed_chunked_amd.pipeline import chunk_ends_before, decode_cache_bytes, kv_footprint
from workloads import TINY_FP32, make_prefill

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_pages_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "footprint_example.json")))
    f = kv_footprint(g["n"], g["P"], g["L"], H=8, hd=g["E"] // 8, N=16)
    assert f["attamba_states"] == g["kv_states"]
    assert f["swa_window"] == g["baseline_window"]
    assert f["attamba_states"] // f["swa_window"] == g["map_ratio"]


def test_compression_tends_to_P():
    g = json.load(open(os.path.join(GOLDEN, "compression_claims.json")))
    for c in g["cases"]:
        f = kv_footprint(c["n"], c["P"], c["L"], H=8, hd=64, N=16)
        assert abs(f["compression"] - c["claimed_ratio"]) / c["claimed_ratio"] < 0.02


def test_per_layer_offsets_change_the_count():
    """Cyclic chunking: layers with different offsets hold different boundary counts after the
    same number of tokens; the count never differs by more than one."""
    n, P = 1003, 8
    counts = [chunk_ends_before(n, P, layer) for layer in range(P)]
    assert max(counts) - min(counts) <= 1 and len(set(counts)) == 2
    for layer in range(2 * P):
        brute = sum(1 for j in range(n) if (j + 1 - layer % P) % P == 0)
        assert chunk_ends_before(n, P, layer) == brute


def test_decode_cache_allocation_matches_accounting():
    B, H, hd, N, P, L = 2, 4, 32, 16, 4, 8
    par = make_prefill(TINY_FP32.with_(d=H * hd, H=H, hd=hd)).param
    n = 100
    cap = chunk_ends_before(n, P, 0)
    cache = att.DecodeCache(B, H, hd, N, P, L, 0, cap, torch.bfloat16, par, device="cpu")
    f = kv_footprint(n, P, L, H, hd, N)
    state = B * f["attamba_bytes"]
    ws = cache.workspace.numel() * 4
    assert decode_cache_bytes(cache) == state + ws


# ---------------------------------------------------------------- attention FLOP accounting
import numpy as np
import pytest

import oracle
from ssm_compressed_chunked_amd.pipeline import attention_flops, visible_pairs


@pytest.mark.parametrize("n,P,L,layer,train", [
    (37, 4, 0, 0, True), (37, 4, 0, 0, False), (50, 3, 5, 2, True), (50, 3, 5, 2, False),
    (64, 8, 64, 3, False), (29, 1, 0, 0, False), (45, 128, 3, 7, True), (41, 5, 1, 9, False)])
def test_visible_pairs_equal_the_dense_mask(n, P, L, layer, train):
    """The pair count behind the FLOP figures equals the number of true entries of the oracle's
    explicit mask (Eq. 5 / Eq. 7 with the window of Eq. 8)."""
    _, tc, ie = oracle.segment([0, n], P, layer)
    m = oracle.dense_mask(tc, ie, L, oracle.TRAIN if train else oracle.TEST)
    assert visible_pairs(n, P, L, layer, train) == int(m.sum())


def test_flops_closed_forms():
    """M_train, L = 0, offset 0, P | n: n (n/P + P) / 2 pairs. With P = 1 and L = 0, or P >= n under
    M_train, the mask is causal and the FLOPs equal the dense transformer's."""
    n, P, H, hd = 256, 8, 4, 32
    f = attention_flops(n, P, 0, H, hd, train=True)
    assert f["pairs"] == n * (n // P + P) // 2
    assert attention_flops(n, 1, 0, H, hd)["attamba"] == attention_flops(n, 1, 0, H, hd)["dense"]
    assert attention_flops(60, 64, 0, H, hd, train=True)["attamba"] == \
        attention_flops(60, 64, 0, H, hd, train=True)["dense"]


def test_flops_against_the_pages_worked_example():
    """The review's example (n = 1024, P = 4, 32 leading tokens, E = 512): Attamba caches
    n/P + L = 288 states, the matched baseline keeps L/P = 8 keys, a 36x smaller map, and the
    baseline's per-query FLOPs are smaller still (its width is E/P)."""
    g = json.load(open(os.path.join(GOLDEN, "footprint_example.json")))
    f = attention_flops(g["n"], g["P"], g["L"], H=8, hd=g["E"] // 8)
    lq = f["last_query"]
    assert lq["attamba_states_cached"] == g["kv_states"]
    assert lq["baseline_keys"] == g["baseline_window"]
    assert lq["attamba_states_cached"] // lq["baseline_keys"] == g["map_ratio"]
    # distinct keys actually attended: the window's positions are not counted twice (8 of the 288
    # cached states are boundaries inside the window)
    assert lq["attamba_keys_attended"] == g["kv_states"] - g["L"] // g["P"]
    assert lq["attamba_flops"] / lq["baseline_flops"] > g["map_ratio"]
    # over the whole sequence Attamba's attention costs less than the dense transformer's
    assert f["attamba"] < f["dense"] and f["footprint_matched"] < f["attamba"]
