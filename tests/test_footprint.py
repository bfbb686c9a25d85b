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
