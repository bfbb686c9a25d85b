"""Pins of the oracle's decode step (boundary-state cache plus L leading tokens).

Sources: pith.science review of "Attamba: Attending To Multi-Token States" — "Core claim"
(at inference only the boundary states are cached) and "If this is right" (cache shrinks by
about P; leading tokens kept). The invariant: generating token i with the cache must give
exactly row i of the prefill attention (M_test plus window) over the whole sequence.
"""
import numpy as np
import pytest

from oracle import (TEST, decode_state_from_prefix, decode_step, is_chunk_end_at,
                    kvssm_forward, segment, selective_scan)


def _inputs(seed, T, d, N):
    rng = np.random.default_rng(seed)
    inp = dict(x=rng.standard_normal((T, d)), q=rng.standard_normal((T, d)))
    for s in ("k", "v"):
        inp[f"dt_{s}"] = rng.standard_normal((T, d)) * 0.5
        inp[f"bm_{s}"] = rng.standard_normal((T, N))
        inp[f"cm_{s}"] = rng.standard_normal((T, N))
        inp[f"A_{s}"] = -np.exp(rng.uniform(0, np.log(16), (d, N)))
        inp[f"bias_{s}"] = rng.uniform(-4, -1, d)
        inp[f"D_{s}"] = np.ones(d)
    return inp


@pytest.mark.parametrize("P,layer,L,n0", [(4, 0, 3, 9), (4, 2, 5, 10), (3, 1, 1, 7),
                                          (4, 0, 0, 12), (2, 1, 8, 5), (5, 3, 2, 13)])
def test_decode_matches_prefill_rows(P, layer, L, n0):
    H, hd, N = 2, 3, 4
    d = H * hd
    o = layer % P
    n_total = n0 + 14
    n_total += (o - n_total) % P           # the last chunk is complete at n_total
    inp = _inputs(P * 100 + n0, n_total, d, N)
    ref = kvssm_forward(inp, [0, n_total], H, hd, P, layer, L, TEST)
    chunk_cu, _, _ = segment([0, n_total], P, layer)
    _, sk = selective_scan(inp["x"], inp["dt_k"], inp["bias_k"], inp["A_k"], inp["bm_k"],
                           inp["cm_k"], inp["D_k"], chunk_cu, snapshot_after={n0 - 1})
    _, sv = selective_scan(inp["x"], inp["dt_v"], inp["bias_v"], inp["A_v"], inp["bm_v"],
                           inp["cm_v"], inp["D_v"], chunk_cu, snapshot_after={n0 - 1})
    st = decode_state_from_prefix(ref["y_k"], ref["y_v"], sk[n0 - 1], sv[n0 - 1], n0, H, hd,
                                  P, layer, L)
    par = {k: inp[k] for k in ("A_k", "A_v", "D_k", "D_v", "bias_k", "bias_v")}
    for i in range(n0, n_total):
        tok = {k: inp[k][i] for k in ("q", "x", "dt_k", "dt_v", "bm_k", "cm_k", "bm_v",
                                      "cm_v")}
        out = decode_step(st, par, tok, H, hd, P, layer, L)
        np.testing.assert_allclose(out, ref["out"][i], rtol=1e-11, atol=1e-12)
        # boundary cache holds exactly the chunk ends at or before i
        assert [b[0] for b in st.bounds] == [j for j in range(i + 1)
                                              if is_chunk_end_at(j, P, layer)]
        assert len(st.recent) == min(L, i + 1)


def test_decode_state_resets_at_chunk_start():
    """Right after a chunk start the state holds only that token's input term."""
    H, hd, N, P = 1, 2, 3, 4
    d = H * hd
    inp = _inputs(7, 8, d, N)
    st = decode_state_from_prefix(np.zeros((4, d)), np.zeros((4, d)), np.full((d, N), 5.0),
                                  np.full((d, N), 5.0), 4, H, hd, P, 0, 2)
    par = {k: inp[k] for k in ("A_k", "A_v", "D_k", "D_v", "bias_k", "bias_v")}
    tok = {k: inp[k][4] for k in ("q", "x", "dt_k", "dt_v", "bm_k", "cm_k", "bm_v", "cm_v")}
    decode_step(st, par, tok, H, hd, P, 0, 2)
    delta = np.logaddexp(0, tok["dt_k"] + par["bias_k"])
    np.testing.assert_allclose(st.h_k, (delta * tok["x"])[:, None] * tok["bm_k"][None, :],
                               rtol=1e-14)
