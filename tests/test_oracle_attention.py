"""Pins of the oracle's chunk mask and masked attention.

Sources: pith.science review of "Attamba: Attending To Multi-Token States" — "What carries
the argument" (M_train, Eq. 5: last token of each completed chunk plus the current partial
chunk; M_test, Eq. 7; sliding window of L leading tokens, Eq. 8; attention map about
n/P + L per query) and the Referee Report's second major comment (causal reading of M_test).
Independent pins: torch's scaled_dot_product_attention for the cases that reduce to plain
causal attention, closed-form nonzero counts, and softmax identities.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import TEST, TRAIN, chunk_attention, dense_mask, masked_attention, segment


def _qkv(seed, T, H=2, hd=8):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, H, hd)) for _ in range(3)]


def _sdpa_causal(q, k, v):
    t = [torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2))) for a in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True)
    return o.numpy().transpose(1, 0, 2)


def ends_before(w: int, P: int, o: int, n: int) -> int:
    """Number of chunk ends at positions < w for uniform chunking with offset o: positions t
    with (t + 1 - o) = 0 mod P while w <= n - 1; at w = n every chunk has ended (the last
    token always ends one), which is ceil(n/P) at o = 0 and 1 + ceil((n-o)/P) otherwise."""
    if w < n:
        return (w + P - 1 - ((o - 1) % P)) // P
    return -(-n // P) if o == 0 else (1 if n <= o else 1 + -(-(n - o) // P))


@pytest.mark.parametrize("mode", [TRAIN, TEST])
def test_reduces_to_causal_attention(mode):
    """P = 1 with L = 0, L >= n, and (M_train) a single chunk all give plain causal
    attention, which torch computes independently."""
    T = 37
    q, k, v = _qkv(0, T)
    ref = _sdpa_causal(q, k, v)
    cases = [dict(P=1, L=0), dict(P=5, L=T), dict(P=3, L=10 ** 6)]
    if mode == TRAIN:
        cases.append(dict(P=T, L=0))
    for c in cases:
        chunk_cu, tc, ie = segment([0, T], P=c["P"])
        out, _ = chunk_attention(q, k, v, [0, T], tc, ie, c["L"], mode)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_train_nnz_closed_form():
    """M_train, L = 0, o = 0, P | n: n (n/P + P) / 2 visible pairs."""
    for n, P in [(256, 4), (64, 8), (60, 6), (12, 1), (16, 16)]:
        _, tc, ie = segment([0, n], P=P)
        assert dense_mask(tc, ie, 0, TRAIN).sum() == n * (n // P + P) // 2


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("L", [0, 1, 3, 5, 64])
@pytest.mark.parametrize("mode", [TRAIN, TEST])
def test_row_counts_closed_form(P, L, mode):
    """Row i sees a contiguous band [w_i, i] plus the chunk ends before w_i:
    count(i) = (i - w_i + 1) + ends_before(w_i), w_i = max(0, i - L + 1) for M_test
    (w_i = i + 1 when L = 0) and min(chunk start of i, i - L + 1) for M_train."""
    n = 39
    for o in range(P):
        chunk_cu, tc, ie = segment([0, n], P=P, layer_idx=o)
        m = dense_mask(tc, ie, L, mode)
        for i in range(n):
            w = max(0, i - L + 1)
            if mode == TRAIN:
                w = min(w, int(chunk_cu[tc[i]]))
            expect = (i - w + 1) + ends_before(w, P, o, n)
            assert m[i].sum() == expect, (P, L, mode, o, i)


def test_sequences_do_not_mix():
    T = 30
    q, k, v = _qkv(1, T)
    seq_cu = [0, 11, 11, 30]
    chunk_cu, tc, ie = segment(seq_cu, P=4, layer_idx=2)
    out, lse = chunk_attention(q, k, v, seq_cu, tc, ie, 3, TEST)
    for a, b in [(0, 11), (11, 30)]:
        _, tcl, iel = segment([0, b - a], P=4, layer_idx=2)
        o2, l2 = chunk_attention(q[a:b], k[a:b], v[a:b], [0, b - a], tcl, iel, 3, TEST)
        np.testing.assert_allclose(out[a:b], o2, rtol=1e-13)
        np.testing.assert_allclose(lse[:, a:b], l2, rtol=1e-13)


def test_single_visible_key_and_equal_scores():
    T = 20
    q, k, v = _qkv(2, T)
    chunk_cu, tc, ie = segment([0, T], P=4)
    # M_test with L = 1 at the first token: it sees only itself
    out, _ = chunk_attention(q, k, v, [0, T], tc, ie, 1, TEST, rows=[0, 1, 2])
    np.testing.assert_array_equal(out[0], v[0])
    # zero queries: every visible score is 0, so O is the mean of the visible V rows
    out, _ = chunk_attention(np.zeros_like(q), k, v, [0, T], tc, ie, 2, TRAIN)
    m = dense_mask(tc, ie, 2, TRAIN)
    for i in range(T):
        np.testing.assert_allclose(out[i], v[m[i]].mean(axis=0), rtol=1e-13)


def test_lse_and_empty_rows():
    T = 18
    q, k, v = _qkv(3, T)
    chunk_cu, tc, ie = segment([0, T], P=4, layer_idx=0)
    out, lse = chunk_attention(q, k, v, [0, T], tc, ie, 0, TEST)
    m = dense_mask(tc, ie, 0, TEST)
    scale = 1 / np.sqrt(q.shape[2])
    for i in range(T):
        for h in range(q.shape[1]):
            s = (k[:, h] @ q[i, h]) * scale
            if m[i].any():
                assert abs(lse[h, i] - logsumexp(s[m[i]])) < 1e-12
            else:                   # before the first chunk end, M_test with L=0 sees nothing
                assert lse[h, i] == -np.inf and (out[i, h] == 0).all()
    assert not m[:3].any() and m[3:].any(axis=1).all()


def test_subset_rows_match_full():
    T = 29
    q, k, v = _qkv(4, T)
    seq_cu = [0, 9, 29]
    chunk_cu, tc, ie = segment(seq_cu, P=3, layer_idx=1)
    full_o, full_l = chunk_attention(q, k, v, seq_cu, tc, ie, 4, TRAIN)
    rows = [28, 0, 9, 13]
    o, l_ = chunk_attention(q, k, v, seq_cu, tc, ie, 4, TRAIN, rows=rows)
    np.testing.assert_allclose(o, full_o[rows], rtol=1e-14)
    np.testing.assert_allclose(l_, full_l[:, rows], rtol=1e-14)


def test_rows_are_convex_combinations():
    """Each output row lies in the convex hull of the visible V rows: weights recovered by
    least squares on an orthonormal V are non-negative and sum to one."""
    T, hd = 12, 16
    rng = np.random.default_rng(5)
    q = rng.standard_normal((T, 1, hd))
    k = rng.standard_normal((T, 1, hd))
    v = np.linalg.qr(rng.standard_normal((hd, hd)))[0][:T].reshape(T, 1, hd)
    _, tc, ie = segment([0, T], P=3)
    out, _ = chunk_attention(q, k, v, [0, T], tc, ie, 2, TEST)
    m = dense_mask(tc, ie, 2, TEST)
    for i in range(T):
        wts = v[:, 0, :] @ out[i, 0]
        assert abs(wts.sum() - 1) < 1e-12 and (wts[m[i]] > 0).all()
        assert np.abs(wts[~m[i]]).max(initial=0) < 1e-12
