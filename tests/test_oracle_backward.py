"""Pins of the oracle's backward pass: every gradient against central finite differences of
the oracle's own forward (float64), on tiny cases with several chunks, both mask modes and a
window; plus the special case of a single visible key."""
import numpy as np
import pytest

import oracle

EPS = 1e-6


def fd(f, x, idx):
    xp, xm = x.copy(), x.copy()
    xp[idx] += EPS
    xm[idx] -= EPS
    return (f(xp) - f(xm)) / (2 * EPS)


def scan_case(seed=0):
    rng = np.random.default_rng(seed)
    T, d, N = 11, 3, 2
    chunk_cu = np.array([0, 3, 4, 9, 11])
    args = dict(x=rng.standard_normal((T, d)), dt=rng.standard_normal((T, d)),
                dt_bias=rng.standard_normal(d) * 0.5, A=-np.exp(rng.uniform(0, 1, (d, N))),
                Bm=rng.standard_normal((T, N)), Cm=rng.standard_normal((T, N)),
                D=rng.standard_normal(d))
    gy = rng.standard_normal((T, d))
    return args, chunk_cu, gy


@pytest.mark.parametrize("name,grad", [("x", "dx"), ("dt", "ddt"), ("dt_bias", "dbias"),
                                       ("A", "dA"), ("Bm", "dBm"), ("Cm", "dCm"), ("D", "dD")])
def test_scan_backward_matches_finite_differences(name, grad):
    args, chunk_cu, gy = scan_case()
    g = oracle.selective_scan_backward(chunk_cu=chunk_cu, gy=gy, **args)

    def loss(val):
        a = dict(args)
        a[name] = val
        y, _ = oracle.selective_scan(chunk_cu=chunk_cu, **a)
        return float((gy * y).sum())

    base = args[name]
    for idx in np.ndindex(base.shape):
        num = fd(loss, base, idx)
        assert abs(g[grad][idx] - num) < 1e-6 * (1 + abs(num)), (name, idx, g[grad][idx], num)


def test_scan_backward_stops_at_chunk_starts():
    """A gradient on the output of one chunk leaves every other chunk's inputs untouched."""
    args, chunk_cu, _ = scan_case(1)
    gy = np.zeros((11, 3))
    gy[6] = 1.0                                   # inside chunk [4, 9)
    g = oracle.selective_scan_backward(chunk_cu=chunk_cu, gy=gy, **args)
    assert not g["dx"][:4].any() and not g["dx"][7:].any()
    assert g["dx"][4:7].any()


@pytest.mark.parametrize("mode,L,P,layer", [("train", 0, 3, 0), ("test", 2, 3, 1),
                                            ("train", 3, 4, 2), ("test", 0, 2, 0)])
def test_attention_backward_matches_finite_differences(mode, L, P, layer):
    rng = np.random.default_rng(7)
    seq_cu = np.array([0, 9, 13])
    T, H, hd = 13, 2, 3
    q, k, v = (rng.standard_normal((T, H, hd)) for _ in range(3))
    dout = rng.standard_normal((T, H, hd))
    _, tc, ie = oracle.segment(seq_cu, P, layer)
    dq, dk, dv = oracle.chunk_attention_backward(q, k, v, seq_cu, tc, ie, L, mode, dout)

    def loss(which, val):
        a = {"q": q, "k": k, "v": v}
        a[which] = val
        o, _ = oracle.chunk_attention(a["q"], a["k"], a["v"], seq_cu, tc, ie, L, mode)
        return float((dout * o).sum())

    for which, g in (("q", dq), ("k", dk), ("v", dv)):
        base = {"q": q, "k": k, "v": v}[which]
        for idx in np.ndindex(base.shape):
            num = fd(lambda val: loss(which, val), base, idx)
            assert abs(g[idx] - num) < 1e-6 * (1 + abs(num)), (which, idx, g[idx], num)


def test_attention_backward_single_key():
    """A row that sees one key passes its output gradient to that key's value unchanged and
    nothing to the query or the key (the softmax weight is constant 1)."""
    q = np.random.default_rng(3).standard_normal((1, 1, 4))
    k = np.random.default_rng(4).standard_normal((1, 1, 4))
    v = np.random.default_rng(5).standard_normal((1, 1, 4))
    dout = np.array([[[1.0, -2.0, 0.5, 3.0]]])
    dq, dk, dv = oracle.masked_attention_backward(q, k, v, np.ones((1, 1), bool), 0.5, dout)
    np.testing.assert_allclose(dv, dout)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
