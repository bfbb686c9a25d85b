"""Pins of the oracle's selective scan (the KV-SSM that replaces W_K and W_V).

The recurrence is the Mamba selective scan the paper cites as its Eq. 3 (pith.science,
"Assumptions & free parameters"); the pages do not print it. These tests tie the oracle to
facts independent of its own loop: closed forms (one-token chunks, constant inputs), a
library routine for the time-invariant special case (scipy.signal.lfilter), the unrolled
sum of the recurrence with cumulative step sizes, and structural invariants (reset at chunk
starts, causality inside a chunk, linearity in x, decay since A < 0).
"""
import numpy as np
import pytest
from scipy.signal import lfilter

from oracle import boundary_states, segment, selective_scan, softplus


def _rand(seed, T=23, d=5, N=4):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((T, d)),
        dt=rng.standard_normal((T, d)) * 0.7,
        bias=rng.uniform(-4.0, -1.0, d),
        A=-np.exp(rng.uniform(0.0, np.log(16.0), (d, N))),
        Bm=rng.standard_normal((T, N)),
        Cm=rng.standard_normal((T, N)),
        D=rng.uniform(0.5, 1.5, d),
    )


def _scan(p, chunk_cu, **kw):
    return selective_scan(p["x"], p["dt"], p["bias"], p["A"], p["Bm"], p["Cm"], p["D"],
                          chunk_cu, **kw)


def test_softplus_values():
    z = np.array([-30.0, -5.0, 0.0, 1.0, 30.0])
    ref = np.array([np.exp(-30.0), 0.006715348489118068, np.log(2.0), 1.3132616875182228,
                    30.0])
    np.testing.assert_allclose(softplus(z), ref, rtol=1e-13)


def test_one_token_chunks_closed_form():
    """P = 1: every token starts a chunk, so y_t = x_t * (delta_t * (Cm_t . Bm_t) + D)."""
    p = _rand(0)
    T = p["x"].shape[0]
    chunk_cu, _, _ = segment([0, T], P=1)
    y, _ = _scan(p, chunk_cu)
    delta = softplus(p["dt"] + p["bias"])
    cb = (p["Cm"] * p["Bm"]).sum(axis=1)
    ref = p["x"] * (delta * cb[:, None] + p["D"])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_constant_inputs_geometric_series():
    """Constant delta, x, Bm, Cm inside a chunk: h after the (tau+1)-th token is
    delta*x*Bm*(1 - a^(tau+1))/(1 - a) with a = exp(delta*A)."""
    d, N, P = 3, 4, 7
    rng = np.random.default_rng(1)
    A = -np.exp(rng.uniform(0.0, np.log(16.0), (d, N)))
    x0, dt0 = rng.standard_normal(d), rng.standard_normal(d)
    bias = np.full(d, -2.0)
    Bm0, Cm0 = rng.standard_normal(N), rng.standard_normal(N)
    T = 2 * P
    p = dict(x=np.tile(x0, (T, 1)), dt=np.tile(dt0, (T, 1)), bias=bias, A=A,
             Bm=np.tile(Bm0, (T, 1)), Cm=np.tile(Cm0, (T, 1)), D=np.ones(d))
    chunk_cu, _, _ = segment([0, T], P=P)
    y, _ = _scan(p, chunk_cu)
    delta = softplus(dt0 + bias)
    a = np.exp(delta[:, None] * A)
    for t in range(T):
        tau = t % P
        h = (delta * x0)[:, None] * Bm0[None, :] * (1 - a ** (tau + 1)) / (1 - a)
        np.testing.assert_allclose(y[t], h @ Cm0 + x0, rtol=1e-12)


def test_vanishing_step_gives_skip_only():
    p = _rand(2)
    p["bias"] = np.full_like(p["bias"], -60.0)     # delta ~ e^-60
    chunk_cu, _, _ = segment([0, p["x"].shape[0]], P=4)
    y, _ = _scan(p, chunk_cu)
    np.testing.assert_allclose(y, p["D"] * p["x"], rtol=0, atol=1e-20)


def test_time_invariant_case_matches_lfilter():
    """Constant step size per channel makes each (channel, state) a first-order IIR filter
    h_t = a h_{t-1} + u_t; scipy's lfilter computes it independently of the oracle loop."""
    p = _rand(3, T=31)
    T, d = p["x"].shape
    N = p["A"].shape[1]
    p["dt"] = np.tile(p["dt"][0], (T, 1))
    P = 9
    chunk_cu, _, _ = segment([0, T], P=P)
    y, _ = _scan(p, chunk_cu)
    delta = softplus(p["dt"][0] + p["bias"])
    ref = np.zeros((T, d))
    for a0, a1 in zip(chunk_cu[:-1], chunk_cu[1:]):
        for c in range(d):
            for n in range(N):
                u = delta[c] * p["x"][a0:a1, c] * p["Bm"][a0:a1, n]
                h = lfilter([1.0], [1.0, -np.exp(delta[c] * p["A"][c, n])], u)
                ref[a0:a1, c] += h * p["Cm"][a0:a1, n]
    ref += p["D"] * p["x"]
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_unrolled_sum_time_varying():
    """y_t = sum_{s in chunk, s<=t} sum_n Cm_t[n] exp(A[c,n] * sum_{r=s+1..t} delta_r)
    Bm_s[n] delta_s x_s + D x_t, evaluated with cumulative sums (no recurrence)."""
    p = _rand(4, T=17, d=4, N=3)
    T, d = p["x"].shape
    chunk_cu, _, _ = segment([0, 6, T], P=5, layer_idx=2)
    y, _ = _scan(p, chunk_cu)
    delta = softplus(p["dt"] + p["bias"])
    ref = p["D"] * p["x"]
    for q in range(len(chunk_cu) - 1):
        a0, a1 = chunk_cu[q], chunk_cu[q + 1]
        cum = np.cumsum(delta[a0:a1], axis=0)        # cum[k] = sum of delta over a0..a0+k
        for t in range(a0, a1):
            for s in range(a0, t + 1):
                acc = cum[t - a0] - cum[s - a0]            # sum_{r=s+1..t} delta_r, [d]
                decay = np.exp(p["A"] * acc[:, None])       # [d, N]
                ref[t] += (decay * p["Bm"][s][None, :] * p["Cm"][t][None, :]).sum(1) \
                    * delta[s] * p["x"][s]
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-13)


def test_reset_equals_independent_segments_and_causality():
    p = _rand(5, T=30)
    T = p["x"].shape[0]
    chunk_cu, _, _ = segment([0, 13, T], P=6, layer_idx=1)
    y, _ = _scan(p, chunk_cu)
    for a0, a1 in zip(chunk_cu[:-1], chunk_cu[1:]):
        sub = {k: (v[a0:a1] if k in ("x", "dt", "Bm", "Cm") else v) for k, v in p.items()}
        ys, _ = _scan(sub, np.array([0, a1 - a0]))
        np.testing.assert_allclose(y[a0:a1], ys, rtol=1e-13, atol=1e-15)
    # a perturbation of token s moves y only at t >= s inside s's chunk
    s = 15
    q = int(np.searchsorted(chunk_cu, s, side="right") - 1)
    p2 = {k: v.copy() for k, v in p.items()}
    p2["x"][s] += 1.0
    p2["Bm"][s] -= 0.5
    y2, _ = _scan(p2, chunk_cu)
    changed = np.abs(y2 - y).max(axis=1) > 0
    expect = np.zeros(T, bool)
    expect[s:chunk_cu[q + 1]] = True
    assert (changed == expect).all()


def test_linear_in_x_and_decay():
    p = _rand(6)
    T = p["x"].shape[0]
    chunk_cu, _, _ = segment([0, T], P=T)
    y1, _ = _scan(p, chunk_cu)
    p2 = dict(p, x=2.5 * p["x"])
    y2, _ = _scan(p2, chunk_cu)
    np.testing.assert_allclose(y2, 2.5 * y1, rtol=1e-12, atol=1e-14)
    # impulse at t=0 only: every state decays in magnitude (A < 0)
    p3 = dict(p, x=np.zeros_like(p["x"]))
    p3["x"][0] = 1.0
    _, snaps = _scan(p3, chunk_cu, snapshot_after=set(range(T)))
    mags = np.array([np.abs(snaps[t]) for t in range(T)])
    assert (mags[0] > 0).all() and (np.diff(mags, axis=0) < 0).all()


def test_boundary_state_is_full_chunk_compression():
    """The boundary state of a chunk is the output after its whole chunk: with constant
    inputs that is the geometric closed form at the chunk's own length (chunks of lengths
    2, 4, 4, 3 here: offset 2, P = 4, n = 13)."""
    d, N = 3, 2
    rng = np.random.default_rng(8)
    A = -np.exp(rng.uniform(0.0, np.log(16.0), (d, N)))
    x0, Bm0, Cm0 = rng.standard_normal(d), rng.standard_normal(N), rng.standard_normal(N)
    T = 13
    p = dict(x=np.tile(x0, (T, 1)), dt=np.zeros((T, d)), bias=np.full(d, -1.5), A=A,
             Bm=np.tile(Bm0, (T, 1)), Cm=np.tile(Cm0, (T, 1)), D=np.zeros(d))
    chunk_cu, _, is_end = segment([0, T], P=4, layer_idx=2)
    y, _ = _scan(p, chunk_cu)
    kb = boundary_states(y, chunk_cu)
    delta = softplus(np.full(d, -1.5))
    a = np.exp(delta[:, None] * A)
    for q, length in enumerate([2, 4, 4, 3]):
        h = (delta * x0)[:, None] * Bm0[None, :] * (1 - a ** length) / (1 - a)
        np.testing.assert_allclose(kb[q], h @ Cm0, rtol=1e-12)
    np.testing.assert_array_equal(kb, y[is_end.astype(bool)])
