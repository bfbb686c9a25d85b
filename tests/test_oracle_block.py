"""Pins of the oracle's Mamba-block variant of the KV-SSM: a causal depthwise convolution with
SiLU on the scan's input and a SiLU gate on its output (the selective SSM is a Mamba block's
core: pith.science, "Assumptions & free parameters", Section 3.2, Eq. 3), with the convolution
restarting at every chunk start like the state ("Core claim": each chunk X^(p) is compressed on
its own).

The convolution is tied to numpy.convolve run on each chunk alone, SiLU to scipy's logistic
function, and the whole block to the plain scan in the cases where it must reduce to it.
"""
import numpy as np
import pytest
from scipy.special import expit

from oracle import chunk_causal_conv, segment, selective_scan, silu, ssm_block_scan


def _case(seed, T=29, d=5, N=4, K=4):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((T, d)),
        dt=rng.standard_normal((T, d)) * 0.7,
        bias=rng.uniform(-4.0, -1.0, d),
        A=-np.exp(rng.uniform(0.0, np.log(16.0), (d, N))),
        Bm=rng.standard_normal((T, N)),
        Cm=rng.standard_normal((T, N)),
        D=rng.uniform(0.5, 1.5, d),
        w=rng.standard_normal((d, K)) * 0.5,
        b=rng.standard_normal(d) * 0.1,
        z=rng.standard_normal((T, d)) * 2.0,
    )


def _chunks(T, P=6, layer=2):
    return segment([0, T], P=P, layer_idx=layer)[0]


def test_silu_against_logistic_function():
    v = np.linspace(-30.0, 30.0, 121)
    np.testing.assert_allclose(silu(v), v * expit(v), rtol=1e-13, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0
    assert abs(silu(np.array([40.0]))[0] - 40.0) < 1e-15 * 40 + 40 * np.exp(-40.0)


@pytest.mark.parametrize("K", [1, 2, 4])
def test_conv_equals_numpy_convolve_per_chunk(K):
    """Within each chunk, channel c's output is numpy.convolve of that chunk's inputs with the
    reversed taps, cut to the chunk length, plus the bias: tap K-1 multiplies the current token,
    and nothing before the chunk start contributes."""
    p = _case(1, K=K)
    T, d = p["x"].shape
    cu = _chunks(T)
    out = chunk_causal_conv(p["x"], p["w"], p["b"], cu)
    for a, e in zip(cu[:-1], cu[1:]):
        for c in range(d):
            ref = np.convolve(p["x"][a:e, c], p["w"][c, ::-1])[: e - a] + p["b"][c]
            np.testing.assert_allclose(out[a:e, c], ref, rtol=1e-13, atol=1e-14)


def test_conv_with_a_delta_kernel_is_the_identity():
    p = _case(2)
    T, d = p["x"].shape
    w = np.zeros((d, 4))
    w[:, 3] = 1.0
    np.testing.assert_array_equal(chunk_causal_conv(p["x"], w, np.zeros(d), _chunks(T)), p["x"])


def test_conv_restarts_at_chunk_starts():
    """A change to the last token of a chunk leaves the next chunk's convolution (and its block
    output) unchanged, although the next chunk's first tokens lie within K - 1 positions."""
    p = _case(3)
    T, d = p["x"].shape
    cu = _chunks(T)
    q = 2
    end = int(cu[q + 1]) - 1
    x2 = p["x"].copy()
    x2[end] += 5.0
    o1 = ssm_block_scan(p["x"], p["dt"], p["bias"], p["A"], p["Bm"], p["Cm"], p["D"], cu,
                        conv_w=p["w"], conv_b=p["b"], z=p["z"])
    o2 = ssm_block_scan(x2, p["dt"], p["bias"], p["A"], p["Bm"], p["Cm"], p["D"], cu,
                        conv_w=p["w"], conv_b=p["b"], z=p["z"])
    assert np.abs(o1[end] - o2[end]).max() > 1e-3
    np.testing.assert_array_equal(o1[end + 1:], o2[end + 1:])
    np.testing.assert_array_equal(o1[:int(cu[q])], o2[:int(cu[q])])


def test_block_without_conv_or_gate_is_the_plain_scan():
    p = _case(4)
    T = p["x"].shape[0]
    cu = _chunks(T)
    y, _ = selective_scan(p["x"], p["dt"], p["bias"], p["A"], p["Bm"], p["Cm"], p["D"], cu)
    np.testing.assert_array_equal(
        ssm_block_scan(p["x"], p["dt"], p["bias"], p["A"], p["Bm"], p["Cm"], p["D"], cu), y)


def test_block_with_delta_kernel_scans_silu_of_the_input():
    """With the delta kernel and zero bias the convolution is the identity, so the block scans
    silu(x), and its skip term uses silu(x), not x."""
    p = _case(5)
    T, d = p["x"].shape
    cu = _chunks(T)
    w = np.zeros((d, 4))
    w[:, 3] = 1.0
    xs = p["x"] * expit(p["x"])
    y, _ = selective_scan(xs, p["dt"], p["bias"], p["A"], p["Bm"], p["Cm"], p["D"], cu)
    got = ssm_block_scan(p["x"], p["dt"], p["bias"], p["A"], p["Bm"], p["Cm"], p["D"], cu,
                         conv_w=w, conv_b=np.zeros(d))
    np.testing.assert_allclose(got, y, rtol=1e-12, atol=1e-14)


def test_gate_multiplies_by_silu_of_z():
    """The gate scales each output by silu(z): zero where z = 0, about z where z is large, and
    x sigmoid(x) elsewhere (scipy's logistic function)."""
    p = _case(6)
    T, d = p["x"].shape
    cu = _chunks(T)
    y, _ = selective_scan(p["x"], p["dt"], p["bias"], p["A"], p["Bm"], p["Cm"], p["D"], cu)
    z = p["z"].copy()
    z[0] = 0.0
    z[1] = 40.0
    got = ssm_block_scan(p["x"], p["dt"], p["bias"], p["A"], p["Bm"], p["Cm"], p["D"], cu, z=z)
    assert np.all(got[0] == 0.0)
    np.testing.assert_allclose(got[1], 40.0 * y[1], rtol=1e-15)
    np.testing.assert_allclose(got, y * z * expit(z), rtol=1e-13, atol=1e-15)


def test_block_output_is_local_to_its_chunk():
    """Block outputs of one chunk depend only on that chunk's inputs (conv, scan and gate all
    restart): scanning a chunk alone gives the same values."""
    p = _case(7)
    T, d = p["x"].shape
    cu = _chunks(T)
    full = ssm_block_scan(p["x"], p["dt"], p["bias"], p["A"], p["Bm"], p["Cm"], p["D"], cu,
                          conv_w=p["w"], conv_b=p["b"], z=p["z"])
    for a, e in zip(cu[:-1], cu[1:]):
        sl = slice(int(a), int(e))
        alone = ssm_block_scan(p["x"][sl], p["dt"][sl], p["bias"], p["A"], p["Bm"][sl],
                               p["Cm"][sl], p["D"], [0, int(e - a)], conv_w=p["w"], conv_b=p["b"],
                               z=p["z"][sl])
        np.testing.assert_allclose(full[sl], alone, rtol=1e-13, atol=1e-15)
