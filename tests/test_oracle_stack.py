"""Pins of the oracle's layer stack: bf16 storage rounding against torch's conversion, the
cyclic offset of every layer (pith.science "What carries the argument": the chunk offset shifts
by layer index), and the chain itself (layer l + 1 is one layer run on layer l's rounded
output, with the next layer index)."""
import numpy as np
import torch

import oracle
from workloads import make_stack


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    a = a.astype(np.float64)        # float32 values: torch's conversion rounds them exactly once
    ref = torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(a), ref)
    # ties go to the even neighbour; zero stays zero
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 0.0])
    np.testing.assert_array_equal(oracle.round_to_bf16(ties), [1.0, 1 + 2.0 ** -6, -1.0, 0.0])


def _stack_case(n_layers=2):
    d, N, H, hd, P, L = 32, 16, 2, 16, 3, 4
    rng = np.random.default_rng(3)
    x = oracle.round_to_bf16(rng.standard_normal((40, d)))
    layers = [{"w": lay["w"].double().numpy(),
               "params": {k: v.double().numpy() for k, v in lay["params"].items()}}
              for lay in make_stack(d, N, n_layers, seed=7)]
    return x, layers, np.array([0, 23, 40]), (H, hd, N, P, L)


def test_each_layer_chunks_at_its_own_offset():
    x, layers, seq_cu, (H, hd, N, P, L) = _stack_case(3)
    res = oracle.stack_forward(x, layers + layers[:1], seq_cu, H, hd, N, P, L, "test", first_layer=1)
    for l, r in enumerate(res):
        ref_cu = oracle.segment(seq_cu, P, 1 + l)[0]
        np.testing.assert_array_equal(r["chunk_cu"], ref_cu)
    # offsets repeat with period P: layers 1 and 1 + P chunk alike
    np.testing.assert_array_equal(res[0]["chunk_cu"], oracle.segment(seq_cu, P, 1 + P)[0])


def test_chain_is_one_layer_on_the_rounded_output():
    x, layers, seq_cu, (H, hd, N, P, L) = _stack_case(2)
    two = oracle.stack_forward(x, layers, seq_cu, H, hd, N, P, L, "test")
    first = oracle.stack_forward(x, layers[:1], seq_cu, H, hd, N, P, L, "test")
    np.testing.assert_array_equal(two[0]["out"], first[0]["out"])
    x1 = oracle.round_to_bf16(first[0]["out"].reshape(x.shape))
    second = oracle.stack_forward(x1, layers[1:], seq_cu, H, hd, N, P, L, "test", first_layer=1)
    np.testing.assert_array_equal(two[1]["out"], second[0]["out"])


def test_one_layer_is_kvssm_forward_on_rounded_projections():
    x, layers, seq_cu, (H, hd, N, P, L) = _stack_case(1)
    d = x.shape[1]
    proj = oracle.round_to_bf16(x @ layers[0]["w"].T)
    inp = {"x": x}
    start = 0
    for name, wd in (("q", d), ("dt_k", d), ("dt_v", d), ("bm_k", N), ("cm_k", N), ("bm_v", N),
                     ("cm_v", N)):
        inp[name] = proj[:, start:start + wd]
        start += wd
    inp.update(layers[0]["params"])
    ref = oracle.kvssm_forward(inp, seq_cu, H, hd, P, 0, L, "test")
    got = oracle.stack_forward(x, layers, seq_cu, H, hd, N, P, L, "test")[0]
    np.testing.assert_array_equal(got["out"], ref["out"])
