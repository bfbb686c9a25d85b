"""GPU parity of a stack of layers (pith.science "What carries the argument": the chunk offset
shifts by layer index): layer l projects its input on the matrix cores, runs the KV-SSM forward
at offset l mod P, and hands its attention output to layer l + 1. The whole stack prefills a
prompt, every layer hands its prefill to its own decode cache on the device, and the next
tokens are decoded through the stack. Every layer's prefill rows and decoded outputs are
compared with the oracle's chain over the full length (decoding is causal, so its output at a
position equals the full-length prefill's row there), bf16 bar 2e-2 absolute + 2e-2 relative."""
import sys

import numpy as np
import pytest
import torch

import oracle
import ssm_compressed_chunked_amd as att
from ssm_compressed_chunked_amd.pipeline import model_decode_caches, model_decode_step, model_forward
from workloads import make_stack

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= 2e-2 + 2e-2 * np.abs(ref))
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside tolerance; max err {err.max():.3e}"


@pytest.mark.parametrize("n_layers,P,L,noalloc", [(3, 4, 5, False), (4, 3, 7, True)])
def test_stack_prefill_then_decode(n_layers, P, L, noalloc):
    B, d, H, hd, N, n0, steps = 2, 128, 2, 64, 16, 21, 6
    n = n0 + steps
    say(f"stack of {n_layers} layers, P={P} L={L}, prefill {n0} then decode {steps} (noalloc={noalloc})")
    rng = np.random.default_rng(60 + n_layers)
    x_full = torch.from_numpy(rng.standard_normal((B, n, d)).astype(np.float32)).to(torch.bfloat16)
    stack = make_stack(d, N, n_layers, seed=61)
    # oracle: the chain over the full length
    seq_full = np.arange(B + 1) * n
    ref = oracle.stack_forward(
        x_full.reshape(B * n, d).double().numpy(),
        [{"w": lay["w"].double().numpy(), "params": {k: v.double().numpy() for k, v in lay["params"].items()}}
         for lay in stack], seq_full, H, hd, N, P, L, "test")
    ref_out = [r["out"].reshape(B, n, H, hd) for r in ref]
    # GPU: prefill the first n0 tokens of each sequence through the stack
    layers = [{"w": lay["w"].cuda(), "params": {k: v.cuda() for k, v in lay["params"].items()}}
              for lay in stack]
    seq_cu = (np.arange(B + 1) * n0).astype(np.int32)
    x0 = x_full[:, :n0].reshape(B * n0, d).contiguous().cuda()
    res = model_forward(x0, layers, seq_cu, H, hd, N, P, L, att.MASK_TEST, h_last=True)
    torch.cuda.synchronize()
    for l, r in enumerate(res):
        np.testing.assert_array_equal(r["layout"].chunk_cu.cpu().numpy(),
                                      oracle.segment(seq_cu, P, l)[0])
        check_close(r["out"].float().cpu().numpy().reshape(B, n0, H, hd), ref_out[l][:, :n0],
                    f"prefill output of layer {l}")
    caches = model_decode_caches(res, layers, seq_cu, H, hd, N, P, L, cap=n // P + 2)
    for s in range(steps):
        x_tok = x_full[:, n0 + s].contiguous().cuda()
        outs = model_decode_step(caches, x_tok, layers, noalloc=noalloc)
        torch.cuda.synchronize()
        for l, o in enumerate(outs):
            check_close(o.float().cpu().numpy(), ref_out[l][:, n0 + s],
                        f"decode step {s}, layer {l}")
    say("  stack matches the oracle chain")
