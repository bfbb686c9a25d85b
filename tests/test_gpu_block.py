"""GPU parity of the Mamba-block variant of the KV-SSM scan (causal depthwise convolution with
SiLU on each SSM's input, SiLU gate on its output, both restarting at chunk starts) against the
oracle's ssm_block_scan, element by element: per-token outputs y_k, y_v and the boundary states
kb, vb (the gated outputs at chunk ends). Bars as for the plain scan: float32 1e-4 relative
(+1e-5), bf16 2e-2 absolute + 2e-2 relative."""
import sys

import numpy as np
import pytest
import torch

import oracle
import ssm_compressed_chunked_amd as att
from ssm_compressed_chunked_amd.pipeline import chunk_layout
from workloads import PREFILL_BF16, TINY_FP32, make_block_inputs, make_prefill, make_ragged_prefill

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_close(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = 1e-4 * np.abs(ref) + 1e-5 if dtype == "fp32" else 2e-2 + 2e-2 * np.abs(ref)
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; max err "
                           f"{err.max():.3e}")


# (dtype, lengths, P or None for random chunks, layer, N, K (0: no conv), gate)
CASES = [
    ("bf16", [203, 37, 64], 8, 3, 16, 4, True),     # chunks of 8 (one-block path) + partial ones
    ("fp32", [150, 61], None, 0, 16, 3, False),     # random chunks of 2..16 (blocks of 8 carry)
    ("bf16", [96, 33], 8, 1, 16, 0, True),          # gate only
    ("fp32", [300], 64, 5, 16, 2, True),            # chunks of 64: eight blocks carry the window
    ("bf16", [120, 19], 8, 0, 32, 4, True),         # N = 32
    ("fp32", [77], 4, 2, 16, 1, False),             # one tap: xc = silu(w x + b)
]


@pytest.mark.parametrize("dtype,lens,P,layer,N,K,gate", CASES)
def test_block_scan_matches_oracle(dtype, lens, P, layer, N, K, gate):
    say(f"block scan dtype={dtype} lens={lens} P={P} layer={layer} N={N} K={K} gate={gate}")
    base = TINY_FP32 if dtype == "fp32" else PREFILL_BF16
    cfg = base.with_(d=128, H=2, hd=64, N=N, P=P or 8, layer_idx=layer)
    chunk_lens = None
    if P is None:
        rng = np.random.default_rng(11)
        chunk_lens = []
        for n in lens:
            tot = 0
            while tot < n:
                c = min(int(rng.integers(2, 17)), n - tot)
                chunk_lens.append(c)
                tot += c
    inp = make_ragged_prefill(cfg, lens, seed=21 + K, chunk_lens=chunk_lens)
    blk = make_block_inputs(inp, max(K, 1), seed=3 + K, gate=gate)
    if K == 0:
        blk = {k: v for k, v in blk.items() if k.startswith("z_")}
    act = {k: v.cuda() for k, v in inp.act.items()}
    par = {k: v.cuda() for k, v in inp.param.items()}
    block = {k: v.cuda() for k, v in blk.items()}
    T = int(inp.seq_cu[-1])
    seq_cu = torch.from_numpy(inp.seq_cu).cuda()
    lay = chunk_layout(inp.seq_cu, seq_cu, T, P, layer, chunk_lens=chunk_lens)
    s = att.kvssm_scan(act["x"], act["dt_k"], act["dt_v"], act["bm_k"], act["cm_k"], act["bm_v"],
                       act["cm_v"], par["A_k"], par["A_v"], par["D_k"], par["D_v"], par["bias_k"],
                       par["bias_v"], lay.chunk_cu, block=block)
    torch.cuda.synchronize()
    ref_cu = oracle.segment(inp.seq_cu, P, layer, chunk_lens)[0]
    np.testing.assert_array_equal(lay.chunk_cu.cpu().numpy(), ref_cu)
    f = {k: inp.f64(k) for k in list(inp.act) + list(inp.param)}
    for tag in ("k", "v"):
        ref = oracle.ssm_block_scan(
            f["x"], f[f"dt_{tag}"], f[f"bias_{tag}"], f[f"A_{tag}"], f[f"bm_{tag}"], f[f"cm_{tag}"],
            f[f"D_{tag}"], ref_cu,
            conv_w=blk[f"conv_w_{tag}"].double().numpy() if K else None,
            conv_b=blk[f"conv_b_{tag}"].double().numpy() if K else None,
            z=blk[f"z_{tag}"].double().numpy() if gate else None)
        check_close(s[f"y_{tag}"].float().cpu().numpy(), ref, dtype, f"y_{tag}")
        check_close(s[f"{tag}b"].float().cpu().numpy(), oracle.boundary_states(ref, ref_cu), dtype,
                    f"{tag}b")


def test_block_without_pieces_equals_plain_scan():
    """A block argument with no convolution and no gate launches the plain scan: bit-identical."""
    cfg = PREFILL_BF16.with_(B=2, n=100, d=128, H=2, hd=64)
    inp = make_prefill(cfg, seed=9)
    act = {k: v.cuda() for k, v in inp.act.items()}
    par = {k: v.cuda() for k, v in inp.param.items()}
    seq_cu = torch.from_numpy(inp.seq_cu).cuda()
    lay = chunk_layout(inp.seq_cu, seq_cu, cfg.T, cfg.P, 1)
    args = (act["x"], act["dt_k"], act["dt_v"], act["bm_k"], act["cm_k"], act["bm_v"], act["cm_v"],
            par["A_k"], par["A_v"], par["D_k"], par["D_v"], par["bias_k"], par["bias_v"], lay.chunk_cu)
    a = att.kvssm_scan(*args)
    b = att.kvssm_scan(*args, block={})
    torch.cuda.synchronize()
    for k in ("y_k", "y_v", "kb", "vb"):
        assert torch.equal(a[k], b[k]), k


def test_block_scan_full_size_every_sequence():
    """The variant at the prefill workload's full size (2 x 8192 tokens, d = 2048, P = 8), both
    SSMs, every token and chunk of both sequences against the oracle."""
    cfg = PREFILL_BF16
    say("block scan full size")
    inp = make_prefill(cfg)
    blk = make_block_inputs(inp, 4, seed=13, gate=True)
    act = {k: v.cuda() for k, v in inp.act.items()}
    par = {k: v.cuda() for k, v in inp.param.items()}
    block = {k: v.cuda() for k, v in blk.items()}
    seq_cu = torch.from_numpy(inp.seq_cu).cuda()
    lay = chunk_layout(inp.seq_cu, seq_cu, cfg.T, cfg.P, cfg.layer_idx)
    s = att.kvssm_scan(act["x"], act["dt_k"], act["dt_v"], act["bm_k"], act["cm_k"], act["bm_v"],
                       act["cm_v"], par["A_k"], par["A_v"], par["D_k"], par["D_v"], par["bias_k"],
                       par["bias_v"], lay.chunk_cu, block=block)
    torch.cuda.synchronize()
    ref_cu = oracle.segment(inp.seq_cu, cfg.P, cfg.layer_idx)[0]
    f = {k: inp.f64(k) for k in list(inp.act) + list(inp.param)}
    got = {k: s[k].float().cpu().numpy() for k in ("y_k", "y_v", "kb", "vb")}
    for si in range(cfg.B):
        a, b = int(inp.seq_cu[si]), int(inp.seq_cu[si + 1])
        cu = ref_cu[(ref_cu >= a) & (ref_cu <= b)] - a
        q0 = int(np.searchsorted(ref_cu, a))
        for tag in ("k", "v"):
            ref = oracle.ssm_block_scan(
                f["x"][a:b], f[f"dt_{tag}"][a:b], f[f"bias_{tag}"], f[f"A_{tag}"],
                f[f"bm_{tag}"][a:b], f[f"cm_{tag}"][a:b], f[f"D_{tag}"], cu,
                conv_w=blk[f"conv_w_{tag}"].double().numpy(), conv_b=blk[f"conv_b_{tag}"].double().numpy(),
                z=blk[f"z_{tag}"][a:b].double().numpy())
            check_close(got[f"y_{tag}"][a:b], ref, "bf16", f"y_{tag} of sequence {si}")
            check_close(got[f"{tag}b"][q0:q0 + len(cu) - 1], oracle.boundary_states(ref, cu), "bf16",
                        f"{tag}b of sequence {si}")
        say(f"  sequence {si}: matches")
