"""A training step of the path (prefill_forward, then prefill_backward) captured once as a HIP
graph and replayed: every replay reproduces an eager step on the same inputs. Outputs written
with plain stores must match bit for bit; the float32 sums the scan backward accumulates with
atomics (dBm, dCm, dA, dD, dbias) differ only in summation order, so they are held to 1e-4 of
their largest magnitude. Before each replay the captured outputs are overwritten with NaN, and
eager steps run between the replays, so a replay that skipped a launch or read a stale buffer
would show.
"""
import sys

import pytest
import torch

import ssm_compressed_chunked_amd as att
from ssm_compressed_chunked_amd.pipeline import prefill_backward, prefill_forward
from workloads import TRAIN_BF16, make_output_grad, make_prefill

pytestmark = pytest.mark.gpu

EXACT = ("out", "lse", "dq", "dk", "dv", "dkb", "dvb", "dx_k", "dx_v", "ddt_k", "ddt_v")
SUMS = ("dbm_k", "dcm_k", "dbm_v", "dcm_v", "dA_k", "dA_v", "dD_k", "dD_v", "dbias_k", "dbias_v")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_train_step_graph_replays_match_eager():
    cfg = TRAIN_BF16
    T, H, hd = cfg.T, cfg.H, cfg.hd
    say(f"graph replay of the training step at {cfg.name}")
    inp = make_prefill(cfg)
    act = {k: v.cuda() for k, v in inp.act.items()}
    par = {k: v.cuda() for k, v in inp.param.items()}
    act["seq_cu"] = torch.from_numpy(inp.seq_cu).cuda()
    dout = make_output_grad((T, H, hd), cfg.dtype, seed=42).cuda()

    def step():
        s = torch.cuda.current_stream()
        res = prefill_forward(act, par, inp.seq_cu, H, hd, cfg.P, cfg.layer_idx, cfg.L,
                              att.MASK_TRAIN, stream=s)
        g = prefill_backward(res, act, par, dout, H, hd, cfg.L, att.MASK_TRAIN, stream=s)
        return {"out": res["out"], "lse": res["lse"], **g}

    ref = {k: v.clone() for k, v in step().items()}
    torch.cuda.synchronize()
    assert set(ref) >= set(EXACT + SUMS)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        outs = step()
    torch.cuda.synchronize()

    for r in range(3):
        for t in outs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in EXACT:
            assert torch.equal(outs[name], ref[name]), f"replay {r}: {name} differs from the eager step"
        for name in SUMS:
            top = float(ref[name].abs().max())
            err = float((outs[name] - ref[name]).abs().max())
            assert err <= 1e-4 * max(top, 1e-30), f"replay {r}: {name} max error {err:.3e} (max |ref| {top:.3e})"
        say(f"  replay {r} matches")
        step()                      # eager work between the replays
        torch.cuda.synchronize()
