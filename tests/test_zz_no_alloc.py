"""The decode step that allocates nothing (attamba_decode_step_noalloc, scratch in the library's
static device array) against attamba_decode_step (scratch in the caller's workspace), through
the C ABI: two calls in a row, the second on a smaller cache, so the second reads a scratch that
still holds the first call's partials. Outputs and the updated caches must be identical (the
two entry points share every kernel; only the scratch address differs)."""
import sys

import numpy as np
import pytest
import torch

import ssm_compressed_chunked_amd as att
from workloads import DECODE_BF16, make_decode

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cache_pair(cfg, n_bound, seed):
    """Two caches with the same contents (the decode workload's synthetic cache)."""
    inp = make_decode(cfg, n_bound=n_bound, steps=2, seed=seed, device="cuda")
    cap = n_bound + 4
    caches = []
    for _ in range(2):
        c = att.DecodeCache(cfg.B, cfg.H, cfg.hd, cfg.N, cfg.P, cfg.L, cfg.layer_idx, cap,
                            inp.kb.dtype, inp.param, pos=cfg.ctx, n_bound=n_bound)
        c.kb[:, :, :n_bound] = inp.kb
        c.vb[:, :, :n_bound] = inp.vb
        c.kw.copy_(inp.kw)
        c.vw.copy_(inp.vw)
        caches.append(c)
    act = {k: v.cuda() for k, v in inp.act.items()}
    return caches, act


@pytest.mark.parametrize("big,small", [
    (dict(B=8, ctx=16384, H=32, hd=128), dict(B=2, ctx=2048, H=8, hd=64)),
])
def test_noalloc_decode_matches_workspace_decode(big, small):
    for tag, shape in (("first (larger)", big), ("second (smaller)", small)):
        cfg = DECODE_BF16.with_(d=shape["H"] * shape["hd"], **shape)
        n_bound = att.count_chunks([0, cfg.ctx], cfg.P, cfg.layer_idx)
        need = cfg.B * cfg.H * (cfg.hd + 2) * 4 * (-(-(n_bound + 4 + cfg.L) // 256) + 1)
        assert need <= att.DECODE_SCRATCH_BYTES, (tag, need)
        say(f"no-alloc decode, {tag} call: B={cfg.B} ctx={cfg.ctx} H={cfg.H} hd={cfg.hd} "
            f"(scratch {need} of {att.DECODE_SCRATCH_BYTES} bytes)")
        (ref_cache, na_cache), act = _cache_pair(cfg, n_bound, seed=7 + cfg.B)
        outs = []
        for cache, noalloc in ((ref_cache, False), (na_cache, True)):
            out = torch.empty((cfg.B, cfg.H, cfg.hd), dtype=cache.dtype, device="cuda")
            att.decode_step(cache, act["q"][0].view(cfg.B, cfg.H, cfg.hd), act["x"][0], act["dt_k"][0],
                            act["dt_v"][0], act["bm_k"][0], act["cm_k"][0], act["bm_v"][0],
                            act["cm_v"][0], out=out, noalloc=noalloc)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.isfinite(outs[0].float()).all()
        assert torch.equal(outs[0], outs[1]), f"{tag}: outputs differ"
        for name in ("kb", "vb", "kw", "vw", "h_k", "h_v"):
            assert torch.equal(getattr(ref_cache, name), getattr(na_cache, name)), f"{tag}: cache {name} differs"
        assert (ref_cache.pos, ref_cache.n_bound) == (na_cache.pos, na_cache.n_bound)
