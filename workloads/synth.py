"""Seeded synthetic inputs for the KV-SSM forward and the decode step.

This module only draws random numbers and rounds them to the storage type; it holds none
of the method's arithmetic, so the CPU oracle and the GPU path can both take their inputs
from here without sharing any computation.

Distributions (the workload text of the five configurations):
  x ~ N(0, 1); every weight ~ N(0, 0.02^2) (std 0.02);
  A = -exp(u), u ~ U[ln 1, ln 16], i.i.d. per (channel, state);
  step-size bias b = softplus^-1(dt0), dt0 = exp(U[ln 1e-3, ln 0.1]) per channel, so that a
  zero pre-activation gives a step size in [1e-3, 0.1];  D = 1.
The per-token projections (q, dt_K, dt_V, Bm/Cm of both SSMs) are x times those weights,
computed in float32 and then rounded to the activation type: the step the method sits
behind, done here only to give the inputs realistic scale and cross-channel correlation.
Random chunk lengths are drawn per sequence from numpy.random.default_rng(seed) with
integers(lo, hi + 1) until the sequence is covered; the last one is cut to fit.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from .configs import DecodeConfig, PrefillConfig

ACT_NAMES = ("x", "q", "dt_k", "dt_v", "bm_k", "cm_k", "bm_v", "cm_v")
PARAM_NAMES = ("A_k", "A_v", "D_k", "D_v", "bias_k", "bias_v")


def torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def draw_chunk_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> list[int]:
    out, total = [], 0
    while total < n:
        length = min(int(rng.integers(lo, hi + 1)), n - total)
        out.append(length)
        total += length
    return out


@dataclass
class PrefillInputs:
    """Activations in the storage type (CPU torch tensors) plus float64 copies of exactly
    those stored values, fp32 parameters, and the sequence/chunk layout."""
    cfg: PrefillConfig
    seq_cu: np.ndarray                 # int32 [S+1]
    chunk_lens: np.ndarray | None      # int32, concatenated per sequence (random chunking)
    act: dict = field(default_factory=dict)      # name -> torch tensor (storage dtype)
    param: dict = field(default_factory=dict)    # name -> torch float32 tensor

    def f64(self, name: str) -> np.ndarray:
        src = self.act.get(name)
        if src is None:
            src = self.param[name]
        return src.to(torch.float64).numpy()


def _params(rng: np.random.Generator, d: int, N: int) -> dict:
    out = {}
    for s in ("k", "v"):
        out[f"A_{s}"] = -np.exp(rng.uniform(np.log(1.0), np.log(16.0), size=(d, N)))
        dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(0.1), size=d))
        out[f"bias_{s}"] = dt0 + np.log(-np.expm1(-dt0))   # inverse of softplus at dt0
        out[f"D_{s}"] = np.ones(d)
    return {k: torch.from_numpy(v.astype(np.float32)) for k, v in out.items()}


def _weights(rng: np.random.Generator, d: int, N: int) -> dict:
    w = {}
    for name, cols in (("q", d), ("dt_k", d), ("dt_v", d),
                       ("bm_k", N), ("cm_k", N), ("bm_v", N), ("cm_v", N)):
        w[name] = rng.standard_normal((d, cols), dtype=np.float32) * np.float32(0.02)
    return w


def _project(x32: np.ndarray, w: dict, dtype: torch.dtype) -> dict:
    act = {"x": torch.from_numpy(x32).to(dtype)}
    for name, mat in w.items():
        act[name] = torch.from_numpy(x32 @ mat).to(dtype)
    return act


def make_prefill(cfg: PrefillConfig, seed: int | None = None) -> PrefillInputs:
    seed = cfg.seed if seed is None else seed
    seq_cu = (np.arange(cfg.B + 1, dtype=np.int64) * cfg.n).astype(np.int32)
    chunk_lens = None
    if cfg.chunking == "random":
        crng = np.random.default_rng(seed)
        lens = []
        for _ in range(cfg.B):
            lens += draw_chunk_lengths(crng, cfg.n, cfg.chunk_len_lo, cfg.chunk_len_hi)
        chunk_lens = np.asarray(lens, dtype=np.int32)
    rng = np.random.default_rng((seed, 1))
    params = _params(rng, cfg.d, cfg.N)
    w = _weights(rng, cfg.d, cfg.N)
    x32 = rng.standard_normal((cfg.T, cfg.d), dtype=np.float32)
    act = _project(x32, w, torch_dtype(cfg.dtype))
    return PrefillInputs(cfg=cfg, seq_cu=seq_cu, chunk_lens=chunk_lens, act=act, param=params)


def make_ragged_prefill(base: PrefillConfig, lengths: list[int], seed: int,
                        chunk_lens: list[int] | None = None) -> PrefillInputs:
    """Packed batch with sequences of the given (possibly zero or unequal) lengths."""
    T = int(sum(lengths))
    seq_cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rng = np.random.default_rng((seed, 1))
    params = _params(rng, base.d, base.N)
    w = _weights(rng, base.d, base.N)
    x32 = rng.standard_normal((T, base.d), dtype=np.float32)
    act = _project(x32, w, torch_dtype(base.dtype))
    cfg = base.with_(B=len(lengths), n=max(lengths) if lengths else 0, seed=seed)
    cl = None if chunk_lens is None else np.asarray(chunk_lens, dtype=np.int32)
    return PrefillInputs(cfg=cfg, seq_cu=seq_cu, chunk_lens=cl, act=act, param=params)


def make_block_inputs(inp: PrefillInputs, K: int, seed: int, gate: bool = True) -> dict:
    """Seeded parameters and inputs of the Mamba-block pieces around both SSMs: depthwise
    convolution taps [d, K] and biases [d] drawn U(-1/sqrt(K), 1/sqrt(K)) (the default
    initialisation of a depthwise convolution, fan-in K), float32; and, if gate, the gate inputs
    z_k, z_v = x W_z with W_z ~ N(0, 0.02^2) like the other projections, computed in float32
    from the stored x and rounded to the activation type. Returns a dict of CPU tensors."""
    rng = np.random.default_rng((seed, 4))
    d = inp.cfg.d
    lim = 1.0 / np.sqrt(K)
    out = {}
    for s in ("k", "v"):
        out[f"conv_w_{s}"] = torch.from_numpy(rng.uniform(-lim, lim, (d, K)).astype(np.float32))
        out[f"conv_b_{s}"] = torch.from_numpy(rng.uniform(-lim, lim, d).astype(np.float32))
    if gate:
        x32 = inp.act["x"].to(torch.float32).numpy()
        for s in ("k", "v"):
            wz = rng.standard_normal((d, d), dtype=np.float32) * np.float32(0.02)
            out[f"z_{s}"] = torch.from_numpy(x32 @ wz).to(inp.act["x"].dtype)
    return out


def make_stack(d: int, N: int, n_layers: int, seed: int) -> list:
    """Weights of a stack of layers: per layer the stacked projection weight [3 d + 4 N, d]
    (q, dt_K, dt_V, Bm_K, Cm_K, Bm_V, Cm_V rows, each ~ N(0, 0.02^2), bf16) and the SSM
    parameters drawn as for make_prefill (float32). CPU tensors."""
    layers = []
    for l in range(n_layers):
        rng = np.random.default_rng((seed, 5, l))
        params = _params(rng, d, N)
        w = rng.standard_normal((3 * d + 4 * N, d), dtype=np.float32) * np.float32(0.02)
        layers.append({"w": torch.from_numpy(w).to(torch.bfloat16), "params": params})
    return layers


@dataclass
class ProjInputs:
    """Layer input x [T, d] and the stacked projection weight w [n_out, d] (one row per
    output feature: q, dt_K, dt_V rows of width d, then Bm_K, Cm_K, Bm_V, Cm_V of width N),
    both in bf16 (CPU tensors), and the segment widths in that order."""
    x: torch.Tensor
    w: torch.Tensor
    widths: list


def make_projection(T: int, d: int, N: int, seed: int) -> ProjInputs:
    """x ~ N(0, 1) and every weight ~ N(0, 0.02^2), as for the prefill inputs."""
    rng = np.random.default_rng((seed, 2))
    widths = [d, d, d, N, N, N, N]
    x = rng.standard_normal((T, d), dtype=np.float32)
    w = rng.standard_normal((sum(widths), d), dtype=np.float32) * np.float32(0.02)
    return ProjInputs(x=torch.from_numpy(x).to(torch.bfloat16),
                      w=torch.from_numpy(w).to(torch.bfloat16), widths=widths)


def make_output_grad(shape, dtype: str, seed: int) -> torch.Tensor:
    """A seeded upstream gradient (of an attention output, an SSM output or a boundary state):
    N(0, 1), rounded to the storage type."""
    rng = np.random.default_rng((seed, 3))
    g = rng.standard_normal(tuple(shape), dtype=np.float32)
    return torch.from_numpy(g).to(torch_dtype(dtype))


@dataclass
class DecodeInputs:
    """Synthetic decode workload: a cache of `n_bound` boundary states and an L-slot window
    per sequence (N(0,1) values rounded to the storage type), zero SSM state, and per-step
    token inputs [steps, B, ...] projected from fresh x ~ N(0, 1)."""
    cfg: DecodeConfig
    n_bound: int
    kb: torch.Tensor        # [B, H, n_bound, hd]
    vb: torch.Tensor
    kw: torch.Tensor        # [B, H, L, hd], slot s holds position p with p mod L == s
    vw: torch.Tensor
    act: dict               # name -> [steps, B, ...] storage dtype
    param: dict


def make_decode(cfg: DecodeConfig, n_bound: int, steps: int | None = None,
                seed: int | None = None, device: str = "cpu") -> DecodeInputs:
    """`n_bound` boundary states per sequence (the caller counts them for cfg.ctx tokens).
    Cache tensors are drawn with torch's seeded generator on `device` (they are large);
    token inputs and parameters with numpy as in make_prefill."""
    steps = cfg.steps if steps is None else steps
    seed = cfg.seed if seed is None else seed
    dtype = torch_dtype(cfg.dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shape_b = (cfg.B, cfg.H, n_bound, cfg.hd)
    shape_w = (cfg.B, cfg.H, cfg.L, cfg.hd)
    kb = torch.randn(shape_b, generator=gen, device=device, dtype=torch.float32).to(dtype)
    vb = torch.randn(shape_b, generator=gen, device=device, dtype=torch.float32).to(dtype)
    kw = torch.randn(shape_w, generator=gen, device=device, dtype=torch.float32).to(dtype)
    vw = torch.randn(shape_w, generator=gen, device=device, dtype=torch.float32).to(dtype)
    rng = np.random.default_rng((seed, 1))
    params = _params(rng, cfg.d, cfg.N)
    w = _weights(rng, cfg.d, cfg.N)
    x32 = rng.standard_normal((steps * cfg.B, cfg.d), dtype=np.float32)
    act = {k: v.reshape(steps, cfg.B, -1) for k, v in _project(x32, w, dtype).items()}
    return DecodeInputs(cfg=cfg, n_bound=n_bound, kb=kb, vb=vb, kw=kw, vw=vw, act=act,
                        param=params)
