"""The named workloads: shapes, chunking and seeds of the five test/bench configurations.

Plain data only (no arithmetic of the method). Both the CPU oracle side (tests, the CPU
baseline) and the GPU side read these, so neither owns them.

Sources for the free parameters: the pith.science review of "Attamba: Attending To
Multi-Token States", section "Assumptions & free parameters" (chunk size P in {4, 8, 64,
128}, leading tokens L, state size, layer-index offset), and its section "What carries the
argument" (M_train / M_test / sliding-window masks, cyclic chunk offset by layer index).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    dtype: str          # "fp32" or "bf16": type of activations in HBM
    B: int              # sequences in the packed batch
    n: int              # tokens per sequence
    d: int              # model width = H * hd (K and V are SSM outputs split into heads)
    H: int
    hd: int
    N: int              # SSM state size per channel
    P: int              # chunk size (uniform chunking)
    L: int              # leading (uncompressed, most recent) tokens
    layer_idx: int      # cyclic chunk offset o = layer_idx mod P
    mode: str           # "train" (M_train) or "test" (M_test)
    chunking: str       # "uniform" or "random"
    seed: int
    chunk_len_lo: int = 2    # random chunking: lengths uniform in [lo, hi]
    chunk_len_hi: int = 16

    @property
    def T(self) -> int:
        return self.B * self.n

    def with_(self, **kw) -> "PrefillConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    dtype: str
    B: int
    ctx: int            # tokens already processed (compressed into ctx/P boundary states)
    d: int
    H: int
    hd: int
    N: int
    P: int
    L: int
    layer_idx: int
    steps: int          # generated tokens
    seed: int

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


TINY_FP32 = PrefillConfig("tiny_fp32", "fp32", B=1, n=256, d=64, H=2, hd=32, N=16, P=4, L=0,
                          layer_idx=0, mode="train", chunking="uniform", seed=0)
TRAIN_BF16 = PrefillConfig("train_bf16", "bf16", B=4, n=2048, d=1024, H=16, hd=64, N=16, P=8,
                           L=64, layer_idx=3, mode="train", chunking="uniform", seed=1)
PREFILL_BF16 = PrefillConfig("prefill_bf16", "bf16", B=2, n=8192, d=2048, H=32, hd=64, N=16,
                             P=8, L=64, layer_idx=0, mode="test", chunking="uniform", seed=2)
VARCHUNK_BF16 = PrefillConfig("varchunk_bf16", "bf16", B=2, n=8192, d=2048, H=32, hd=64, N=16,
                              P=8, L=64, layer_idx=0, mode="test", chunking="random", seed=3)
DECODE_BF16 = DecodeConfig("decode_bf16", "bf16", B=32, ctx=32768, d=4096, H=32, hd=128, N=16,
                           P=4, L=256, layer_idx=0, steps=256, seed=4)

PREFILL_CONFIGS = {c.name: c for c in (TINY_FP32, TRAIN_BF16, PREFILL_BF16, VARCHUNK_BF16)}
DECODE_CONFIGS = {DECODE_BF16.name: DECODE_BF16}
