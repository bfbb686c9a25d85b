"""The prefill forward as the three library calls in order (marshalling only):
segmentation -> KV-SSM scan -> chunk attention, all enqueued on the current stream."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import _binding as B


@dataclass
class ChunkLayout:
    n_chunks: int
    chunk_cu: torch.Tensor      # [n_chunks + 1] int32
    token_chunk: torch.Tensor   # [T] int32
    is_end: torch.Tensor        # [T] uint8


def chunk_layout(seq_cu_host, seq_cu: torch.Tensor, T: int, P: int | None, layer_idx: int,
                 chunk_lens=None, stream=None) -> ChunkLayout:
    """Uniform chunks with cyclic offset (computed on the GPU), or explicit chunk lengths
    (validated and summed on the host, per-token maps on the GPU)."""
    if chunk_lens is None:
        n = B.count_chunks(seq_cu_host, P, layer_idx)
        cu, tc, ie = B.chunk_boundaries(seq_cu, T, P, layer_idx, n, stream=stream)
    else:
        cu_host = B.chunk_cu_from_lengths(seq_cu_host, chunk_lens)
        n = len(cu_host) - 1
        cu = torch.from_numpy(cu_host).to(seq_cu.device, non_blocking=False)
        tc, ie = B.chunk_index(cu, T, stream=stream)
    return ChunkLayout(n, cu, tc, ie)


def prefill_forward(act: dict, params: dict, seq_cu_host, H: int, hd: int, P: int | None,
                    layer_idx: int, L: int, mode: int, chunk_lens=None, layout=None,
                    stream=None, want_lse: bool = True) -> dict:
    """act: device tensors x, q, dt_k, dt_v, bm_k, cm_k, bm_v, cm_v; params: A_k, A_v, D_k,
    D_v, bias_k, bias_v (float32). Returns the layout, the scan outputs and (out, lse)."""
    x = act["x"]
    T, d = x.shape
    seq_cu_host = np.asarray(seq_cu_host, dtype=np.int32)
    seq_cu = act.get("seq_cu")
    if seq_cu is None:
        seq_cu = torch.from_numpy(seq_cu_host).to(x.device)
    if layout is None:
        layout = chunk_layout(seq_cu_host, seq_cu, T, P, layer_idx, chunk_lens, stream)
    scan = B.kvssm_scan(act["x"], act["dt_k"], act["dt_v"], act["bm_k"], act["cm_k"],
                        act["bm_v"], act["cm_v"], params["A_k"], params["A_v"], params["D_k"],
                        params["D_v"], params["bias_k"], params["bias_v"], layout.chunk_cu,
                        stream=stream)
    max_len = int(np.max(np.diff(seq_cu_host))) if len(seq_cu_host) > 1 else 0
    n = layout.n_chunks
    out, lse = B.chunk_attn_fwd(act["q"].view(T, H, hd), scan["y_k"].view(T, H, hd),
                                scan["y_v"].view(T, H, hd), scan["kb"].view(n, H, hd),
                                scan["vb"].view(n, H, hd), seq_cu, layout.chunk_cu,
                                layout.token_chunk, max(max_len, 1), L, mode,
                                return_lse=want_lse, stream=stream)
    return dict(layout=layout, scan=scan, out=out, lse=lse, seq_cu=seq_cu)
