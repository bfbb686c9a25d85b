"""Attamba KV-SSM forward on AMD Instinct MI355X (gfx950): HIP kernels behind a C ABI.

The library libattamba.so (built in-tree by `python -m ssm_compressed_chunked_amd.build`)
does all the work; this package is a thin ctypes binding over it with the same names as the
C entry points (attamba_chunk_boundaries -> chunk_boundaries, and so on).
"""
from ._binding import (BF16, DECODE_SCRATCH_BYTES, ERR_CAPACITY, FP32, LIB_PATH, MASK_TEST, MASK_TRAIN, AttambaError, DecodeCache,
                       chunk_attn_bwd, chunk_attn_bwd_workspace, chunk_attn_fwd, chunk_boundaries,
                       chunk_cu_from_lengths,
                       chunk_index, count_chunks, decode_step, input_proj, kvssm_scan,
                       kvssm_scan_bwd, lib, version)

__all__ = ["BF16", "DECODE_SCRATCH_BYTES", "ERR_CAPACITY", "FP32", "LIB_PATH", "MASK_TEST", "MASK_TRAIN", "AttambaError", "DecodeCache",
           "chunk_attn_bwd", "chunk_attn_bwd_workspace", "chunk_attn_fwd", "chunk_boundaries",
           "chunk_cu_from_lengths",
           "chunk_index", "count_chunks", "decode_step", "input_proj", "kvssm_scan",
           "kvssm_scan_bwd", "lib", "version"]
