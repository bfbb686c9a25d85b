"""Thin ctypes binding of libattamba.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; PyTorch only provides device
memory and the current stream. The binding checks tensor dtype, device and contiguity,
allocates missing outputs with torch, forwards data pointers, and turns a non-zero status
into an exception carrying attamba_last_error(). If the library is missing it raises.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattamba.so")

OK, ERR_NULL_ARG, ERR_BAD_SHAPE, ERR_BAD_DTYPE, ERR_CAPACITY, ERR_UNSUPPORTED, ERR_HIP = range(7)
# bytes of the static device scratch of attamba_decode_step_noalloc (ATTAMBA_DECODE_SCRATCH_BYTES)
DECODE_SCRATCH_BYTES = 32 << 20
FP32, BF16 = 0, 1
MASK_TRAIN, MASK_TEST = 0, 1

_vp = C.c_void_p
_i32 = C.c_int32
_i32p = C.POINTER(C.c_int32)


class SsmBlockArgs(C.Structure):
    _fields_ = [("conv_width", _i32), ("conv_w_k", _vp), ("conv_b_k", _vp), ("conv_w_v", _vp),
                ("conv_b_v", _vp), ("z_k", _vp), ("z_v", _vp)]


class ScanArgs(C.Structure):
    _fields_ = [("T", _i32), ("d", _i32), ("N", _i32), ("dtype", _i32), ("n_chunks", _i32),
                ("chunk_cu", _vp), ("x", _vp), ("dt_k", _vp), ("dt_v", _vp), ("bm_k", _vp),
                ("cm_k", _vp), ("bm_v", _vp), ("cm_v", _vp), ("A_k", _vp), ("A_v", _vp),
                ("D_k", _vp), ("D_v", _vp), ("bias_k", _vp), ("bias_v", _vp), ("y_k", _vp),
                ("y_v", _vp), ("kb", _vp), ("vb", _vp), ("seq_cu", _vp), ("S", _i32),
                ("h_last_k", _vp), ("h_last_v", _vp), ("x_v", _vp),
                ("block", C.POINTER(SsmBlockArgs))]


PROJ_MAX_SEGMENTS = 12


class ProjArgs(C.Structure):
    _fields_ = [("T", _i32), ("d", _i32), ("n_out", _i32), ("dtype", _i32), ("n_seg", _i32),
                ("x", _vp), ("w", _vp), ("seg_start", _i32 * (PROJ_MAX_SEGMENTS + 1)),
                ("out", _vp * PROJ_MAX_SEGMENTS)]


class AttnArgs(C.Structure):
    _fields_ = [("T", _i32), ("H", _i32), ("hd", _i32), ("dtype", _i32), ("S", _i32),
                ("max_seqlen", _i32), ("n_chunks", _i32), ("L", _i32), ("mode", _i32),
                ("scale", C.c_float), ("q", _vp), ("k", _vp), ("v", _vp), ("kb", _vp),
                ("vb", _vp), ("seq_cu", _vp), ("chunk_cu", _vp), ("token_chunk", _vp),
                ("out", _vp), ("lse", _vp)]


class DecodePrefixStruct(C.Structure):
    _fields_ = [("S", _i32), ("n0", _i32), ("seq_cu_host", _i32p), ("seq_cu", _vp),
                ("token_chunk", _vp), ("y_k", _vp), ("y_v", _vp), ("kb", _vp), ("vb", _vp),
                ("h_last_k", _vp), ("h_last_v", _vp)]


class AttnBwdArgs(C.Structure):
    _fields_ = [("fwd", AttnArgs), ("dout", _vp), ("dq", _vp), ("dk", _vp), ("dv", _vp),
                ("dkb", _vp), ("dvb", _vp), ("workspace", _vp), ("workspace_elems", C.c_size_t)]


class ScanBwdArgs(C.Structure):
    _fields_ = [("fwd", ScanArgs), ("gy_k", _vp), ("gy_v", _vp), ("gkb", _vp), ("gvb", _vp),
                ("dx_k", _vp), ("dx_v", _vp), ("ddt_k", _vp), ("ddt_v", _vp), ("dbm_k", _vp),
                ("dcm_k", _vp), ("dbm_v", _vp), ("dcm_v", _vp), ("dA_k", _vp), ("dA_v", _vp),
                ("dD_k", _vp), ("dD_v", _vp), ("dbias_k", _vp), ("dbias_v", _vp)]


class DecodeCacheStruct(C.Structure):
    _fields_ = [("B", _i32), ("H", _i32), ("hd", _i32), ("d", _i32), ("N", _i32), ("P", _i32),
                ("L", _i32), ("layer_idx", _i32), ("cap", _i32), ("dtype", _i32),
                ("pos", C.c_int64), ("n_bound", _i32), ("kb", _vp), ("vb", _vp), ("kw", _vp),
                ("vw", _vp), ("h_k", _vp), ("h_v", _vp), ("A_k", _vp), ("A_v", _vp),
                ("D_k", _vp), ("D_v", _vp), ("bias_k", _vp), ("bias_v", _vp),
                ("workspace", _vp), ("workspace_bytes", C.c_size_t)]


class DecodeInputsStruct(C.Structure):
    _fields_ = [("q", _vp), ("x", _vp), ("dt_k", _vp), ("dt_v", _vp), ("bm_k", _vp),
                ("cm_k", _vp), ("bm_v", _vp), ("cm_v", _vp), ("out", _vp)]


EXPORTS = {
    "attamba_version": ([], C.c_char_p),
    "attamba_status_string": ([C.c_int], C.c_char_p),
    "attamba_last_error": ([], C.c_char_p),
    "attamba_count_chunks": ([_i32p, _i32, _i32, _i32, _i32p], C.c_int),
    "attamba_chunk_cu_from_lengths": ([_i32p, _i32, _i32p, _i32, _i32p], C.c_int),
    "attamba_chunk_boundaries": ([_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp], C.c_int),
    "attamba_chunk_index": ([_vp, _i32, _i32, _vp, _vp, _vp], C.c_int),
    "attamba_kvssm_scan": ([C.POINTER(ScanArgs), _vp], C.c_int),
    "attamba_chunk_attn_fwd": ([C.POINTER(AttnArgs), _vp], C.c_int),
    "attamba_input_proj": ([C.POINTER(ProjArgs), _vp], C.c_int),
    "attamba_decode_workspace_size": ([C.POINTER(DecodeCacheStruct), C.POINTER(C.c_size_t)],
                                      C.c_int),
    "attamba_decode_step": ([C.POINTER(DecodeCacheStruct), C.POINTER(DecodeInputsStruct), _vp],
                            C.c_int),
    "attamba_decode_step_noalloc": ([C.POINTER(DecodeCacheStruct), C.POINTER(DecodeInputsStruct),
                                     _vp], C.c_int),
    "attamba_decode_load_prefix": ([C.POINTER(DecodeCacheStruct), C.POINTER(DecodePrefixStruct), _vp],
                                   C.c_int),
    "attamba_chunk_attn_bwd": ([C.POINTER(AttnBwdArgs), _vp], C.c_int),
    "attamba_chunk_attn_bwd_workspace_size": ([C.POINTER(AttnBwdArgs), C.POINTER(C.c_size_t)], C.c_int),
    "attamba_kvssm_scan_bwd": ([C.POINTER(ScanBwdArgs), _vp], C.c_int),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m ssm_compressed_chunked_amd.build")
        h = C.CDLL(LIB_PATH)
        for name, (argtypes, restype) in EXPORTS.items():
            fn = getattr(h, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _lib = h
    return _lib


class AttambaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{lib().attamba_status_string(status).decode()}: {detail}")
        self.status = status


def _check(status: int) -> None:
    if status != OK:
        raise AttambaError(status, lib().attamba_last_error().decode())


def version() -> str:
    return lib().attamba_version().decode()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor | None, name: str, dtype=None, numel=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


# ------------------------------------------------------------------------------------------
def count_chunks(seq_cu_host, P: int, layer_idx: int) -> int:
    s = _host_i32(seq_cu_host)
    n = C.c_int32()
    _check(lib().attamba_count_chunks(s.ctypes.data_as(_i32p), len(s) - 1, P, layer_idx,
                                      C.byref(n)))
    return n.value


def chunk_cu_from_lengths(seq_cu_host, chunk_lens) -> np.ndarray:
    s = _host_i32(seq_cu_host)
    cl = _host_i32(chunk_lens)
    out = np.zeros(len(cl) + 1, dtype=np.int32)
    _check(lib().attamba_chunk_cu_from_lengths(s.ctypes.data_as(_i32p), len(s) - 1,
                                               cl.ctypes.data_as(_i32p), len(cl),
                                               out.ctypes.data_as(_i32p)))
    return out


def chunk_boundaries(seq_cu: torch.Tensor, T: int, P: int, layer_idx: int, n_chunks: int,
                     chunk_cu=None, token_chunk=None, is_end=None, stream=None):
    """Uniform chunking with cyclic offset on the GPU. Returns (chunk_cu, token_chunk, is_end)."""
    dev = seq_cu.device
    if chunk_cu is None:
        chunk_cu = torch.empty(n_chunks + 1, dtype=torch.int32, device=dev)
    if token_chunk is None:
        token_chunk = torch.empty(T, dtype=torch.int32, device=dev)
    if is_end is None:
        is_end = torch.empty(T, dtype=torch.uint8, device=dev)
    _check(lib().attamba_chunk_boundaries(
        _dev(seq_cu, "seq_cu", torch.int32), seq_cu.numel() - 1, T, P, layer_idx, n_chunks,
        _dev(chunk_cu, "chunk_cu", torch.int32, n_chunks + 1),
        _dev(token_chunk, "token_chunk", torch.int32, T), _dev(is_end, "is_end", torch.uint8, T),
        _stream(stream)))
    return chunk_cu, token_chunk, is_end


def chunk_index(chunk_cu: torch.Tensor, T: int, token_chunk=None, is_end=None, stream=None):
    dev = chunk_cu.device
    if token_chunk is None:
        token_chunk = torch.empty(T, dtype=torch.int32, device=dev)
    if is_end is None:
        is_end = torch.empty(T, dtype=torch.uint8, device=dev)
    _check(lib().attamba_chunk_index(
        _dev(chunk_cu, "chunk_cu", torch.int32), chunk_cu.numel() - 1, T,
        _dev(token_chunk, "token_chunk", torch.int32, T), _dev(is_end, "is_end", torch.uint8, T),
        _stream(stream)))
    return token_chunk, is_end


def _scan_inputs(x, dt_k, dt_v, bm_k, cm_k, bm_v, cm_v, A_k, A_v, D_k, D_v, bias_k, bias_v,
                 chunk_cu, x_v) -> ScanArgs:
    """ScanArgs with the sizes and the forward inputs filled in (outputs left NULL)."""
    T, d = x.shape
    N = A_k.shape[1]
    act = x.dtype
    a = ScanArgs()
    a.T, a.d, a.N, a.dtype, a.n_chunks = T, d, N, _dtype_code(x), chunk_cu.numel() - 1
    a.chunk_cu = _dev(chunk_cu, "chunk_cu", torch.int32)
    for name, t, n in (("x", x, T * d), ("dt_k", dt_k, T * d), ("dt_v", dt_v, T * d),
                       ("bm_k", bm_k, T * N), ("cm_k", cm_k, T * N), ("bm_v", bm_v, T * N),
                       ("cm_v", cm_v, T * N)):
        setattr(a, name, _dev(t, name, act, n))
    for name, t, n in (("A_k", A_k, d * N), ("A_v", A_v, d * N), ("D_k", D_k, d),
                       ("D_v", D_v, d), ("bias_k", bias_k, d), ("bias_v", bias_v, d)):
        setattr(a, name, _dev(t, name, torch.float32, n))
    a.x_v = _dev(x_v, "x_v", act, T * d)
    return a


def kvssm_scan(x, dt_k, dt_v, bm_k, cm_k, bm_v, cm_v, A_k, A_v, D_k, D_v, bias_k, bias_v,
               chunk_cu, *, y_k=None, y_v=None, kb=None, vb=None, boundaries=True,
               seq_cu=None, h_last=False, x_v=None, block=None, stream=None) -> dict:
    """Both selective scans in one pass. x_v: optional separate input of SSM_V (x then feeds
    SSM_K only). block: optional Mamba-block pieces, a dict with conv_w_k, conv_b_k, conv_w_v,
    conv_b_v (float32 [d, K] taps and [d] biases, K <= 4) and/or z_k, z_v ([T, d] gate inputs in
    the activation dtype). Returns dict(y_k, y_v, kb, vb, h_last_k, h_last_v)."""
    T, d = x.shape
    N = A_k.shape[1]
    n_chunks = chunk_cu.numel() - 1
    act = x.dtype
    if y_k is None:
        y_k = torch.empty_like(x)
    if y_v is None:
        y_v = torch.empty_like(x)
    if boundaries and kb is None:
        kb = torch.empty((n_chunks, d), dtype=act, device=x.device)
    if boundaries and vb is None:
        vb = torch.empty((n_chunks, d), dtype=act, device=x.device)
    hk = hv = None
    S = 0
    if h_last:
        S = seq_cu.numel() - 1
        hk = torch.empty((S, d, N), dtype=torch.float32, device=x.device)
        hv = torch.empty((S, d, N), dtype=torch.float32, device=x.device)
    a = _scan_inputs(x, dt_k, dt_v, bm_k, cm_k, bm_v, cm_v, A_k, A_v, D_k, D_v, bias_k, bias_v,
                     chunk_cu, x_v)
    a.y_k = _dev(y_k, "y_k", act, T * d)
    a.y_v = _dev(y_v, "y_v", act, T * d)
    a.kb = _dev(kb, "kb", act, n_chunks * d)
    a.vb = _dev(vb, "vb", act, n_chunks * d)
    a.seq_cu = _dev(seq_cu, "seq_cu", torch.int32) if h_last else None
    a.S = S
    a.h_last_k = _dev(hk, "h_last_k")
    a.h_last_v = _dev(hv, "h_last_v")
    if block is not None:
        bl = SsmBlockArgs()
        w_k = block.get("conv_w_k")
        if w_k is not None:
            K = w_k.shape[1]
            bl.conv_width = K
            for name in ("conv_w_k", "conv_w_v"):
                setattr(bl, name, _dev(block[name], name, torch.float32, d * K))
            for name in ("conv_b_k", "conv_b_v"):
                setattr(bl, name, _dev(block[name], name, torch.float32, d))
        for name in ("z_k", "z_v"):
            if block.get(name) is not None:
                setattr(bl, name, _dev(block[name], name, act, T * d))
        a.block = C.pointer(bl)
    _check(lib().attamba_kvssm_scan(C.byref(a), _stream(stream)))
    return dict(y_k=y_k, y_v=y_v, kb=kb, vb=vb, h_last_k=hk, h_last_v=hv)


def kvssm_scan_bwd(x, dt_k, dt_v, bm_k, cm_k, bm_v, cm_v, A_k, A_v, D_k, D_v, bias_k, bias_v,
                   chunk_cu, gy_k, gy_v, *, gkb=None, gvb=None, x_v=None, stream=None) -> dict:
    """Gradients of both selective scans for the output gradients gy_k, gy_v [T, d] (and gkb,
    gvb [n_chunks, d] of the boundary states). dx_k / dx_v are the gradients of each SSM's input
    (when both read x, x's gradient is their sum). Returns a dict of the gradient tensors."""
    T, d = x.shape
    N = A_k.shape[1]
    n_chunks = chunk_cu.numel() - 1
    act = x.dtype
    dev = x.device
    b = ScanBwdArgs()
    b.fwd = _scan_inputs(x, dt_k, dt_v, bm_k, cm_k, bm_v, cm_v, A_k, A_v, D_k, D_v, bias_k,
                         bias_v, chunk_cu, x_v)
    b.gy_k = _dev(gy_k, "gy_k", act, T * d)
    b.gy_v = _dev(gy_v, "gy_v", act, T * d)
    b.gkb = _dev(gkb, "gkb", act, n_chunks * d)
    b.gvb = _dev(gvb, "gvb", act, n_chunks * d)
    g = {}
    for name in ("dx_k", "dx_v", "ddt_k", "ddt_v"):
        g[name] = torch.empty((T, d), dtype=act, device=dev)
    for name in ("dbm_k", "dcm_k", "dbm_v", "dcm_v"):
        g[name] = torch.empty((T, N), dtype=torch.float32, device=dev)
    for name in ("dA_k", "dA_v"):
        g[name] = torch.empty((d, N), dtype=torch.float32, device=dev)
    for name in ("dD_k", "dD_v", "dbias_k", "dbias_v"):
        g[name] = torch.empty((d,), dtype=torch.float32, device=dev)
    for name, t in g.items():
        setattr(b, name, t.data_ptr())
    _check(lib().attamba_kvssm_scan_bwd(C.byref(b), _stream(stream)))
    return g


def input_proj(x: torch.Tensor, w: torch.Tensor, widths, outs=None, stream=None):
    """Y = x w^T (bf16, fp32 accumulation) split by features into len(widths) row-major
    tensors [T, widths[i]]: x [T, d], w [sum(widths), d]. Returns the list of outputs."""
    T, d = x.shape
    n_out = int(sum(widths))
    if w.shape != (n_out, d):
        raise ValueError(f"w has shape {tuple(w.shape)}, expected {(n_out, d)}")
    if not 1 <= len(widths) <= PROJ_MAX_SEGMENTS:
        raise ValueError(f"1 .. {PROJ_MAX_SEGMENTS} output segments")
    if outs is None:
        outs = [torch.empty((T, int(wd)), dtype=x.dtype, device=x.device) for wd in widths]
    a = ProjArgs()
    a.T, a.d, a.n_out, a.n_seg = T, d, n_out, len(widths)
    a.dtype = _dtype_code(x)
    a.x = _dev(x, "x", torch.bfloat16, T * d)
    a.w = _dev(w, "w", torch.bfloat16, n_out * d)
    start = 0
    for i, wd in enumerate(widths):
        a.seg_start[i] = start
        a.out[i] = _dev(outs[i], f"out[{i}]", torch.bfloat16, T * int(wd))
        start += int(wd)
    a.seg_start[len(widths)] = start
    _check(lib().attamba_input_proj(C.byref(a), _stream(stream)))
    return outs


def _attn_inputs(q, k, v, kb, vb, seq_cu, chunk_cu, token_chunk, max_seqlen, L, mode,
                 scale) -> AttnArgs:
    """AttnArgs with sizes, mask and inputs filled in (out and lse left NULL)."""
    T, H, hd = q.shape
    n_chunks = chunk_cu.numel() - 1
    act = q.dtype
    a = AttnArgs()
    a.T, a.H, a.hd, a.dtype = T, H, hd, _dtype_code(q)
    a.S, a.max_seqlen, a.n_chunks, a.L, a.mode = seq_cu.numel() - 1, max_seqlen, n_chunks, L, mode
    a.scale = scale
    a.q = _dev(q, "q", act, T * H * hd)
    a.k = _dev(k, "k", act, T * H * hd)
    a.v = _dev(v, "v", act, T * H * hd)
    a.kb = _dev(kb, "kb", act, n_chunks * H * hd)
    a.vb = _dev(vb, "vb", act, n_chunks * H * hd)
    a.seq_cu = _dev(seq_cu, "seq_cu", torch.int32)
    a.chunk_cu = _dev(chunk_cu, "chunk_cu", torch.int32)
    a.token_chunk = _dev(token_chunk, "token_chunk", torch.int32, T)
    return a


def chunk_attn_fwd(q, k, v, kb, vb, seq_cu, chunk_cu, token_chunk, max_seqlen: int, L: int,
                   mode: int, scale: float = 0.0, out=None, lse=None, return_lse: bool = True,
                   stream=None):
    """q, k, v: [T, H, hd]; kb, vb: [n_chunks, H, hd]. Returns (out, lse or None)."""
    T, H, hd = q.shape
    n_chunks = chunk_cu.numel() - 1
    act = q.dtype
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    a = _attn_inputs(q, k, v, kb, vb, seq_cu, chunk_cu, token_chunk, max_seqlen, L, mode, scale)
    a.out = _dev(out, "out", act, T * H * hd)
    a.lse = _dev(lse, "lse", torch.float32, H * T) if lse is not None else None
    _check(lib().attamba_chunk_attn_fwd(C.byref(a), _stream(stream)))
    return out, lse


def chunk_attn_bwd_workspace(T: int, H: int, hd: int, n_chunks: int, dtype, device="cuda"):
    """A workspace for chunk_attn_bwd at these sizes (float32, sized by the library; allocate
    once and pass it to every call of that shape)."""
    b = AttnBwdArgs()
    b.fwd.T, b.fwd.H, b.fwd.hd, b.fwd.n_chunks = T, H, hd, n_chunks
    b.fwd.dtype = BF16 if dtype == torch.bfloat16 else FP32
    need = C.c_size_t(0)
    _check(lib().attamba_chunk_attn_bwd_workspace_size(C.byref(b), C.byref(need)))
    return torch.empty(max(need.value, 1), dtype=torch.float32, device=device)


def chunk_attn_bwd(q, k, v, kb, vb, seq_cu, chunk_cu, token_chunk, max_seqlen: int, L: int,
                   mode: int, out, lse, dout, scale: float = 0.0, workspace=None,
                   stream=None) -> dict:
    """Gradients of the chunk attention for the output gradient dout, given the forward's
    out and lse. Returns dict(dq, dk, dv, dkb, dvb): dk/dv for the per-token keys and values,
    dkb/dvb for the boundary states."""
    T, H, hd = q.shape
    n_chunks = chunk_cu.numel() - 1
    act = q.dtype
    b = AttnBwdArgs()
    b.fwd = _attn_inputs(q, k, v, kb, vb, seq_cu, chunk_cu, token_chunk, max_seqlen, L, mode,
                         scale)
    b.fwd.out = _dev(out, "out", act, T * H * hd)
    b.fwd.lse = _dev(lse, "lse", torch.float32, H * T)
    b.dout = _dev(dout, "dout", act, T * H * hd)
    need = C.c_size_t(0)
    _check(lib().attamba_chunk_attn_bwd_workspace_size(C.byref(b), C.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(need.value, 1), dtype=torch.float32, device=q.device)
    b.workspace = _dev(workspace, "workspace", torch.float32)
    b.workspace_elems = workspace.numel()
    g = dict(dq=torch.empty_like(q), dk=torch.empty_like(q), dv=torch.empty_like(q),
             dkb=torch.empty((n_chunks, H, hd), dtype=act, device=q.device),
             dvb=torch.empty((n_chunks, H, hd), dtype=act, device=q.device))
    for name, t in g.items():
        setattr(b, name, t.data_ptr())
    _check(lib().attamba_chunk_attn_bwd(C.byref(b), _stream(stream)))
    return g


class DecodeCache:
    """Decode state of a batch: boundary-state cache [B, H, cap, hd], window [B, H, L, hd],
    SSM states [B, d, N], parameters, workspace, and the host mirrors pos / n_bound."""

    def __init__(self, B, H, hd, N, P, L, layer_idx, cap, dtype, params: dict, device="cuda",
                 pos: int = 0, n_bound: int = 0):
        d = H * hd
        self.kb = torch.zeros((B, H, cap, hd), dtype=dtype, device=device)
        self.vb = torch.zeros((B, H, cap, hd), dtype=dtype, device=device)
        self.kw = torch.zeros((B, H, max(L, 1), hd), dtype=dtype, device=device)
        self.vw = torch.zeros((B, H, max(L, 1), hd), dtype=dtype, device=device)
        self.h_k = torch.zeros((B, d, N), dtype=torch.float32, device=device)
        self.h_v = torch.zeros((B, d, N), dtype=torch.float32, device=device)
        self.params = {k: params[k].to(device=device, dtype=torch.float32).contiguous()
                       for k in ("A_k", "A_v", "D_k", "D_v", "bias_k", "bias_v")}
        s = DecodeCacheStruct()
        s.B, s.H, s.hd, s.d, s.N, s.P, s.L, s.layer_idx, s.cap = B, H, hd, d, N, P, L, layer_idx, cap
        s.dtype = FP32 if dtype == torch.float32 else BF16
        s.pos, s.n_bound = pos, n_bound
        nbytes = C.c_size_t()
        _check(lib().attamba_decode_workspace_size(C.byref(s), C.byref(nbytes)))
        self.workspace = torch.empty(max(nbytes.value // 4, 1), dtype=torch.float32,
                                     device=device)
        s.kb, s.vb = self.kb.data_ptr(), self.vb.data_ptr()
        s.kw, s.vw = self.kw.data_ptr(), self.vw.data_ptr()
        s.h_k, s.h_v = self.h_k.data_ptr(), self.h_v.data_ptr()
        for k, t in self.params.items():
            setattr(s, k, t.data_ptr())
        s.workspace, s.workspace_bytes = self.workspace.data_ptr(), self.workspace.numel() * 4
        self.struct = s
        self.dtype = dtype
        self.B, self.H, self.hd, self.d, self.N = B, H, hd, d, N

    @property
    def pos(self) -> int:
        return self.struct.pos

    @property
    def n_bound(self) -> int:
        return self.struct.n_bound

    def set_position(self, pos: int, n_bound: int) -> None:
        self.struct.pos, self.struct.n_bound = pos, n_bound

    def load_prefix(self, seq_cu_host, seq_cu, token_chunk, y_k, y_v, kb, vb, h_last_k, h_last_v,
                    stream=None) -> None:
        """Fill the cache from a prefill of B sequences of equal length n0 (uniform chunking
        with this cache's P and layer index; the scan run with h_last): completed boundary
        states, the last L per-token keys/values and the SSM states. Sets pos = n0."""
        seq_h = _host_i32(seq_cu_host)
        S = len(seq_h) - 1
        d, N = self.d, self.N
        T = int(seq_h[-1])
        pf = DecodePrefixStruct()
        pf.S, pf.n0 = S, int(seq_h[1] - seq_h[0]) if S > 0 else 0
        pf.seq_cu_host = seq_h.ctypes.data_as(_i32p)
        pf.seq_cu = _dev(seq_cu, "seq_cu", torch.int32, S + 1)
        pf.token_chunk = _dev(token_chunk, "token_chunk", torch.int32, T)
        pf.y_k = _dev(y_k, "y_k", self.dtype, T * d)
        pf.y_v = _dev(y_v, "y_v", self.dtype, T * d)
        pf.kb = _dev(kb, "kb", self.dtype)
        pf.vb = _dev(vb, "vb", self.dtype)
        pf.h_last_k = _dev(h_last_k, "h_last_k", torch.float32, S * d * N)
        pf.h_last_v = _dev(h_last_v, "h_last_v", torch.float32, S * d * N)
        _check(lib().attamba_decode_load_prefix(C.byref(self.struct), C.byref(pf), _stream(stream)))


def decode_step(cache: DecodeCache, q, x, dt_k, dt_v, bm_k, cm_k, bm_v, cm_v, out=None,
                stream=None, noalloc: bool = False):
    """One generated token for every sequence. q: [B, H, hd]; x, dt_*: [B, d]; bm/cm: [B, N].
    noalloc: call attamba_decode_step_noalloc, whose scratch is the library's static device
    array (the cache's workspace is not used); out must then be given."""
    B, d, N, act = cache.B, cache.d, cache.N, cache.dtype
    if out is None:
        if noalloc:
            raise ValueError("decode_step(noalloc=True) needs a preallocated out")
        out = torch.empty((B, cache.H, cache.hd), dtype=act, device=q.device)
    i = DecodeInputsStruct()
    i.q = _dev(q, "q", act, B * d)
    i.x = _dev(x, "x", act, B * d)
    i.dt_k = _dev(dt_k, "dt_k", act, B * d)
    i.dt_v = _dev(dt_v, "dt_v", act, B * d)
    i.bm_k = _dev(bm_k, "bm_k", act, B * N)
    i.cm_k = _dev(cm_k, "cm_k", act, B * N)
    i.bm_v = _dev(bm_v, "bm_v", act, B * N)
    i.cm_v = _dev(cm_v, "cm_v", act, B * N)
    i.out = _dev(out, "out", act, B * d)
    fn = lib().attamba_decode_step_noalloc if noalloc else lib().attamba_decode_step
    _check(fn(C.byref(cache.struct), C.byref(i), _stream(stream)))
    return out
