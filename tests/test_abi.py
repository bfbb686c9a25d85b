"""The C ABI library loads, exports every entry point declared in include/attamba.h, and its
host-side checks return the documented status codes before anything is launched (no GPU
needed: every call below fails validation or is host-only)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import ssm_compressed_chunked_amd as att
from ssm_compressed_chunked_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attamba.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attamba_[a-z_0-9]+)\s*\(", text)))


def test_header_and_exports_agree():
    names = declared_functions()
    assert len(names) == 17, names
    assert set(names) == set(B.EXPORTS), (set(names) ^ set(B.EXPORTS))
    lib = att.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {att.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_version_and_status_strings():
    assert att.version().startswith("attamba-mi355x")
    lib = att.lib()
    assert lib.attamba_status_string(0) == b"ok"
    assert lib.attamba_status_string(4) == b"capacity exceeded"
    assert lib.attamba_status_string(99) == b"unknown status"


def test_count_chunks_closed_form_and_errors():
    assert att.count_chunks([0, 256], 4, 0) == 64
    assert att.count_chunks([0, 2048, 4096, 6144, 8192], 8, 3) == 4 * 257
    assert att.count_chunks([0, 5, 5, 17, 18], 4, 1) == 2 + 0 + 4 + 1
    for bad in ([1, 5], [0, 5, 3]):
        with pytest.raises(att.AttambaError) as e:
            att.count_chunks(bad, 4, 0)
        assert e.value.status == B.ERR_BAD_SHAPE
    with pytest.raises(att.AttambaError):
        att.count_chunks([0, 5], 0, 0)


def test_chunk_cu_from_lengths():
    np.testing.assert_array_equal(att.chunk_cu_from_lengths([0, 5, 9], [2, 3, 4]), [0, 2, 5, 9])
    np.testing.assert_array_equal(att.chunk_cu_from_lengths([0, 0, 3], [3]), [0, 3])
    for lens in ([2, 4, 3], [2, 3], [2, 3, 4, 1], [0, 5, 4]):
        with pytest.raises(att.AttambaError) as e:
            att.chunk_cu_from_lengths([0, 5, 9], lens)
        assert e.value.status == B.ERR_BAD_SHAPE


def test_device_entry_points_validate_before_launch():
    lib = att.lib()
    assert lib.attamba_kvssm_scan(None, None) == B.ERR_NULL_ARG
    a = B.ScanArgs()
    a.T, a.d, a.N, a.dtype, a.n_chunks = 16, 64, 16, 7, 4
    assert lib.attamba_kvssm_scan(C.byref(a), None) == B.ERR_BAD_DTYPE
    a.dtype = B.BF16
    a.d = 96
    assert lib.attamba_kvssm_scan(C.byref(a), None) == B.ERR_BAD_SHAPE
    a.d, a.N = 64, 8
    assert lib.attamba_kvssm_scan(C.byref(a), None) == B.ERR_UNSUPPORTED
    a.N = 16
    assert lib.attamba_kvssm_scan(C.byref(a), None) == B.ERR_NULL_ARG
    assert b"required pointer" in lib.attamba_last_error()

    t = B.AttnArgs()
    t.T, t.H, t.hd, t.dtype, t.S, t.max_seqlen, t.n_chunks, t.L, t.mode = 8, 2, 48, 1, 1, 8, 2, 0, 1
    assert lib.attamba_chunk_attn_fwd(C.byref(t), None) == B.ERR_UNSUPPORTED
    t.hd, t.mode = 64, 5
    assert lib.attamba_chunk_attn_fwd(C.byref(t), None) == B.ERR_BAD_SHAPE
    t.mode, t.L = 1, -1
    assert lib.attamba_chunk_attn_fwd(C.byref(t), None) == B.ERR_BAD_SHAPE
    t.L = 0
    assert lib.attamba_chunk_attn_fwd(C.byref(t), None) == B.ERR_NULL_ARG

    assert lib.attamba_chunk_boundaries(None, 1, 4, 4, 0, 1, None, None, None, None) == B.ERR_NULL_ARG
    assert lib.attamba_chunk_index(None, 1, 4, None, None, None) == B.ERR_NULL_ARG

    c = B.DecodeCacheStruct()
    c.B, c.H, c.hd, c.d, c.N, c.P, c.L, c.cap, c.dtype = 1, 2, 64, 128, 16, 4, 8, 4, 1
    n = C.c_size_t()
    assert lib.attamba_decode_workspace_size(C.byref(c), C.byref(n)) == 0 and n.value > 0
    i = B.DecodeInputsStruct()
    assert lib.attamba_decode_step(C.byref(c), C.byref(i), None) == B.ERR_NULL_ARG
    c.d = 100
    assert lib.attamba_decode_step(C.byref(c), C.byref(i), None) == B.ERR_BAD_SHAPE
    c.d, c.hd, c.H = 96, 48, 2
    assert lib.attamba_decode_step(C.byref(c), C.byref(i), None) == B.ERR_UNSUPPORTED
    # the variant with the library's static scratch checks its pointers before anything else
    assert lib.attamba_decode_step_noalloc(None, C.byref(i), None) == B.ERR_NULL_ARG
    assert lib.attamba_decode_step_noalloc(C.byref(c), None, None) == B.ERR_NULL_ARG


def test_decode_noalloc_rejects_steps_beyond_its_scratch():
    """attamba_decode_step_noalloc fails with CAPACITY, on the host and before looking up or
    touching any device memory, when the step's split partials (4 B H (hd + 2) (ceil((cap + L) /
    256) + 1) bytes) exceed ATTAMBA_DECODE_SCRATCH_BYTES; the pointers are never dereferenced."""
    lib = att.lib()
    c = B.DecodeCacheStruct()
    c.B, c.H, c.hd, c.d, c.N, c.P, c.L, c.layer_idx, c.dtype = 64, 32, 128, 4096, 16, 4, 256, 0, 1
    c.pos, c.n_bound = 32768, 8192
    c.cap = 8192 + 4
    for f in ("kb", "vb", "kw", "vw", "h_k", "h_v", "A_k", "A_v", "D_k", "D_v", "bias_k", "bias_v"):
        setattr(c, f, 4096)           # placeholders: the size check fails first
    i = B.DecodeInputsStruct()
    for f in ("q", "x", "dt_k", "dt_v", "bm_k", "cm_k", "bm_v", "cm_v", "out"):
        setattr(i, f, 4096)
    need = 4 * c.B * c.H * (c.hd + 2) * (-(-(c.cap + c.L) // 256) + 1)
    assert need > B.DECODE_SCRATCH_BYTES
    assert lib.attamba_decode_step_noalloc(C.byref(c), C.byref(i), None) == B.ERR_CAPACITY
    assert b"scratch" in lib.attamba_last_error()
    assert c.pos == 32768 and c.n_bound == 8192     # unchanged on error


def test_input_proj_validates_before_launch():
    lib = att.lib()
    assert lib.attamba_input_proj(None, None) == B.ERR_NULL_ARG
    a = B.ProjArgs()
    a.T, a.d, a.n_out, a.dtype, a.n_seg = 16, 128, 24, 5, 2
    assert lib.attamba_input_proj(C.byref(a), None) == B.ERR_BAD_DTYPE
    a.dtype = B.FP32
    assert lib.attamba_input_proj(C.byref(a), None) == B.ERR_UNSUPPORTED
    a.dtype = B.BF16
    a.seg_start[0], a.seg_start[1], a.seg_start[2] = 0, 16, 24
    a.d = 96
    assert lib.attamba_input_proj(C.byref(a), None) == B.ERR_BAD_SHAPE      # d not a multiple of 64
    a.d = 128
    a.seg_start[1] = 18
    assert lib.attamba_input_proj(C.byref(a), None) == B.ERR_BAD_SHAPE      # start not 4-aligned
    a.seg_start[1] = 16
    a.seg_start[2] = 20
    assert lib.attamba_input_proj(C.byref(a), None) == B.ERR_BAD_SHAPE      # does not reach n_out
    a.n_out = a.seg_start[2] = 22
    assert lib.attamba_input_proj(C.byref(a), None) == B.ERR_BAD_SHAPE      # end not 4-aligned
    a.n_out = a.seg_start[2] = 24
    a.n_seg = B.PROJ_MAX_SEGMENTS + 1
    assert lib.attamba_input_proj(C.byref(a), None) == B.ERR_BAD_SHAPE      # too many segments
    a.n_seg = 2
    assert lib.attamba_input_proj(C.byref(a), None) == B.ERR_NULL_ARG       # x, w, out null
    a.T = 1 << 24
    assert lib.attamba_input_proj(C.byref(a), None) == B.ERR_UNSUPPORTED    # T*d >= 2^31


def test_backward_entry_points_validate_before_launch():
    lib = att.lib()
    assert lib.attamba_chunk_attn_bwd(None, None) == B.ERR_NULL_ARG
    assert lib.attamba_kvssm_scan_bwd(None, None) == B.ERR_NULL_ARG
    fake = C.c_void_p(0x1000)          # never dereferenced: validation fails before any launch
    b = B.AttnBwdArgs()
    f = b.fwd
    f.T, f.H, f.hd, f.dtype, f.S, f.max_seqlen, f.n_chunks, f.L, f.mode = 64, 2, 64, 1, 1, 64, 8, 0, 0
    for name in ("q", "k", "v", "kb", "vb", "seq_cu", "chunk_cu", "token_chunk", "out"):
        setattr(f, name, fake)
    assert lib.attamba_chunk_attn_bwd(C.byref(b), None) == B.ERR_NULL_ARG   # lse, dout, grads
    f.hd = 48
    assert lib.attamba_chunk_attn_bwd(C.byref(b), None) == B.ERR_UNSUPPORTED
    f.hd, f.mode = 64, 7
    assert lib.attamba_chunk_attn_bwd(C.byref(b), None) == B.ERR_BAD_SHAPE
    f.mode, f.dtype = 0, 9
    assert lib.attamba_chunk_attn_bwd(C.byref(b), None) == B.ERR_BAD_DTYPE
    # workspace: size query, then a workspace below it (CAPACITY) or misaligned (BAD_SHAPE)
    f.dtype = 1
    f.lse = fake
    for name in ("dout", "dq", "dk", "dv", "dkb", "dvb", "workspace"):
        setattr(b, name, fake)
    need = C.c_size_t(0)
    assert lib.attamba_chunk_attn_bwd_workspace_size(C.byref(b), C.byref(need)) == 0
    # 64 tokens, 8 chunks, 2 heads x 64 (bf16): (H + 2) T rounded up to 64, plus 8 n_chunks H hd
    assert need.value == 256 + 8 * 8 * 2 * 64
    b.workspace_elems = need.value - 1
    assert lib.attamba_chunk_attn_bwd(C.byref(b), None) == B.ERR_CAPACITY
    b.workspace_elems = need.value
    b.workspace = C.c_void_p(0x1004)
    assert lib.attamba_chunk_attn_bwd(C.byref(b), None) == B.ERR_BAD_SHAPE
    f.n_chunks = 64                    # one token per chunk: no split, no partial sums
    assert lib.attamba_chunk_attn_bwd_workspace_size(C.byref(b), C.byref(need)) == 0
    assert need.value == (2 + 2) * 64
    f.dtype = 0                        # float32 takes the row-wise kernels
    f.n_chunks = 8
    assert lib.attamba_chunk_attn_bwd_workspace_size(C.byref(b), C.byref(need)) == 0
    assert need.value == (2 + 2) * 64
    assert lib.attamba_chunk_attn_bwd_workspace_size(None, C.byref(need)) == B.ERR_NULL_ARG

    s = B.ScanBwdArgs()
    a = s.fwd
    a.T, a.d, a.N, a.dtype, a.n_chunks = 64, 128, 16, 1, 8
    for name in ("chunk_cu", "x", "dt_k", "dt_v", "bm_k", "cm_k", "bm_v", "cm_v", "A_k", "A_v",
                 "D_k", "D_v", "bias_k", "bias_v"):
        setattr(a, name, fake)
    assert lib.attamba_kvssm_scan_bwd(C.byref(s), None) == B.ERR_NULL_ARG   # gradients null
    a.N = 8
    assert lib.attamba_kvssm_scan_bwd(C.byref(s), None) == B.ERR_UNSUPPORTED
    a.N, a.d = 16, 96
    assert lib.attamba_kvssm_scan_bwd(C.byref(s), None) == B.ERR_BAD_SHAPE
    a.d = 128
    for name in ("gy_k", "gy_v", "dx_k", "dx_v", "ddt_k", "ddt_v", "dbm_k", "dcm_k", "dbm_v",
                 "dcm_v", "dA_k", "dA_v", "dD_k", "dD_v", "dbias_k", "dbias_v"):
        setattr(s, name, fake)
    s.gkb = fake
    assert lib.attamba_kvssm_scan_bwd(C.byref(s), None) == B.ERR_NULL_ARG   # gkb without gvb
    s.gkb = None
    a.bm_v = C.c_void_p(0x1008)
    assert lib.attamba_kvssm_scan_bwd(C.byref(s), None) == B.ERR_BAD_SHAPE  # misaligned Bm


def test_decode_load_prefix_validates_before_launch():
    import numpy as np
    lib = att.lib()
    assert lib.attamba_decode_load_prefix(None, None, None) == B.ERR_NULL_ARG
    fake = C.c_void_p(0x1000)          # never dereferenced: validation fails before any launch
    c = B.DecodeCacheStruct()
    c.B, c.H, c.hd, c.d, c.N, c.P, c.L, c.layer_idx, c.cap, c.dtype = 2, 2, 64, 128, 16, 4, 3, 1, 2, 1
    for name in ("kb", "vb", "kw", "vw", "h_k", "h_v"):
        setattr(c, name, fake)
    pf = B.DecodePrefixStruct()
    seq = np.array([0, 10, 20], dtype=np.int32)
    pf.S, pf.n0, pf.seq_cu_host = 2, 10, seq.ctypes.data_as(C.POINTER(C.c_int32))
    for name in ("seq_cu", "token_chunk", "y_k", "y_v", "kb", "vb", "h_last_k", "h_last_v"):
        setattr(pf, name, fake)
    assert lib.attamba_decode_load_prefix(C.byref(c), C.byref(pf), None) == B.ERR_CAPACITY  # 3 ends > cap 2
    c.cap = 8
    pf.S = 3
    assert lib.attamba_decode_load_prefix(C.byref(c), C.byref(pf), None) == B.ERR_BAD_SHAPE  # S != B
    pf.S = 2
    seq[2] = 19
    assert lib.attamba_decode_load_prefix(C.byref(c), C.byref(pf), None) == B.ERR_BAD_SHAPE  # ragged
    seq[2] = 20
    pf.h_last_v = None
    assert lib.attamba_decode_load_prefix(C.byref(c), C.byref(pf), None) == B.ERR_NULL_ARG
    pf.h_last_v = fake
    c.hd, c.d = 48, 96
    assert lib.attamba_decode_load_prefix(C.byref(c), C.byref(pf), None) == B.ERR_UNSUPPORTED


def test_decode_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTAMBA_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m, "ATTAMBA_DECODE_SCRATCH_BYTES not found"
    assert int(m.group(1)) << int(m.group(2)) == B.DECODE_SCRATCH_BYTES
