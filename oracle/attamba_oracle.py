"""Plain, slow CPU oracle of Attamba's KV-SSM forward, chunk-aware attention and decode, and
the reverse-mode gradients of the scan and of the attention (training with M_train).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link this module:
only the tests, the smoke check and the CPU-baseline leg of the benchmark use it. It shares
no code with the HIP path; both take their inputs from the seeded generators in
`workloads/`, which hold none of the method's arithmetic.

Everything is float64 NumPy, computed in the plainest order: a sequential recurrence over
tokens, an explicit dense boolean mask, and a naive (max-subtracted) softmax. Page
references are to "Attamba: Attending To Multi-Token States" (arXiv 2411.17685) as
summarised on pith.science ("What carries the argument", "Core claim", "If this is
right", the Referee Report, "Assumptions & free parameters") and on rohan-paul.com
("Solution in this Paper", "Key Insights").

Readings taken where the pages are silent (each is listed with its reason in the design
notes of the repository):
  * SSM (the paper's Eq. 3, not printed on the pages; Mamba-style selective scan):
    h_t = exp(delta_t * A) * h_{t-1} + delta_t * x_t * Bm_t,  y_t = Cm_t . h_t + D * x_t,
    per channel c with state size N, A[c, :] < 0, delta = softplus(dt + bias).
  * The state is zero at every chunk start (each chunk is compressed on its own); the
    boundary state of a chunk is the SSM output y at its last token.
  * Cyclic offset o = layer_idx mod P: chunk starts are the sequence start and every local
    position t with t = o (mod P); a trailing partial chunk is a chunk.
  * Mask: a key position j is visible from query i (same sequence) iff j <= i and
    (j ends a chunk, or (M_train and j is in i's chunk), or i - j < L). This is the causal
    reading of M_test: the current chunk's boundary is visible only once it is complete.
  * A query row with no visible key gives O = 0 and LSE = -inf.
  * Backward: the gradients are those of the forward above, by the chain rule (reverse mode);
    they are pinned against central finite differences of this module's forward.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

TRAIN, TEST = "train", "test"


# ----------------------------------------------------------------------------------------
# Input projections: queries and the SSMs' per-token inputs dt, Bm, Cm are linear maps of the
# layer input (pith.science "Core claim": the SSMs replace the key and value projections; the
# selective SSM's inputs, the paper's Eq. 3, cited in "Assumptions & free parameters").
# ----------------------------------------------------------------------------------------
def linear(x, w):
    """y[t, f] = sum_k x[t, k] * w[f, k]: x [T, d], w [n_out, d] (one row per output
    feature). Returns float64 [T, n_out]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    return x @ w.T


# ----------------------------------------------------------------------------------------
# Segmentation: uniform chunks of P tokens with a cyclic offset per layer (pith.science
# "What carries the argument": cyclic chunking shifts the chunk offset by layer index;
# "Assumptions & free parameters": offset = layer index), or variable-length chunks given
# as lengths, i.e. chunk cu_seqlens ("If this is right": boundaries via cu_seqlens).
# ----------------------------------------------------------------------------------------
def uniform_chunk_starts(n: int, P: int, layer_idx: int) -> list[int]:
    """Local start positions of the chunks of one sequence of n tokens."""
    if P < 1:
        raise ValueError("P must be >= 1")
    o = layer_idx % P
    return [t for t in range(n) if t == 0 or (t - o) % P == 0]


def segment(seq_cu, P: int | None = None, layer_idx: int = 0, chunk_lens=None):
    """Chunk layout of a packed batch.

    seq_cu: sequence offsets [S+1]. Either uniform chunking (P, layer_idx) or explicit
    chunk lengths (concatenated per sequence, each >= 1, summing to each sequence length).
    Returns chunk_cu [n_chunks+1], token_chunk [T] (chunk of each token), is_end [T] (1 at the
    last token of every chunk).
    """
    seq_cu = [int(v) for v in seq_cu]
    T = seq_cu[-1]
    starts: list[int] = []
    if chunk_lens is None:
        for s in range(len(seq_cu) - 1):
            a, b = seq_cu[s], seq_cu[s + 1]
            if b < a:
                raise ValueError("seq_cu must be non-decreasing")
            starts += [a + t for t in uniform_chunk_starts(b - a, P, layer_idx)]
    else:
        lens = [int(v) for v in chunk_lens]
        k = 0
        for s in range(len(seq_cu) - 1):
            pos, end = seq_cu[s], seq_cu[s + 1]
            while pos < end:
                if k >= len(lens) or lens[k] < 1 or pos + lens[k] > end:
                    raise ValueError("chunk lengths do not tile the sequences")
                starts.append(pos)
                pos += lens[k]
                k += 1
        if k != len(lens):
            raise ValueError("more chunk lengths than tokens")
    chunk_cu = np.array(starts + [T], dtype=np.int64)
    token_chunk = np.empty(T, dtype=np.int64)
    is_end = np.zeros(T, dtype=np.uint8)
    for q in range(len(starts)):
        token_chunk[chunk_cu[q]:chunk_cu[q + 1]] = q
        is_end[chunk_cu[q + 1] - 1] = 1
    return chunk_cu, token_chunk, is_end


# ----------------------------------------------------------------------------------------
# KV-SSM: two selective scans replace W_K and W_V (pith.science "Core claim": K^(p) =
# SSM_K(X^(p)), V^(p) = SSM_V(X^(p)) per chunk; rohan-paul.com "Solution in this Paper").
# ----------------------------------------------------------------------------------------
def softplus(z):
    """log(1 + exp(z)), exactly (no threshold)."""
    return np.logaddexp(0.0, z)


def selective_scan(x, dt, dt_bias, A, Bm, Cm, D, chunk_cu, t_begin: int = 0,
                   t_end: int | None = None, snapshot_after=()):
    """Sequential selective scan over tokens [t_begin, t_end).

    x, dt: [T, d]; dt_bias, D: [d]; A: [d, N]; Bm, Cm: [T, N]; chunk_cu: chunk offsets.
    t_begin must be a chunk start. Returns y [t_end - t_begin, d] and a dict
    {t: state [d, N] after token t} for t in snapshot_after.
    """
    x = np.asarray(x, np.float64)
    T, d = x.shape
    t_end = T if t_end is None else t_end
    starts = set(int(v) for v in chunk_cu[:-1])
    if t_begin < t_end and t_begin not in starts:
        raise ValueError("t_begin must be a chunk start")
    delta = softplus(np.asarray(dt, np.float64)[t_begin:t_end] + np.asarray(dt_bias, np.float64))
    A = np.asarray(A, np.float64)
    D = np.asarray(D, np.float64)
    y = np.empty((t_end - t_begin, d))
    h = np.zeros_like(A)
    snaps = {}
    for t in range(t_begin, t_end):
        if t in starts:
            h = np.zeros_like(A)
        k = t - t_begin
        decay = np.exp(delta[k][:, None] * A)                       # [d, N]
        inject = (delta[k] * x[t])[:, None] * np.asarray(Bm[t], np.float64)[None, :]
        h = decay * h + inject
        y[k] = h @ np.asarray(Cm[t], np.float64) + D * x[t]
        if t in snapshot_after:
            snaps[t] = h.copy()
    return y, snaps


def selective_scan_backward(x, dt, dt_bias, A, Bm, Cm, D, chunk_cu, gy):
    """Gradients of sum(gy * y) for y = selective_scan(x, dt, dt_bias, A, Bm, Cm, D, chunk_cu)
    over all tokens: reverse mode of the recurrence, token by token backwards within each chunk
    (the state restarts at every chunk start, so no gradient crosses a chunk start).

    Returns dict(dx [T, d], ddt [T, d], dbias [d], dA [d, N], dBm [T, N], dCm [T, N], dD [d]).
    """
    x = np.asarray(x, np.float64)
    T, d = x.shape
    A = np.asarray(A, np.float64)
    D = np.asarray(D, np.float64)
    Bm = np.asarray(Bm, np.float64)
    Cm = np.asarray(Cm, np.float64)
    gy = np.asarray(gy, np.float64)
    z = np.asarray(dt, np.float64) + np.asarray(dt_bias, np.float64)
    delta = softplus(z)
    sig = 1.0 / (1.0 + np.exp(-z))             # derivative of softplus
    starts = set(int(v) for v in chunk_cu[:-1])
    # forward, keeping every state
    hs = np.zeros((T, d, A.shape[1]))
    h = np.zeros_like(A)
    for t in range(T):
        if t in starts:
            h = np.zeros_like(A)
        h = np.exp(delta[t][:, None] * A) * h + (delta[t] * x[t])[:, None] * Bm[t][None, :]
        hs[t] = h
    g = dict(dx=np.zeros((T, d)), ddt=np.zeros((T, d)), dbias=np.zeros(d),
             dA=np.zeros_like(A), dBm=np.zeros_like(Bm), dCm=np.zeros_like(Cm), dD=np.zeros(d))
    cu = [int(v) for v in chunk_cu]
    for a, b in zip(cu[:-1], cu[1:]):
        dh = np.zeros_like(A)                  # gradient with respect to the state after t
        for t in range(b - 1, a - 1, -1):
            # y_t = Cm_t . h_t + D x_t
            g["dD"] += gy[t] * x[t]
            g["dx"][t] += gy[t] * D
            g["dCm"][t] += gy[t] @ hs[t]
            dh = dh + gy[t][:, None] * Cm[t][None, :]
            # h_t = exp(delta_t A) h_{t-1} + (delta_t x_t) Bm_t
            e = np.exp(delta[t][:, None] * A)
            u = delta[t] * x[t]
            hprev = hs[t - 1] if t > a else np.zeros_like(A)
            g["dBm"][t] += (dh * u[:, None]).sum(axis=0)
            du = (dh * Bm[t][None, :]).sum(axis=1)
            de = dh * hprev
            ddelta = du * x[t] + (de * e * A).sum(axis=1)
            g["dx"][t] += du * delta[t]
            g["dA"] += de * e * delta[t][:, None]
            dz = ddelta * sig[t]
            g["ddt"][t] += dz
            g["dbias"] += dz
            dh = dh * e
    return g


# ----------------------------------------------------------------------------------------
# Mamba-block variant of the KV-SSM. The selective SSM is the core of a Mamba block
# (pith.science "Assumptions & free parameters": selective state-space models, Mamba, Section
# 3.2, Eq. 3). Around the scan, a Mamba block puts a short causal depthwise convolution followed
# by SiLU on the scan's input, and multiplies the scan's output by SiLU of a second projection
# of the layer input (the gate). The block runs on each chunk on its own ("Core claim": K^(p) =
# SSM_K(X^(p)) per chunk), so the convolution restarts at every chunk start, as the state does:
# positions before the chunk start count as zero.
# ----------------------------------------------------------------------------------------
def silu(v):
    """SiLU: v * sigmoid(v) = v / (1 + exp(-v))."""
    v = np.asarray(v, np.float64)
    return v / (1.0 + np.exp(-v))


def chunk_causal_conv(x, w, b, chunk_cu):
    """Depthwise causal convolution that restarts at every chunk:
    out[t, c] = b[c] + sum_k w[c, k] * x[t - (K - 1) + k, c], where positions before the start
    of t's chunk count as zero. x: [T, d]; w: [d, K] (tap K - 1 multiplies the current token);
    b: [d]. Returns float64 [T, d]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    b = np.asarray(b, np.float64)
    T, d = x.shape
    K = w.shape[1]
    out = np.empty((T, d))
    cu = [int(v) for v in chunk_cu]
    for a, e in zip(cu[:-1], cu[1:]):
        for t in range(a, e):
            acc = b.copy()
            for k in range(K):
                s = t - (K - 1) + k
                if s >= a:
                    acc = acc + w[:, k] * x[s]
            out[t] = acc
    return out


def ssm_block_scan(x, dt, dt_bias, A, Bm, Cm, D, chunk_cu, conv_w=None, conv_b=None, z=None):
    """The scan of one SSM inside a Mamba block, chunk by chunk: xc = silu(conv(x)) when conv_w
    is given (else xc = x); y = selective_scan(xc, ...), whose skip term D * xc uses the scan's
    own input; out = y * silu(z) when the gate input z [T, d] is given (else out = y).
    Returns out [T, d]; its value at a chunk's last token is the chunk's boundary state."""
    xc = x if conv_w is None else silu(chunk_causal_conv(x, conv_w, conv_b, chunk_cu))
    y, _ = selective_scan(xc, dt, dt_bias, A, Bm, Cm, D, chunk_cu)
    return y if z is None else y * silu(z)


def boundary_states(y, chunk_cu):
    """One state per chunk: the SSM output y at the chunk's last token (pith.science review,
    Referee Report, comment on Eq. 7: the boundary state K^(p)[-1] is the output once the
    whole chunk has been processed)."""
    return y[np.asarray(chunk_cu[1:], dtype=np.int64) - 1]


# ----------------------------------------------------------------------------------------
# Chunk-aware causal mask (M_train, Eq. 5; M_test, Eq. 7; leading-token window, Eq. 8 of the
# paper, described in pith.science "What carries the argument" and the Referee Report's
# second major comment).
# ----------------------------------------------------------------------------------------
def dense_mask(token_chunk, is_end, L: int, mode: str, rows=None):
    """Boolean mask [len(rows), n] of one sequence (local indices).

    token_chunk, is_end: per-token chunk id and chunk-end flag of the sequence.
    """
    tc = np.asarray(token_chunk)
    ie = np.asarray(is_end).astype(bool)
    n = len(tc)
    i = np.arange(n)[:, None] if rows is None else np.asarray(rows)[:, None]
    j = np.arange(n)[None, :]
    visible = ie[j] | ((i - j) < L)
    if mode == TRAIN:
        visible = visible | (tc[j] == tc[i])
    elif mode != TEST:
        raise ValueError(mode)
    return (j <= i) & visible


def masked_attention(q, k, v, mask, scale: float):
    """Naive softmax attention of one sequence, all heads.

    q: [m, H, hd] (query rows), k, v: [n, H, hd], mask: [m, n] bool.
    Returns O [m, H, hd] and LSE [H, m] (natural log; -inf for a row with no key).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    m_rows, H, hd = q.shape
    out = np.zeros((m_rows, H, hd))
    lse = np.full((H, m_rows), -np.inf)
    live = mask.any(axis=1)
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        s = np.where(mask, s, -np.inf)
        mx = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
        p = np.exp(s - mx[:, None])
        denom = p.sum(axis=1)
        out[live, h, :] = (p[live] @ v[:, h, :]) / denom[live, None]
        lse[h, live] = mx[live] + np.log(denom[live])
    return out, lse


def masked_attention_backward(q, k, v, mask, scale: float, dout):
    """Gradients of sum(dout * O) for O = masked_attention(q, k, v, mask, scale): the softmax
    rows, dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dP P)), dQ = scale dS K,
    dK = scale dS^T Q. Rows with no visible key pass no gradient. Returns dq, dk, dv."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    live = mask.any(axis=1)
    for h in range(q.shape[1]):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        s = np.where(mask, s, -np.inf)
        mx = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
        p = np.exp(s - mx[:, None])
        p[live] /= p[live].sum(axis=1, keepdims=True)
        dv[:, h, :] = p.T @ dout[:, h, :]
        dp = dout[:, h, :] @ v[:, h, :].T
        ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
        dq[:, h, :] = scale * (ds @ k[:, h, :])
        dk[:, h, :] = scale * (ds.T @ q[:, h, :])
    return dq, dk, dv


def chunk_attention_backward(q, k, v, seq_cu, token_chunk, is_end, L: int, mode: str, dout,
                             scale: float | None = None):
    """Gradients of sum(dout * O) for O = chunk_attention(...) over a packed batch: dq, dk, dv
    [T, H, hd]. dk and dv are the total gradients of the per-token keys and values, through
    their use as window keys and as boundary states alike (one position, one key)."""
    T, H, hd = np.shape(q)
    scale = 1.0 / math.sqrt(hd) if scale is None else scale
    seq_cu = np.asarray(seq_cu, dtype=np.int64)
    dq = np.zeros((T, H, hd))
    dk = np.zeros((T, H, hd))
    dv = np.zeros((T, H, hd))
    for b in range(len(seq_cu) - 1):
        s0, s1 = int(seq_cu[b]), int(seq_cu[b + 1])
        if s1 <= s0:
            continue
        mask = dense_mask(np.asarray(token_chunk)[s0:s1], np.asarray(is_end)[s0:s1], L, mode)
        a, bk, c = masked_attention_backward(q[s0:s1], k[s0:s1], v[s0:s1], mask, scale,
                                             dout[s0:s1])
        dq[s0:s1], dk[s0:s1], dv[s0:s1] = a, bk, c
    return dq, dk, dv


def chunk_attention(q, k, v, seq_cu, token_chunk, is_end, L: int, mode: str,
                    scale: float | None = None, rows=None):
    """Attention of a packed batch over per-token K/V with the chunk mask.

    q, k, v: [T, H, hd]. rows: optional global query rows to evaluate (default all).
    Returns O [m, H, hd] and LSE [H, m] for the evaluated rows, in the order given.
    """
    T, H, hd = np.shape(q)
    scale = 1.0 / math.sqrt(hd) if scale is None else scale
    seq_cu = np.asarray(seq_cu, dtype=np.int64)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), H, hd))
    lse = np.full((H, len(rows)), -np.inf)
    seq_of = np.searchsorted(seq_cu, rows, side="right") - 1
    for s in np.unique(seq_of):
        a, b = int(seq_cu[s]), int(seq_cu[s + 1])
        sel = np.nonzero(seq_of == s)[0]
        local = rows[sel] - a
        mask = dense_mask(token_chunk[a:b], is_end[a:b], L, mode, rows=local)
        o, l_ = masked_attention(np.asarray(q)[rows[sel]], np.asarray(k)[a:b],
                                 np.asarray(v)[a:b], mask, scale)
        out[sel] = o
        lse[:, sel] = l_
    return out, lse


# ----------------------------------------------------------------------------------------
# The whole forward of one layer's attention block with KV-SSM (configs of the prefill).
# ----------------------------------------------------------------------------------------
def kvssm_forward(inp: dict, seq_cu, H: int, hd: int, P: int | None, layer_idx: int,
                  L: int, mode: str, chunk_lens=None, scale: float | None = None,
                  attn_rows=None):
    """inp: float64 arrays x, q, dt_k, dt_v, bm_k, cm_k, bm_v, cm_v, A_k, A_v, D_k, D_v,
    bias_k, bias_v. Returns a dict with chunk_cu, token_chunk, is_end, y_k, y_v, kb, vb,
    out, lse."""
    chunk_cu, token_chunk, is_end = segment(seq_cu, P, layer_idx, chunk_lens)
    y_k, _ = selective_scan(inp["x"], inp["dt_k"], inp["bias_k"], inp["A_k"], inp["bm_k"],
                            inp["cm_k"], inp["D_k"], chunk_cu)
    # SSM_V reads x, or its own input x_v (explicit key and value projections kept in front of
    # the SSMs, pith.science "If this is right")
    y_v, _ = selective_scan(inp.get("x_v", inp["x"]), inp["dt_v"], inp["bias_v"], inp["A_v"],
                            inp["bm_v"], inp["cm_v"], inp["D_v"], chunk_cu)
    T = y_k.shape[0]
    k3 = y_k.reshape(T, H, hd)
    v3 = y_v.reshape(T, H, hd)
    q3 = np.asarray(inp["q"], np.float64).reshape(T, H, hd)
    out, lse = chunk_attention(q3, k3, v3, seq_cu, token_chunk, is_end, L, mode, scale,
                               rows=attn_rows)
    return dict(chunk_cu=chunk_cu, token_chunk=token_chunk, is_end=is_end, y_k=y_k, y_v=y_v,
                kb=boundary_states(y_k, chunk_cu).reshape(-1, H, hd),
                vb=boundary_states(y_v, chunk_cu).reshape(-1, H, hd), out=out, lse=lse)


# ----------------------------------------------------------------------------------------
# A stack of layers (pith.science "What carries the argument": cyclic chunking shifts the chunk
# offset by layer index). Layer l uses layer index first_layer + l; its attention output is the
# next layer's input (the output projection, MLP and norms between attention layers are outside
# the path). The path stores what one call hands to the next in bf16, so the chain rounds the
# projections and each layer's output to bf16 (round to nearest, ties to even) where the next
# call reads them.
# ----------------------------------------------------------------------------------------
def round_to_bf16(a):
    """a rounded to the nearest bf16 value (8 significant bits), ties to even; float64 out."""
    a = np.asarray(a, np.float64)
    m, e = np.frexp(a)                   # a = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0), e - 8)


def stack_forward(x, layers, seq_cu, H: int, hd: int, N: int, P: int, L: int, mode: str,
                  first_layer: int = 0):
    """x [T, d] (layer 0's input); layers[l] = dict(w [3 d + 4 N, d], params) with params A_k,
    A_v, D_k, D_v, bias_k, bias_v. Returns the per-layer kvssm_forward results ("out" is
    [T, H, hd], before the bf16 rounding that feeds the next layer)."""
    x = np.asarray(x, np.float64)
    T, d = x.shape
    widths = [("q", d), ("dt_k", d), ("dt_v", d), ("bm_k", N), ("cm_k", N), ("bm_v", N), ("cm_v", N)]
    results = []
    for l, lay in enumerate(layers):
        proj = round_to_bf16(linear(x, lay["w"]))
        inp = {"x": x}
        start = 0
        for name, wd in widths:
            inp[name] = proj[:, start:start + wd]
            start += wd
        for k, v in lay["params"].items():
            inp[k] = np.asarray(v, np.float64)
        res = kvssm_forward(inp, seq_cu, H, hd, P, first_layer + l, L, mode)
        results.append(res)
        x = round_to_bf16(res["out"].reshape(T, d))
    return results


# ----------------------------------------------------------------------------------------
# Decode with a cache of boundary states plus the L most recent tokens (pith.science
# "Core claim": at inference only the boundary states are cached; "If this is right":
# KV-cache shrinks by about P; leading tokens stay uncompressed).
# ----------------------------------------------------------------------------------------
@dataclass
class DecodeSeq:
    """Decode state of one sequence: next position, SSM states, and the cached keys."""
    pos: int
    h_k: np.ndarray                  # [d, N]
    h_v: np.ndarray
    bounds: list = field(default_factory=list)   # (position, k_row [H, hd], v_row)
    recent: list = field(default_factory=list)   # (position, k_row, v_row), last L tokens


def is_chunk_start_at(pos: int, P: int, layer_idx: int) -> bool:
    return pos == 0 or (pos - layer_idx % P) % P == 0


def is_chunk_end_at(pos: int, P: int, layer_idx: int) -> bool:
    return is_chunk_start_at(pos + 1, P, layer_idx)


def decode_state_from_prefix(y_k, y_v, h_k, h_v, n0: int, H: int, hd: int, P: int,
                             layer_idx: int, L: int) -> DecodeSeq:
    """Cache of one sequence after its first n0 tokens were processed: the boundary states
    of the completed chunks, the last L per-token K/V rows, and the SSM states after token
    n0 - 1 (h_k, h_v; zeros if n0 starts a new chunk)."""
    st = DecodeSeq(pos=n0, h_k=np.array(h_k, np.float64), h_v=np.array(h_v, np.float64))
    for j in range(n0):
        row = (j, y_k[j].reshape(H, hd), y_v[j].reshape(H, hd))
        if is_chunk_end_at(j, P, layer_idx):
            st.bounds.append(row)
        if j >= n0 - L:
            st.recent.append(row)
    return st


def decode_step(st: DecodeSeq, par: dict, tok: dict, H: int, hd: int, P: int,
                layer_idx: int, L: int, scale: float | None = None):
    """One generated token for one sequence. par: A_k, A_v, D_k, D_v, bias_k, bias_v;
    tok: q [d], x, dt_k, dt_v [d], bm_k, cm_k, bm_v, cm_v [N]. Returns O [H, hd]."""
    scale = 1.0 / math.sqrt(hd) if scale is None else scale
    i = st.pos
    if is_chunk_start_at(i, P, layer_idx):
        st.h_k = np.zeros_like(st.h_k)
        st.h_v = np.zeros_like(st.h_v)
    ys = {}
    for s in ("k", "v"):
        h = getattr(st, f"h_{s}")
        delta = softplus(tok[f"dt_{s}"] + par[f"bias_{s}"])
        h = np.exp(delta[:, None] * par[f"A_{s}"]) * h \
            + (delta * tok["x"])[:, None] * tok[f"bm_{s}"][None, :]
        setattr(st, f"h_{s}", h)
        ys[s] = (h @ tok[f"cm_{s}"] + par[f"D_{s}"] * tok["x"]).reshape(H, hd)
    row = (i, ys["k"], ys["v"])
    st.recent.append(row)
    st.recent = [r for r in st.recent if r[0] > i - L]
    if is_chunk_end_at(i, P, layer_idx):
        st.bounds.append(row)
    w = max(0, i - L + 1)
    keys = [r for r in st.bounds if r[0] < w] + [r for r in st.recent if r[0] >= w]
    st.pos = i + 1
    q = np.asarray(tok["q"], np.float64).reshape(H, hd)
    if not keys:
        return np.zeros((H, hd))
    kk = np.stack([r[1] for r in keys], axis=0)        # [m, H, hd]
    vv = np.stack([r[2] for r in keys], axis=0)
    out = np.empty((H, hd))
    for h in range(H):
        s = (kk[:, h, :] @ q[h]) * scale
        p = np.exp(s - s.max())
        out[h] = (p @ vv[:, h, :]) / p.sum()
    return out
