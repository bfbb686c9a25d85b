"""GPU parity: every call of libattamba against the CPU oracle on the same seeded inputs.

Bars: chunk layout bit-exact; float32 outputs within 1e-4 relative (+1e-5 absolute for values
near zero); bf16 outputs within 2e-2 absolute + 2e-2 relative. Small cases are compared
element by element; the full-size workloads on sampled chunks and query rows.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import ssm_compressed_chunked_amd as att
from ssm_compressed_chunked_amd.pipeline import chunk_layout, layer_forward, prefill_forward
from workloads import (PREFILL_BF16, TINY_FP32, TRAIN_BF16, VARCHUNK_BF16, make_prefill, make_projection,
                       make_ragged_prefill)

pytestmark = pytest.mark.gpu

MODE = {"train": att.MASK_TRAIN, "test": att.MASK_TEST}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_close(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if dtype == "fp32":
        bound = 1e-4 * np.abs(ref) + 1e-5
    else:
        bound = 2e-2 + 2e-2 * np.abs(ref)
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; max err "
                           f"{err.max():.3e} at {np.unravel_index(np.argmax(err - bound), err.shape)}")
    return float(err.max())


def to_dev(inp):
    act = {k: v.cuda() for k, v in inp.act.items()}
    par = {k: v.cuda() for k, v in inp.param.items()}
    return act, par


def f64_inputs(inp):
    names = list(inp.act) + list(inp.param)
    return {k: inp.f64(k) for k in names}


# ---------------------------------------------------------------------------------- layout
@pytest.mark.parametrize("seq_lens,P,layer", [
    ([256], 4, 0), ([2048] * 4, 8, 3), ([8192] * 2, 8, 0), ([5, 0, 12, 1, 33], 4, 1),
    ([1, 1, 1], 3, 2), ([100], 1, 0), ([7, 64, 3], 64, 5), ([3000] * 3 + [1], 128, 130)])
def test_uniform_boundaries_bit_exact(seq_lens, P, layer):
    say(f"boundaries lens={seq_lens[:4]} P={P} layer={layer}")
    seq_cu_h = np.concatenate([[0], np.cumsum(seq_lens)]).astype(np.int32)
    T = int(seq_cu_h[-1])
    lay = chunk_layout(seq_cu_h, torch.from_numpy(seq_cu_h).cuda(), T, P, layer)
    ref_cu, ref_tc, ref_ie = oracle.segment(seq_cu_h, P, layer)
    assert lay.n_chunks == len(ref_cu) - 1
    np.testing.assert_array_equal(lay.chunk_cu.cpu().numpy(), ref_cu)
    np.testing.assert_array_equal(lay.token_chunk.cpu().numpy(), ref_tc)
    np.testing.assert_array_equal(lay.is_end.cpu().numpy(), ref_ie)


@pytest.mark.parametrize("n_seq,P,layer", [(3000, 6, 4), (4096, 3, 1), (4097, 7, 0), (6000, 5, 2)])
def test_many_sequences_boundaries(n_seq, P, layer):
    """Batches up to 4096 sequences take the one-launch layout kernel, larger ones the
    two-kernel path; empty sequences included."""
    say(f"boundaries n_seq={n_seq} P={P} layer={layer}")
    rng = np.random.default_rng(5 + n_seq)
    lens = rng.integers(0, 40, size=n_seq)
    lens[0] = 0
    seq_cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(seq_cu_h[-1])
    lay = chunk_layout(seq_cu_h, torch.from_numpy(seq_cu_h).cuda(), T, P, layer)
    ref_cu, ref_tc, ref_ie = oracle.segment(seq_cu_h, P, layer)
    np.testing.assert_array_equal(lay.chunk_cu.cpu().numpy(), ref_cu)
    np.testing.assert_array_equal(lay.token_chunk.cpu().numpy(), ref_tc)
    np.testing.assert_array_equal(lay.is_end.cpu().numpy(), ref_ie)


def test_empty_batch_boundaries():
    """All sequences empty: no chunks, chunk_cu = [0]."""
    seq_cu_h = np.zeros(4, dtype=np.int32)
    lay = chunk_layout(seq_cu_h, torch.from_numpy(seq_cu_h).cuda(), 0, 4, 1)
    assert lay.n_chunks == 0
    np.testing.assert_array_equal(lay.chunk_cu.cpu().numpy(), [0])
    assert lay.token_chunk.numel() == 0 and lay.is_end.numel() == 0


def test_random_chunk_index_bit_exact():
    inp = make_prefill(VARCHUNK_BF16)
    T = VARCHUNK_BF16.T
    lay = chunk_layout(inp.seq_cu, torch.from_numpy(inp.seq_cu).cuda(), T, None, 0,
                       chunk_lens=inp.chunk_lens)
    ref_cu, ref_tc, ref_ie = oracle.segment(inp.seq_cu, chunk_lens=inp.chunk_lens)
    assert lay.n_chunks == len(ref_cu) - 1 == 1855
    np.testing.assert_array_equal(lay.chunk_cu.cpu().numpy(), ref_cu)
    np.testing.assert_array_equal(lay.token_chunk.cpu().numpy(), ref_tc)
    np.testing.assert_array_equal(lay.is_end.cpu().numpy(), ref_ie)


# ------------------------------------------------------------------------- whole forward
SMALL_CASES = [
    # (name, base config, overrides, sequence lengths or None, random chunks)
    ("tiny_fp32", TINY_FP32, {}, None, False),
    ("tiny_fp32_ragged_test_L3", TINY_FP32, dict(mode="test", L=3, layer_idx=2), [70, 1, 130], False),
    ("bf16_train_L64_o3", TRAIN_BF16, dict(B=2, n=300, d=256, H=4), None, False),
    ("bf16_test_L64", PREFILL_BF16, dict(B=2, n=333, d=256, H=4), None, False),
    ("bf16_test_L0", PREFILL_BF16, dict(B=1, n=200, d=128, H=2, L=0), None, False),
    ("bf16_train_L0_P4", PREFILL_BF16, dict(B=1, n=257, d=128, H=2, L=0, P=4, mode="train"), None, False),
    ("bf16_test_L1_ragged", PREFILL_BF16, dict(d=128, H=2, L=1, P=5, layer_idx=7), [1, 190, 0, 67], False),
    ("bf16_random_chunks", VARCHUNK_BF16, dict(d=128, H=2), [150, 211], True),
    ("bf16_hd128", PREFILL_BF16, dict(B=1, n=260, d=256, H=2, hd=128), None, False),
    ("bf16_hd32_N32", PREFILL_BF16, dict(B=1, n=150, d=128, H=4, hd=32, N=32, mode="train", L=5), None, False),
    ("fp32_hd64_train", TINY_FP32, dict(d=128, H=2, hd=64, n=190, P=3, L=7, layer_idx=1), None, False),
    # every token its own chunk: each key is a boundary state, E_i = i
    ("bf16_P1_test_L0", PREFILL_BF16, dict(B=1, n=300, d=128, H=2, P=1, L=0), None, False),
    # chunks longer than a key tile: token-loop scan; M_train band reaching 127 tokens back
    ("bf16_P128_train_L16", TRAIN_BF16, dict(B=1, n=700, d=128, H=2, P=128, L=16, layer_idx=5), None, False),
    ("bf16_P64_test_L3", PREFILL_BF16, dict(B=2, n=270, d=128, H=2, P=64, L=3, layer_idx=1), None, False),
    # hd 128 on the matrix cores with a window wider than two key tiles
    ("bf16_hd128_train_L200", TRAIN_BF16, dict(B=1, n=520, d=256, H=2, hd=128, P=8, L=200), None, False),
    # many short sequences: query tiles mostly past their sequence's end
    ("bf16_tiny_seqs", PREFILL_BF16, dict(d=128, H=2, L=2, P=3, layer_idx=1), [1, 2, 3, 1, 64, 129, 0, 5], False),
]


def _build_inputs(base, over, lens, rnd, seed=11):
    cfg = base.with_(**over)
    if lens is None:
        inp = make_prefill(cfg, seed=seed) if not rnd else make_prefill(cfg.with_(chunking="random"), seed=seed)
        return cfg, inp
    chunk_lens = None
    if rnd:
        from workloads import draw_chunk_lengths
        crng = np.random.default_rng(seed)
        chunk_lens = []
        for n in lens:
            chunk_lens += draw_chunk_lengths(crng, n, cfg.chunk_len_lo, cfg.chunk_len_hi)
    inp = make_ragged_prefill(cfg, lens, seed=seed, chunk_lens=chunk_lens)
    return inp.cfg, inp


@pytest.mark.parametrize("name,base,over,lens,rnd", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_forward_small_elementwise(name, base, over, lens, rnd):
    cfg, inp = _build_inputs(base, over, lens, rnd)
    say(f"forward {name}: T={int(inp.seq_cu[-1])} d={cfg.d} H={cfg.H} hd={cfg.hd} N={cfg.N} "
        f"P={cfg.P} L={cfg.L} layer={cfg.layer_idx} mode={cfg.mode} random={rnd}")
    act, par = to_dev(inp)
    P = None if rnd else cfg.P
    res = prefill_forward(act, par, inp.seq_cu, cfg.H, cfg.hd, P, cfg.layer_idx, cfg.L,
                          MODE[cfg.mode], chunk_lens=inp.chunk_lens)
    torch.cuda.synchronize()
    ref = oracle.kvssm_forward(f64_inputs(inp), inp.seq_cu, cfg.H, cfg.hd, P, cfg.layer_idx,
                               cfg.L, cfg.mode, chunk_lens=inp.chunk_lens)
    T = int(inp.seq_cu[-1])
    np.testing.assert_array_equal(res["layout"].chunk_cu.cpu().numpy(), ref["chunk_cu"])
    for key in ("y_k", "y_v"):
        check_close(res["scan"][key].float().cpu().numpy(), ref[key], cfg.dtype, key)
    n = res["layout"].n_chunks
    check_close(res["scan"]["kb"].float().cpu().numpy().reshape(n, cfg.H, cfg.hd), ref["kb"],
                cfg.dtype, "kb")
    check_close(res["scan"]["vb"].float().cpu().numpy().reshape(n, cfg.H, cfg.hd), ref["vb"],
                cfg.dtype, "vb")
    check_close(res["out"].float().cpu().numpy(), ref["out"], cfg.dtype, "out")
    lse = res["lse"].cpu().numpy()
    fin = np.isfinite(ref["lse"])
    assert (np.isfinite(lse) == fin).all()
    check_close(lse[fin], ref["lse"][fin], cfg.dtype, "lse")


def test_h_last_handoff():
    cfg = TRAIN_BF16.with_(d=128, H=2, n=75, B=3)
    inp = make_ragged_prefill(cfg, [75, 9, 40], seed=3)
    act, par = to_dev(inp)
    seq_cu = torch.from_numpy(inp.seq_cu).cuda()
    T = int(inp.seq_cu[-1])
    lay = chunk_layout(inp.seq_cu, seq_cu, T, cfg.P, cfg.layer_idx)
    s = att.kvssm_scan(act["x"], act["dt_k"], act["dt_v"], act["bm_k"], act["cm_k"], act["bm_v"],
                       act["cm_v"], par["A_k"], par["A_v"], par["D_k"], par["D_v"], par["bias_k"],
                       par["bias_v"], lay.chunk_cu, seq_cu=seq_cu, h_last=True)
    torch.cuda.synchronize()
    f = f64_inputs(inp)
    ends = set(int(v) - 1 for v in inp.seq_cu[1:])
    for tag in ("k", "v"):
        _, snaps = oracle.selective_scan(f["x"], f[f"dt_{tag}"], f[f"bias_{tag}"], f[f"A_{tag}"],
                                         f[f"bm_{tag}"], f[f"cm_{tag}"], f[f"D_{tag}"],
                                         oracle.segment(inp.seq_cu, cfg.P, cfg.layer_idx)[0],
                                         snapshot_after=ends)
        got = s[f"h_last_{tag}"].cpu().numpy()
        for si, e in enumerate(sorted(ends)):
            # the state itself is float32 on the GPU: 1e-3 relative to the state scale
            ref = snaps[e]
            assert np.abs(got[si] - ref).max() <= 1e-3 * (np.abs(ref).max() + 1e-6)


# --------------------------------------------------- full-size workloads, every sequence
def _attn_heads(cfg, s):
    """Heads checked on every row of sequence s: all of them at train_bf16 (n = 2048), else two
    that differ from one sequence to the next."""
    if cfg.n <= 2048:
        return list(range(cfg.H))
    a = (5 * s) % cfg.H
    return sorted({a, cfg.H - 1 - a})


@pytest.mark.parametrize("cfg", [TRAIN_BF16, PREFILL_BF16, VARCHUNK_BF16], ids=lambda c: c.name)
def test_full_size_every_sequence(cfg):
    """The full workloads in the launch configuration the benchmark times (segmentation, the
    scan with boundary outputs, the attention with its LSE). For every sequence: y_k, y_v at
    every token and kb, vb at every chunk against the oracle's scan of that whole sequence;
    O and LSE of every row for some heads (all heads at train_bf16), and of 44 rows (the first
    two, the last two and 40 drawn) for every head, against the oracle's attention over the
    oracle's own keys and values."""
    say(f"full-size {cfg.name}")
    inp = make_prefill(cfg)
    act, par = to_dev(inp)
    rnd = cfg.chunking == "random"
    P = None if rnd else cfg.P
    res = prefill_forward(act, par, inp.seq_cu, cfg.H, cfg.hd, P, cfg.layer_idx, cfg.L,
                          MODE[cfg.mode], chunk_lens=inp.chunk_lens)
    torch.cuda.synchronize()
    ref_cu, ref_tc, ref_ie = oracle.segment(inp.seq_cu, P, cfg.layer_idx, inp.chunk_lens)
    np.testing.assert_array_equal(res["layout"].chunk_cu.cpu().numpy(), ref_cu)
    np.testing.assert_array_equal(res["layout"].token_chunk.cpu().numpy(), ref_tc)
    np.testing.assert_array_equal(res["layout"].is_end.cpu().numpy(), ref_ie)
    f = f64_inputs(inp)
    T, H, hd = cfg.T, cfg.H, cfg.hd
    got = {k: res["scan"][k].float().cpu().numpy() for k in ("y_k", "y_v", "kb", "vb")}
    out_all = res["out"].float().cpu().numpy()
    lse_all = res["lse"].cpu().numpy()
    q3 = f["q"].reshape(T, H, hd)
    rng = np.random.default_rng(0)
    for si in range(len(inp.seq_cu) - 1):
        a, b = int(inp.seq_cu[si]), int(inp.seq_cu[si + 1])
        qa, qb = int(ref_tc[a]), int(ref_tc[b - 1]) + 1          # the sequence's chunks
        ys = {}
        for tag in ("k", "v"):
            y, _ = oracle.selective_scan(f["x"], f[f"dt_{tag}"], f[f"bias_{tag}"], f[f"A_{tag}"],
                                         f[f"bm_{tag}"], f[f"cm_{tag}"], f[f"D_{tag}"], ref_cu,
                                         t_begin=a, t_end=b)
            ys[tag] = y
            check_close(got[f"y_{tag}"][a:b], y, cfg.dtype, f"y_{tag} of sequence {si}")
            bref = oracle.boundary_states(y, ref_cu[qa:qb + 1] - a)
            check_close(got[f"{tag}b"][qa:qb], bref, cfg.dtype, f"{tag}b of sequence {si}")
        # attention of this sequence over the oracle's keys and values (rows of the other
        # sequences never see them, so zeros stand in there)
        k3 = np.zeros((T, H, hd)); v3 = np.zeros((T, H, hd))
        k3[a:b] = ys["k"].reshape(-1, H, hd)
        v3[a:b] = ys["v"].reshape(-1, H, hd)
        heads = _attn_heads(cfg, si)
        o_h, l_h = oracle.chunk_attention(q3[:, heads], k3[:, heads], v3[:, heads], inp.seq_cu,
                                          ref_tc, ref_ie, cfg.L, cfg.mode, rows=np.arange(a, b))
        check_close(out_all[a:b][:, heads], o_h, cfg.dtype, f"O of sequence {si}, heads {heads}")
        check_close(lse_all[heads, a:b], l_h, cfg.dtype, f"LSE of sequence {si}, heads {heads}")
        rows = np.unique(np.concatenate([rng.integers(a, b, 40), [a, a + 1, b - 2, b - 1]]))
        o_r, l_r = oracle.chunk_attention(q3, k3, v3, inp.seq_cu, ref_tc, ref_ie, cfg.L,
                                          cfg.mode, rows=rows)
        check_close(out_all[rows], o_r, cfg.dtype, f"O rows of sequence {si}, all heads")
        check_close(lse_all[:, rows], l_r, cfg.dtype, f"LSE rows of sequence {si}, all heads")
        say(f"  sequence {si}: scan and attention match")


@pytest.mark.parametrize("cfg", [PREFILL_BF16, VARCHUNK_BF16], ids=lambda c: c.name)
def test_full_size_handoff_and_boundaries(cfg):
    """At full size (prefill_bf16's grid walks two chunks per wave, varchunk_bf16's one, with
    chunks of up to 16 tokens in two blocks): every sequence's hand-off state against the oracle
    run over that sequence's last chunk alone (the state restarts at every chunk start, so the
    last chunk fixes it), and every boundary state equal to the per-token output at its chunk's
    last token (the same value, stored twice)."""
    say(f"full-size hand-off {cfg.name}")
    inp = make_prefill(cfg)
    act, par = to_dev(inp)
    rnd = cfg.chunking == "random"
    P = None if rnd else cfg.P
    seq_cu = torch.from_numpy(inp.seq_cu).cuda()
    T = cfg.T
    lay = chunk_layout(inp.seq_cu, seq_cu, T, P, cfg.layer_idx, chunk_lens=inp.chunk_lens)
    s = att.kvssm_scan(act["x"], act["dt_k"], act["dt_v"], act["bm_k"], act["cm_k"], act["bm_v"],
                       act["cm_v"], par["A_k"], par["A_v"], par["D_k"], par["D_v"], par["bias_k"],
                       par["bias_v"], lay.chunk_cu, seq_cu=seq_cu, h_last=True)
    torch.cuda.synchronize()
    ref_cu = oracle.segment(inp.seq_cu, P, cfg.layer_idx, inp.chunk_lens)[0]
    ends = ref_cu[1:] - 1
    for tag in ("k", "v"):
        y, kb = s[f"y_{tag}"], s[f"{tag}b"]
        assert torch.equal(kb, y[torch.from_numpy(ends.astype(np.int64)).cuda()]), f"{tag}b != y at chunk ends"
    f = f64_inputs(inp)
    got = {tag: s[f"h_last_{tag}"].cpu().numpy() for tag in ("k", "v")}
    for si in range(len(inp.seq_cu) - 1):
        e = int(inp.seq_cu[si + 1]) - 1
        q = int(np.searchsorted(ref_cu, e, side="right")) - 1     # the sequence's last chunk
        a = int(ref_cu[q])
        for tag in ("k", "v"):
            _, snaps = oracle.selective_scan(f["x"], f[f"dt_{tag}"], f[f"bias_{tag}"], f[f"A_{tag}"],
                                             f[f"bm_{tag}"], f[f"cm_{tag}"], f[f"D_{tag}"], ref_cu,
                                             t_begin=a, t_end=e + 1, snapshot_after={e})
            ref = snaps[e]
            # the state is float32 on the GPU from bf16 inputs: 1e-3 relative to its scale
            assert np.abs(got[tag][si] - ref).max() <= 1e-3 * (np.abs(ref).max() + 1e-6), \
                f"h_last_{tag} of sequence {si}"


# ------------------------------------------------------------------------------ decode
@pytest.mark.parametrize("H,hd,N,P,L,layer,n0,steps,dtype", [
    (2, 128, 16, 4, 8, 0, 21, 13, "bf16"),
    (4, 64, 16, 4, 5, 1, 9, 11, "bf16"),
    (2, 32, 32, 3, 1, 2, 7, 9, "bf16"),
    (2, 64, 16, 4, 0, 0, 12, 10, "bf16"),
    (2, 32, 16, 2, 600, 1, 300, 8, "bf16"),
    (2, 32, 16, 4, 6, 3, 17, 9, "fp32"),
    (2, 64, 16, 1, 1, 0, 5, 7, "bf16"),       # every position ends a chunk; window of one
])
def test_decode_matches_prefill_rows(H, hd, N, P, L, layer, n0, steps, dtype):
    say(f"decode H={H} hd={hd} N={N} P={P} L={L} layer={layer} n0={n0} dtype={dtype}")
    B = 3
    d = H * hd
    o = layer % P
    n_total = n0 + steps
    n_total += (o - n_total) % P
    base = PREFILL_BF16 if dtype == "bf16" else TINY_FP32
    cfg = base.with_(B=B, n=n_total, d=d, H=H, hd=hd, N=N, P=P, L=L, layer_idx=layer, mode="test")
    inp = make_prefill(cfg, seed=100 + n0)
    f = f64_inputs(inp)
    T = cfg.T
    ref = oracle.kvssm_forward(f, inp.seq_cu, H, hd, P, layer, L, "test")
    chunk_cu = ref["chunk_cu"]
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    cap = n_total // P + 4
    n_bound0 = sum(1 for j in range(n0) if oracle.is_chunk_end_at(j, P, layer))
    cache = att.DecodeCache(B, H, hd, N, P, L, layer, cap, tdt, inp.param, pos=n0, n_bound=n_bound0)
    for b in range(B):
        a = int(inp.seq_cu[b])
        snaps = {}
        for tag in ("k", "v"):
            _, sn = oracle.selective_scan(f["x"], f[f"dt_{tag}"], f[f"bias_{tag}"], f[f"A_{tag}"],
                                          f[f"bm_{tag}"], f[f"cm_{tag}"], f[f"D_{tag}"], chunk_cu,
                                          t_begin=a, t_end=a + n0, snapshot_after={a + n0 - 1})
            snaps[tag] = sn[a + n0 - 1]
        st = oracle.decode_state_from_prefix(ref["y_k"][a:a + n0], ref["y_v"][a:a + n0],
                                             snaps["k"], snaps["v"], n0, H, hd, P, layer, L)
        for idx, (_, kr, vr) in enumerate(st.bounds):
            cache.kb[b, :, idx] = torch.from_numpy(kr).to(tdt)
            cache.vb[b, :, idx] = torch.from_numpy(vr).to(tdt)
        for (pos, kr, vr) in st.recent:
            cache.kw[b, :, pos % L] = torch.from_numpy(kr).to(tdt)
            cache.vw[b, :, pos % L] = torch.from_numpy(vr).to(tdt)
        cache.h_k[b] = torch.from_numpy(st.h_k).float()
        cache.h_v[b] = torch.from_numpy(st.h_v).float()
    act = {k: v.cuda() for k, v in inp.act.items()}
    for i in range(n0, n_total):
        rows = torch.from_numpy(inp.seq_cu[:-1] + i).long().cuda()
        out = att.decode_step(cache, act["q"][rows].view(B, H, hd).contiguous(),
                              act["x"][rows].contiguous(), act["dt_k"][rows].contiguous(),
                              act["dt_v"][rows].contiguous(), act["bm_k"][rows].contiguous(),
                              act["cm_k"][rows].contiguous(), act["bm_v"][rows].contiguous(),
                              act["cm_v"][rows].contiguous())
        torch.cuda.synchronize()
        check_close(out.float().cpu().numpy(), ref["out"][inp.seq_cu[:-1] + i], dtype, f"decode pos {i}")
    assert cache.pos == n_total
    assert cache.n_bound == sum(1 for j in range(n_total) if oracle.is_chunk_end_at(j, P, layer))


def test_decode_rejects_full_cache_and_bad_mirror():
    B, H, hd, N, P, L = 1, 2, 32, 16, 4, 4
    par = make_prefill(TINY_FP32.with_(d=64, H=H, hd=hd)).param
    cache = att.DecodeCache(B, H, hd, N, P, L, 0, 1, torch.bfloat16, par, pos=3, n_bound=0)
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    args = (z(B, H, hd), z(B, H * hd), z(B, H * hd), z(B, H * hd), z(B, N), z(B, N), z(B, N), z(B, N))
    att.decode_step(cache, *args)              # pos 3 ends a chunk: appended at slot 0
    assert cache.n_bound == 1
    cache.set_position(7, 1)                   # pos 7 ends the next chunk: cache full
    with pytest.raises(att.AttambaError) as e:
        att.decode_step(cache, *args)
    assert e.value.status == 4
    cache.set_position(8, 1)                   # two ends (3, 7) precede pos 8, not one
    with pytest.raises(att.AttambaError) as e:
        att.decode_step(cache, *args)
    assert e.value.status == 2


@pytest.mark.parametrize("H,hd,ctx", [(32, 128, 32768), (64, 64, 8192), (128, 32, 8192)])
def test_decode_full_size_wide_split(H, hd, ctx):
    """decode_bf16 at full size (32 sequences x 32 heads, 8 192 boundary states plus a window of
    256 per sequence), and the same width split into 64 heads of 64 or 128 heads of 32 at a
    quarter of the context: the key lists are cut into splits of 1 024 keys, the launch the
    decode bench times. Two steps from a random cache; sequences 0 and 31 are checked against
    the oracle's decode step on the same cache contents."""
    from workloads import DECODE_CONFIGS, make_decode
    cfg = DECODE_CONFIGS["decode_bf16"].with_(H=H, hd=hd, ctx=ctx)
    assert cfg.H * cfg.hd == cfg.d
    say(f"decode full size B={cfg.B} H={cfg.H} hd={cfg.hd} ctx={cfg.ctx}")
    P, L, layer = cfg.P, cfg.L, cfg.layer_idx
    ends = [j for j in range(cfg.ctx) if oracle.is_chunk_end_at(j, P, layer)]
    n_bound = len(ends)
    assert n_bound == att.count_chunks([0, cfg.ctx], P, layer)
    steps = 2
    inp = make_decode(cfg, n_bound=n_bound, steps=steps, device="cuda")
    cache = att.DecodeCache(cfg.B, cfg.H, cfg.hd, cfg.N, P, L, layer, n_bound + 4, torch.bfloat16,
                            inp.param, pos=cfg.ctx, n_bound=n_bound)
    cache.kb[:, :, :n_bound] = inp.kb
    cache.vb[:, :, :n_bound] = inp.vb
    cache.kw.copy_(inp.kw)
    cache.vw.copy_(inp.vw)
    act = {k: v.cuda() for k, v in inp.act.items()}
    outs = []
    for s in range(steps):
        out = att.decode_step(cache, act["q"][s].view(cfg.B, cfg.H, cfg.hd).contiguous(), act["x"][s],
                              act["dt_k"][s], act["dt_v"][s], act["bm_k"][s], act["cm_k"][s],
                              act["bm_v"][s], act["cm_v"][s])
        outs.append(out.float().cpu().numpy())
    torch.cuda.synchronize()
    par = {k: v.double().numpy() for k, v in inp.param.items()}
    for b in (0, cfg.B - 1):
        kb = inp.kb[b].double().cpu().numpy()          # [H, n_bound, hd]
        vb = inp.vb[b].double().cpu().numpy()
        kw = inp.kw[b].double().cpu().numpy()          # [H, L, hd]
        vw = inp.vw[b].double().cpu().numpy()
        st = oracle.DecodeSeq(pos=cfg.ctx, h_k=np.zeros((cfg.d, cfg.N)), h_v=np.zeros((cfg.d, cfg.N)))
        st.bounds = [(j, kb[:, idx], vb[:, idx]) for idx, j in enumerate(ends)]
        st.recent = [(j, kw[:, j % L], vw[:, j % L]) for j in range(cfg.ctx - L, cfg.ctx)]
        for s in range(steps):
            tok = {k: v[s, b].double().numpy() for k, v in inp.act.items()}
            ref = oracle.decode_step(st, par, tok, cfg.H, cfg.hd, P, layer, L)
            check_close(outs[s][b], ref, "bf16", f"full-size decode sequence {b} step {s}")


def test_decode_snapshot_resume_bit_exact():
    """The cache buffers plus the host mirrors (pos, n_bound) are the whole decode state: a
    snapshot restored after more steps replays those steps with identical outputs."""
    B, H, hd, N, P, L, layer = 2, 4, 64, 16, 4, 6, 1
    d = H * hd
    cfg = PREFILL_BF16.with_(B=B, n=64, d=d, H=H, hd=hd, N=N, P=P, L=L, layer_idx=layer)
    inp = make_prefill(cfg, seed=77)
    act = {k: v.cuda() for k, v in inp.act.items()}
    cache = att.DecodeCache(B, H, hd, N, P, L, layer, 64 // P + 4, torch.bfloat16, inp.param,
                            pos=0, n_bound=0)

    def step(i):
        rows = torch.from_numpy(inp.seq_cu[:-1] + i).long().cuda()
        return att.decode_step(cache, act["q"][rows].view(B, H, hd).contiguous(),
                               act["x"][rows].contiguous(), act["dt_k"][rows].contiguous(),
                               act["dt_v"][rows].contiguous(), act["bm_k"][rows].contiguous(),
                               act["cm_k"][rows].contiguous(), act["bm_v"][rows].contiguous(),
                               act["cm_v"][rows].contiguous()).clone()

    for i in range(13):
        step(i)
    names = ("kb", "vb", "kw", "vw", "h_k", "h_v")
    snap = {k: getattr(cache, k).clone() for k in names}
    pos, nb = cache.pos, cache.n_bound
    first = [step(i) for i in range(13, 30)]
    for k in names:
        getattr(cache, k).copy_(snap[k])
    cache.set_position(pos, nb)
    second = [step(i) for i in range(13, 30)]
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a, b)
    assert cache.pos == 30


@pytest.mark.parametrize("hd,mode,L", [(64, "test", 64), (128, "train", 5), (64, "test", 0)])
def test_attention_growing_scores(hd, mode, L):
    """Scores that grow along the sequence by far more than 2^64 per row (keys k_j = a_j u with
    a_j rising, queries along u) force the rare exact-maximum path of the lazy softmax again
    and again, and scores that fall far below the first ones must not disturb the result."""
    say(f"attention growing scores hd={hd} mode={mode} L={L}")
    rng = np.random.default_rng(hd + L)
    n, H, P = 700, 2, 4
    seq_cu = np.array([0, n], dtype=np.int32)
    u = rng.standard_normal(hd)
    u /= np.linalg.norm(u)
    a = np.concatenate([np.linspace(0.0, 60.0, n // 2), np.linspace(60.0, -40.0, n - n // 2)])
    k = (a[:, None, None] * u[None, None, :] + 0.05 * rng.standard_normal((n, H, hd)))
    q = np.sqrt(hd) * np.ones((n, H, 1)) * u[None, None, :] + 0.05 * rng.standard_normal((n, H, hd))
    v = rng.standard_normal((n, H, hd))
    bf = lambda x: torch.from_numpy(x).to(torch.bfloat16)
    qt, kt, vt = bf(q), bf(k), bf(v)
    cu, tc, ie = oracle.segment(seq_cu, P, 0)
    ends = np.asarray(cu[1:], dtype=np.int64) - 1
    dev = lambda t: t.contiguous().cuda()
    out, lse = att.chunk_attn_fwd(dev(qt), dev(kt), dev(vt), dev(kt[ends]), dev(vt[ends]),
                                  torch.from_numpy(seq_cu).cuda(), torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda(),
                                  torch.from_numpy(tc.astype(np.int32)).cuda(), n, L, MODE[mode])
    torch.cuda.synchronize()
    f = lambda t: t.double().numpy()
    ref_o, ref_l = oracle.chunk_attention(f(qt), f(kt), f(vt), seq_cu, tc, ie, L, mode)
    check_close(out.float().cpu().numpy(), ref_o, "bf16", "out")
    got_l = lse.cpu().numpy()
    fin = np.isfinite(ref_l)
    assert (np.isfinite(got_l) == fin).all()
    check_close(got_l[fin], ref_l[fin], "bf16", "lse")


# ------------------------------------------------------------------------ input projections
@pytest.mark.parametrize("T,d,widths", [
    (300, 128, [128, 128, 128, 16, 16, 16, 16]),   # the layer's seven outputs, ragged token tail
    (129, 64, [64, 4, 60]),                         # feature segments inside one tile
    (1, 256, [256]),
    (517, 192, [192, 192, 192, 32, 32, 32, 32, 4]),  # N = 32, eight segments, ragged both ways
    # a last feature tile of at most 64 features goes to the tail kernel
    (300, 128, [256, 16, 16, 16, 16]),              # 64 past the full tile, as at the prefill shape
    (517, 192, [512, 4, 32, 8]),                    # 44 past two full tiles, ragged tokens
    (77, 64, [20, 8]),                              # no full tile at all
])
def test_input_proj_elementwise(T, d, widths):
    say(f"input_proj T={T} d={d} widths={widths}")
    n_out = sum(widths)
    inp = make_projection(T, d, 16, seed=T + d)
    rng = np.random.default_rng(T)
    w = (torch.from_numpy(rng.standard_normal((n_out, d)).astype(np.float32)) * 0.02).to(torch.bfloat16)
    outs = att.input_proj(inp.x.cuda(), w.cuda(), widths)
    torch.cuda.synchronize()
    ref = oracle.linear(inp.x.double().numpy(), w.double().numpy())
    start = 0
    for i, wd in enumerate(widths):
        check_close(outs[i].float().cpu().numpy(), ref[:, start:start + wd], "bf16", f"segment {i}")
        start += wd


def test_input_proj_full_size_sampled():
    """The projection of the prefill workload (T = 16384, d = 2048, N = 16) in the launch
    configuration the benchmark times, checked on sampled rows (tile edges included)."""
    T, d, N = 16384, 2048, 16
    inp = make_projection(T, d, N, seed=2)
    outs = att.input_proj(inp.x.cuda(), inp.w.cuda(), inp.widths)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 129, 4095, 8191, 8192, 12000, T - 129, T - 2, T - 1])
    ref = oracle.linear(inp.x[rows].double().numpy(), inp.w.double().numpy())
    start = 0
    for i, wd in enumerate(inp.widths):
        got = outs[i][torch.from_numpy(rows).cuda()].float().cpu().numpy()
        check_close(got, ref[:, start:start + wd], "bf16", f"segment {i}")
        start += wd


@pytest.mark.parametrize("layer,explicit_kv", [(0, False), (3, False), (6, False), (1, True)])
def test_layer_forward_from_x(layer, explicit_kv):
    """Projections on the matrix cores feeding the KV-SSM forward, for three layers whose
    chunk boundaries are shifted by the layer index. The oracle projects in float64 and rounds
    to bf16 with round-to-nearest-even, the storage type the GPU path hands to the scan."""
    T, d, H, hd, N, P, L = 330, 128, 2, 64, 16, 4, 5
    say(f"layer forward layer={layer} explicit_kv={explicit_kv}")
    pj = make_projection(T, d, N, seed=40 + layer)
    names = ["q", "dt_k", "dt_v", "bm_k", "cm_k", "bm_v", "cm_v"]
    widths = [d, d, d, N, N, N, N]
    if explicit_kv:   # two more weight blocks: the key and value projections
        rng = np.random.default_rng(50 + layer)
        extra = torch.from_numpy(rng.standard_normal((2 * d, d)).astype(np.float32) * 0.05).to(torch.bfloat16)
        pj.w = torch.cat([pj.w[:d], extra, pj.w[d:]])
        names = ["q", "x", "x_v"] + names[1:]
        widths = [d, d, d] + widths[1:]
    par = make_prefill(PREFILL_BF16.with_(B=1, n=T, d=d, H=H, hd=hd, N=N), seed=41).param
    seq_cu = np.array([0, 200, T], dtype=np.int32)
    res = layer_forward(pj.x.cuda(), pj.w.cuda(), {k: v.cuda() for k, v in par.items()}, seq_cu,
                        H, hd, N, P, layer, L, att.MASK_TEST, explicit_kv=explicit_kv)
    torch.cuda.synchronize()
    proj = oracle.linear(pj.x.double().numpy(), pj.w.double().numpy())
    proj = torch.from_numpy(proj).to(torch.bfloat16).double().numpy()   # storage rounding
    f = {"x": pj.x.double().numpy()}
    start = 0
    for name, wd in zip(names, widths):
        f[name] = proj[:, start:start + wd]
        start += wd
    for k, v in par.items():
        f[k] = v.double().numpy()
    ref = oracle.kvssm_forward(f, seq_cu, H, hd, P, layer, L, "test")
    np.testing.assert_array_equal(res["layout"].chunk_cu.cpu().numpy(), ref["chunk_cu"])
    check_close(res["scan"]["y_k"].float().cpu().numpy(), ref["y_k"], "bf16", "y_k")
    check_close(res["out"].float().cpu().numpy(), ref["out"], "bf16", "out")


def test_scan_separate_value_input():
    """SSM_V on its own input (explicit value projection kept in front of the SSM): y_K is the
    usual result, y_V follows x_v."""
    cfg = PREFILL_BF16.with_(B=2, n=150, d=128, H=2, P=8, L=4)
    inp = make_prefill(cfg, seed=31)
    rng = np.random.default_rng(31)
    xv = torch.from_numpy(rng.standard_normal((cfg.T, cfg.d)).astype(np.float32)).to(torch.bfloat16)
    act, par = to_dev(inp)
    lay = chunk_layout(inp.seq_cu, torch.from_numpy(inp.seq_cu).cuda(), cfg.T, cfg.P, 0)
    res = att.kvssm_scan(act["x"], act["dt_k"], act["dt_v"], act["bm_k"], act["cm_k"], act["bm_v"],
                         act["cm_v"], par["A_k"], par["A_v"], par["D_k"], par["D_v"], par["bias_k"],
                         par["bias_v"], lay.chunk_cu, x_v=xv.cuda())
    torch.cuda.synchronize()
    f = f64_inputs(inp)
    f["x_v"] = xv.double().numpy()
    ref = oracle.kvssm_forward(f, inp.seq_cu, cfg.H, cfg.hd, cfg.P, 0, cfg.L, "test")
    check_close(res["y_k"].float().cpu().numpy(), ref["y_k"], "bf16", "y_k")
    check_close(res["y_v"].float().cpu().numpy(), ref["y_v"], "bf16", "y_v")
    check_close(res["vb"].float().cpu().numpy().reshape(-1, cfg.H, cfg.hd), ref["vb"], "bf16", "vb")


# ------------------------------------------------ prefill -> decode, one cache per layer
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_multilayer_prefill_then_decode(dtype):
    """Serving on the GPU alone: every layer (cyclic offsets 0, 1, 2 at P = 3) prefills a prompt
    of n0 tokens per sequence, hands the prefill to its own decode cache on the device
    (attamba_decode_load_prefix: completed boundary states, the last L keys/values, the SSM
    states) and decodes the next tokens. Each decoded output equals the row of the oracle's
    prefill over the whole length."""
    from ssm_compressed_chunked_amd.pipeline import decode_from_prefill
    B, H, hd, N, P, L, n0, steps = 2, 2, 64, 16, 3, 4, 19, 8
    n_total = n0 + steps
    base = PREFILL_BF16 if dtype == "bf16" else TINY_FP32
    for layer in (0, 1, 2):
        cfg = base.with_(B=B, n=n_total, d=H * hd, H=H, hd=hd, N=N, P=P, L=L, layer_idx=layer, mode="test")
        inp = make_prefill(cfg, seed=200 + layer)
        say(f"multilayer decode dtype={dtype} layer={layer}")
        ref = oracle.kvssm_forward(f64_inputs(inp), inp.seq_cu, H, hd, P, layer, L, "test")
        # the prompts: the first n0 tokens of every sequence, packed
        rows = np.concatenate([np.arange(n0) + int(inp.seq_cu[b]) for b in range(B)])
        act_full = {k: v.cuda() for k, v in inp.act.items()}
        act = {k: v[torch.from_numpy(rows).cuda()].contiguous() for k, v in act_full.items()}
        par = {k: v.cuda() for k, v in inp.param.items()}
        seq_cu_h = (np.arange(B + 1) * n0).astype(np.int32)
        res = prefill_forward(act, par, seq_cu_h, H, hd, P, layer, L, att.MASK_TEST, h_last=True)
        cache = decode_from_prefill(res, seq_cu_h, par, H, hd, N, P, layer, L, cap=n_total // P + 2)
        assert cache.pos == n0
        assert cache.n_bound == sum(1 for j in range(n0) if oracle.is_chunk_end_at(j, P, layer))
        for i in range(n0, n_total):
            r = torch.from_numpy(inp.seq_cu[:-1] + i).long().cuda()
            out = att.decode_step(cache, act_full["q"][r].view(B, H, hd).contiguous(),
                                  *[act_full[k][r].contiguous() for k in ("x", "dt_k", "dt_v", "bm_k", "cm_k",
                                                                          "bm_v", "cm_v")])
            torch.cuda.synchronize()
            check_close(out.float().cpu().numpy(), ref["out"][inp.seq_cu[:-1] + i], dtype,
                        f"layer {layer} decode pos {i}")
