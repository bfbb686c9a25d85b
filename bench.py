"""Throughput of the Attamba KV-SSM forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input already resident
in HBM: chunk segmentation, the fused SSM_K/SSM_V scan, and the chunk-aware attention. The
default workload is the prefill configuration (bf16, B=2, n=8192, d=2048, 32 heads x 64,
N=16, P=8, L=64, uniform chunks, M_test + window). Prints one JSON line. Its value is the hot
back-to-back rate; the line also carries per-step times with the caches flushed first (the
train_bf16 forward's working set fits in the 256 MB MALL, so both are reported).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload prefill_bf16|varchunk_bf16|train_bf16]
    python bench.py --workload decode_bf16      # decode configuration, separate line
    python bench.py --workload proj_bf16        # input projections (x W^T) at the prefill shape
    python bench.py --workload layer_bf16       # projections + KV-SSM forward from the layer input
    python bench.py --workload train_step_bf16  # forward + backward at the M_train workload
    python bench.py --workload copy             # reference bandwidth (512 MiB device copy)
    python bench.py --workload valu_issue       # clocks per wave64 VALU / MFMA instruction
    python bench.py --workload block_bf16       # prefill_bf16 with the Mamba-block pieces
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/sec fwd (KV-SSM scan+chunk attn); scan HBM GB/s %peak; attn MFMA %"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# VALU issue capacity: 256 CUs x 4 SIMDs x 32 fp32 lanes per clock x 2.4 GHz = 78.6 T
# lane-instruction slots per second (the 157.3 TFLOP/s fp32 vector peak counts an FMA as two).
VALU_SLOTS_PER_S = 256 * 4 * 32 * 2.4e9
# Issue costs measured by `--workload valu_issue` (shader clocks per wave64 instruction per SIMD
# with several waves per SIMD): a VOP2 instruction with VGPR operands (v_mul, v_fmac) 2.2, and
# v_exp_f32 8.1. One slot is one such VOP2 instruction, so v_exp_f32 counts 8.1 / 2.2 = 3.7.
EXP_SLOTS = 3.7
# Slots per state update of the scan in its cheapest form: multiply for the exponent, v_exp_f32,
# multiply for the input term, FMA state, FMA output (the kernel issues the last two with an SGPR
# row operand, ~4.1 clocks each; that penalty is the kernel's, not the algorithm's).
SLOTS_PER_UPDATE = 4.0 + EXP_SLOTS
PROBE_LIB = os.path.join(ROOT, "ssm_compressed_chunked_amd", "libattamba_probe.so")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="prefill_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--batch", type=int, default=None,
                    help="decode and forward workloads: number of sequences (default: the "
                         "workload's; other batch sizes are not the headline configuration)")
    return ap.parse_args()


def source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "ssm_compressed_chunked_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, sources, workload: str) -> dict | None:
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on
    the current kernel source and on this workload (the bytes depend on the shapes)."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(*sources) or rec.get("workload") != workload:
        return None
    return rec


def scan_algorithmic_bytes(cfg) -> int:
    """x once, dt_K, dt_V, Bm/Cm of both SSMs, y_K and y_V (parameters and the boundary copy
    excluded): 2 * (5 d + 4 N) bytes per token at bf16."""
    e = 2 if cfg.dtype == "bf16" else 4
    return cfg.T * e * (5 * cfg.d + 4 * cfg.N)


def attention_pairs(seq_cu, chunk_cu_np, token_chunk_np, L, train) -> int:
    """Visible (query, key) pairs per head: for every row, (i - w_i + 1) band keys plus the
    E_i boundary states of chunks that end before w_i."""
    total = 0
    for s in range(len(seq_cu) - 1):
        s0, s1 = int(seq_cu[s]), int(seq_cu[s + 1])
        if s1 <= s0:
            continue
        i = np.arange(s0, s1)
        w = np.maximum(s0, i - L + 1)
        if train:
            w = np.minimum(w, chunk_cu_np[token_chunk_np[i]])
        c0 = token_chunk_np[s0]
        wi = np.minimum(w, s1 - 1)
        E = np.where(w < s1, token_chunk_np[wi] - c0, token_chunk_np[s1 - 1] + 1 - c0)
        total += int(((i - w + 1) + E).sum())
    return total


def cpu_baseline(cfg, inp, T_full, scan_budget_s=3.0, attn_budget_s=8.0):
    """The oracle as it stands, on a bounded sample of the same workload: the scan over a
    whole-chunk prefix of sequence 0 (all channels, both SSMs; the prefix grows from 1024
    tokens until about scan_budget_s of work) and the attention of sequence 0 for as many
    heads as fit in about attn_budget_s; scaled to the whole batch (the scan is linear in
    tokens, the attention in sequence-head pairs)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    f = {k: inp.f64(k) for k in list(inp.act) + list(inp.param)}
    chunk_cu, tc, ie = oracle.segment(inp.seq_cu, None if inp.chunk_lens is not None else cfg.P,
                                      cfg.layer_idx, inp.chunk_lens)
    s0, s1 = int(inp.seq_cu[0]), int(inp.seq_cu[1])

    def scan_prefix(n_tok):
        n_tok = int(chunk_cu[np.searchsorted(chunk_cu, min(n_tok, s1))])   # whole chunks
        t0 = time.perf_counter()
        for tag in ("k", "v"):
            oracle.selective_scan(f["x"], f[f"dt_{tag}"], f[f"bias_{tag}"], f[f"A_{tag}"],
                                  f[f"bm_{tag}"], f[f"cm_{tag}"], f[f"D_{tag}"], chunk_cu,
                                  t_begin=0, t_end=n_tok)
        return n_tok, time.perf_counter() - t0

    n_scan, t_scan = scan_prefix(1024)
    if t_scan < scan_budget_s and n_scan < s1:
        n_scan, t_scan = scan_prefix(int(n_scan * scan_budget_s / max(t_scan, 1e-3)))
    H, hd = cfg.H, cfg.hd
    rng = np.random.default_rng(0)
    t_attn, heads = 0.0, 0
    while heads < H and t_attn < attn_budget_s:
        q = f["q"][s0:s1].reshape(-1, H, hd)[:, heads:heads + 1]
        k = rng.standard_normal((s1 - s0, 1, hd))
        v = rng.standard_normal((s1 - s0, 1, hd))
        t0 = time.perf_counter()
        oracle.chunk_attention(q, k, v, [0, s1 - s0], tc[s0:s1] - tc[s0], ie[s0:s1], cfg.L,
                               cfg.mode)
        t_attn += time.perf_counter() - t0
        heads += 1
    n_pairs = (len(inp.seq_cu) - 1) * H
    est = t_scan * (T_full / n_scan) + t_attn / heads * n_pairs
    return {"value": T_full / est, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"oracle scan of tokens 0..{n_scan - 1} of sequence 0 (all {cfg.d} channels, "
                       f"both SSMs: {t_scan:.2f} s) scaled by {T_full / n_scan:.2f}; oracle attention of "
                       f"sequence 0, heads 0..{heads - 1} ({s1 - s0} rows each: {t_attn:.2f} s) scaled "
                       f"to {n_pairs} sequence-head pairs; estimated {est:.1f} s per step")}


WARMUP_MIN_S = 0.5
EVENT_EVERY = 5   # timed prefill steps per step with per-kernel HIP events


def clock_warmup(step, torch) -> int:
    """Untimed steps after the W warm-up steps until at least WARMUP_MIN_S of work has run:
    the GPU raises its clock over the first tens of milliseconds of load, and a timed region
    that starts earlier measures the ramp rather than the kernels. Returns the steps run."""
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < WARMUP_MIN_S:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        n += 10
    return n


def bench_prefill(args):
    import torch
    import ssm_compressed_chunked_amd as att
    from ssm_compressed_chunked_amd import _binding as Bd
    from ssm_compressed_chunked_amd.pipeline import chunk_layout
    from workloads import PREFILL_CONFIGS, make_prefill

    # block_bf16: the prefill workload with the Mamba-block pieces around both SSMs (a 4-tap
    # causal convolution with SiLU on their input, a SiLU gate on their output)
    with_block = args.workload == "block_bf16"
    cfg = PREFILL_CONFIGS["prefill_bf16" if with_block else args.workload]
    if args.batch is not None:
        cfg = cfg.with_(B=args.batch)
    inp = make_prefill(cfg)
    dev = torch.device("cuda", 0)
    act = {k: v.to(dev) for k, v in inp.act.items()}
    par = {k: v.to(dev) for k, v in inp.param.items()}
    block = None
    if with_block:
        from workloads import make_block_inputs
        block = {k: v.to(dev) for k, v in make_block_inputs(inp, 4, seed=cfg.seed).items()}
    seq_cu = torch.from_numpy(inp.seq_cu).to(dev)
    T, d, H, hd = cfg.T, cfg.d, cfg.H, cfg.hd
    rnd = cfg.chunking == "random"
    P = None if rnd else cfg.P
    mode = att.MASK_TRAIN if cfg.mode == "train" else att.MASK_TEST
    max_len = int(np.max(np.diff(inp.seq_cu)))
    # outputs allocated once (the library never allocates)
    lay0 = chunk_layout(inp.seq_cu, seq_cu, T, P, cfg.layer_idx, inp.chunk_lens)
    n = lay0.n_chunks
    chunk_cu_host = None if not rnd else att.chunk_cu_from_lengths(inp.seq_cu, inp.chunk_lens)
    chunk_cu = torch.empty(n + 1, dtype=torch.int32, device=dev)
    if rnd:
        chunk_cu.copy_(torch.from_numpy(chunk_cu_host))
    token_chunk = torch.empty(T, dtype=torch.int32, device=dev)
    is_end = torch.empty(T, dtype=torch.uint8, device=dev)
    y_k = torch.empty_like(act["x"])
    y_v = torch.empty_like(act["x"])
    kb = torch.empty((n, d), dtype=act["x"].dtype, device=dev)
    vb = torch.empty((n, d), dtype=act["x"].dtype, device=dev)
    out = torch.empty((T, H, hd), dtype=act["x"].dtype, device=dev)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if rnd:
            att.chunk_index(chunk_cu, T, token_chunk, is_end, stream=stream)
        else:
            att.chunk_boundaries(seq_cu, T, cfg.P, cfg.layer_idx, n, chunk_cu, token_chunk,
                                 is_end, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        att.kvssm_scan(act["x"], act["dt_k"], act["dt_v"], act["bm_k"], act["cm_k"], act["bm_v"],
                       act["cm_v"], par["A_k"], par["A_v"], par["D_k"], par["D_v"], par["bias_k"],
                       par["bias_v"], chunk_cu, y_k=y_k, y_v=y_v, kb=kb, vb=vb, block=block,
                       stream=stream)
        if ev is not None:
            ev[2].record(stream)
        att.chunk_attn_fwd(act["q"].view(T, H, hd), y_k.view(T, H, hd), y_v.view(T, H, hd),
                           kb.view(n, H, hd), vb.view(n, H, hd), seq_cu, chunk_cu, token_chunk,
                           max_len, cfg.L, mode, out=out, lse=lse, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    extra_warmup = clock_warmup(step, torch)
    # Whole-job timing: exactly K steps, synchronised on both sides, right after the clock
    # warm-up. HIP events recorded on the launch stream between the kernels of every
    # EVENT_EVERY-th of these same steps give the per-kernel durations (each recorded event costs
    # the stream a few microseconds, about 5 % of the step when all four are on every step).
    n_ev = max(1, args.steps // EVENT_EVERY)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_ev)]
    sampled = {min(args.steps - 1, EVENT_EVERY * i + EVENT_EVERY - 1): i for i in range(n_ev)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        i = sampled.get(k)
        step(evs[i] if i is not None else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    scan_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    attn_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    # Then the same steps with the caches flushed before each one (a 512 MiB write evicts the L2s and
    # the 256 MB MALL, which can otherwise hold a small configuration's whole working set).
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for k, e in enumerate(evf):
        flush_buf.fill_(k & 0xFF)
        step(e)
    torch.cuda.synchronize()
    del flush_buf
    flushed = {"kernels_us": {"segmentation": round(float(np.mean([e[0].elapsed_time(e[1]) for e in evf])) * 1e3, 2),
                              "kvssm_scan": round(float(np.mean([e[1].elapsed_time(e[2]) for e in evf])) * 1e3, 2),
                              "chunk_attn": round(float(np.mean([e[2].elapsed_time(e[3]) for e in evf])) * 1e3, 2)},
               "step_us": round(float(np.mean([e[0].elapsed_time(e[3]) for e in evf])) * 1e3, 2),
               "note": "HIP events around each step after a 512 MiB device write; value and kernels_us are hot"}
    ms = wall * 1e3 / args.steps
    tok_s = T / (wall / args.steps)
    pairs = attention_pairs(inp.seq_cu, lay0.chunk_cu.cpu().numpy(), lay0.token_chunk.cpu().numpy(),
                            cfg.L, mode == att.MASK_TRAIN)
    attn_flop = 4.0 * hd * H * pairs
    attn_tflops = attn_flop / (attn_ms * 1e-3) / 1e12
    scan_bytes = scan_algorithmic_bytes(cfg) + (2 * T * d * 2 if with_block else 0)   # + z_k, z_v
    scan_gbps = scan_bytes / (scan_ms * 1e-3) / 1e9
    updates = 2 * T * d * cfg.N
    scan_slots = SLOTS_PER_UPDATE * updates
    scan_alu_tslots = scan_slots / (scan_ms * 1e-3) / 1e12
    alu_peak = VALU_SLOTS_PER_S / 1e12
    # the committed counter runs were taken at the workload's own batch
    own_shape = args.batch is None
    traffic = None if with_block or not own_shape else measured_traffic(
        "kvssm_scan_kernel", ["kvssm_scan.hip", "common.h"], args.workload)
    attn_traffic = None if not own_shape else measured_traffic(
        "attn_mfma_kernel", ["attn_mfma.hip", "attn_geom.h", "attn_tiles.h", "common.h"], args.workload)
    # The scan is the dominant kernel; its roofline is HBM: algorithmic bytes per launch over
    # its event-timed launch duration, against 8 TB/s. Its instruction-issue figure (the stream
    # of VALU slots it must issue, against the chip's issue rate) is reported beside it.
    roofline = {"bound": "hbm", "kernel": "kvssm_scan_kernel", "achieved": round(scan_gbps, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(scan_gbps / HBM_PEAK_GBPS, 4),
                "traffic": None if traffic is None else traffic["bytes_per_launch"],
                "algorithmic_bytes_per_launch": scan_bytes,
                "avg_launch_us": round(scan_ms * 1e3, 2)}
    scan_valu = {"achieved": round(scan_alu_tslots, 3), "peak": round(alu_peak, 3),
                 "unit": "T VALU-slot/s", "frac": round(scan_alu_tslots / alu_peak, 4),
                 "work_per_launch": f"{updates} state updates x {SLOTS_PER_UPDATE} slots"}
    line = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "extra_warmup_steps": extra_warmup,
        "data": "synthetic (seeded; x~N(0,1), weights~N(0,0.02^2), projections computed)",
        "config": {"workload": args.workload if with_block else cfg.name, "B": cfg.B, "n": cfg.n, "d_model": d, "heads": H,
                   "head_dim": hd, "N": cfg.N, "P": cfg.P, "L": cfg.L, "layer_idx": cfg.layer_idx,
                   "mask": "M_train+window" if mode == att.MASK_TRAIN else "M_test+window",
                   "chunking": cfg.chunking, "n_chunks": n},
        "roofline": roofline,
        "kernels_us": {"segmentation": round(seg_ms * 1e3, 2), "kvssm_scan": round(scan_ms * 1e3, 2),
                       "chunk_attn": round(attn_ms * 1e3, 2)},
        "flushed": flushed,
        "scan_valu": scan_valu,
        "attn_mfma": {"algorithmic_flop": attn_flop, "visible_pairs_per_head": pairs,
                      "TFLOPs": round(attn_tflops, 2),
                      "frac_of_2.5PF": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                      "traffic": None if attn_traffic is None else attn_traffic["bytes_per_launch"]},
    }
    mp = measured_peaks()
    if mp.get("copy_GBps"):
        mp["scan_frac_of_copy"] = round(scan_gbps / mp["copy_GBps"], 4)
    if mp.get("mfma_bf16_TFLOPs"):
        mp["attn_frac_of_mfma"] = round(attn_tflops / mp["mfma_bf16_TFLOPs"], 4)
    line["measured_peaks"] = mp
    if not args.no_cpu_baseline and not with_block:
        line["cpu_baseline"] = cpu_baseline(cfg, inp, T)
    print(json.dumps(line), flush=True)


def bench_decode(args):
    import torch
    import ssm_compressed_chunked_amd as att
    from workloads import DECODE_CONFIGS, make_decode

    cfg = DECODE_CONFIGS[args.workload]
    if args.batch is not None:
        cfg = cfg.with_(B=args.batch)
    n_bound = att.count_chunks([0, cfg.ctx], cfg.P, cfg.layer_idx)
    o = cfg.layer_idx % cfg.P
    if (cfg.ctx - o) % cfg.P != 0:
        raise SystemExit("decode bench expects a context that ends on a chunk boundary")
    steps = min(args.steps, cfg.steps)
    inp = make_decode(cfg, n_bound=n_bound, steps=cfg.steps, device="cuda")
    dtype = inp.kb.dtype
    cap = n_bound + cfg.steps // cfg.P + 2
    cache = att.DecodeCache(cfg.B, cfg.H, cfg.hd, cfg.N, cfg.P, cfg.L, cfg.layer_idx, cap, dtype,
                            inp.param, pos=cfg.ctx, n_bound=n_bound)
    cache.kb[:, :, :n_bound] = inp.kb
    cache.vb[:, :, :n_bound] = inp.vb
    cache.kw.copy_(inp.kw)
    cache.vw.copy_(inp.vw)
    del inp.kb, inp.vb
    a = {k: v.cuda() for k, v in inp.act.items()}
    out = torch.empty((cfg.B, cfg.H, cfg.hd), dtype=dtype, device="cuda")

    def run(n_steps):
        for s in range(n_steps):
            att.decode_step(cache, a["q"][s].view(cfg.B, cfg.H, cfg.hd), a["x"][s], a["dt_k"][s],
                            a["dt_v"][s], a["bm_k"][s], a["cm_k"][s], a["bm_v"][s], a["cm_v"][s], out=out)

    run(min(args.warmup, cfg.steps))
    torch.cuda.synchronize()
    cache.set_position(cfg.ctx, n_bound)
    t0 = time.perf_counter()
    run(cfg.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    keys = 0
    for s in range(cfg.steps):
        pos = cfg.ctx + s
        w = max(0, pos - cfg.L + 1)
        keys += att_ends_before(w, cfg.P, o) + (pos - w + 1)
    e = 2 if cfg.dtype == "bf16" else 4
    kv_bytes = keys * cfg.B * cfg.H * cfg.hd * 2 * e
    state_bytes = cfg.steps * 2 * 2 * cfg.B * cfg.d * cfg.N * 4
    gbps = (kv_bytes + state_bytes) / wall / 1e9
    traffic = (measured_traffic("decode_step", ["decode.hip", "common.h"], args.workload)
               if args.batch is None else None)
    line = {"metric": "decode tokens/s (boundary-state cache)", "value": round(cfg.B * cfg.steps / wall, 1),
            "unit": "tokens/s", "n_gpus": 1, "steps": cfg.steps, "warmup": args.warmup,
            "ms_per_step": round(wall * 1e3 / cfg.steps, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
            "config": {"workload": cfg.name, "B": cfg.B, "ctx": cfg.ctx, "d_model": cfg.d,
                       "heads": cfg.H, "head_dim": cfg.hd, "N": cfg.N, "P": cfg.P, "L": cfg.L},
            "roofline": {"bound": "hbm", "kernel": "decode step (update + split attention + combine)",
                         "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "traffic": None if traffic is None else traffic["bytes_per_launch"],
                         "algorithmic_bytes_per_step": round((kv_bytes + state_bytes) / cfg.steps)}}
    mp = measured_peaks(want_mfma=False)
    if mp.get("read_GBps"):
        mp["decode_frac_of_read"] = round(gbps / mp["read_GBps"], 4)
    line["measured_peaks"] = mp
    print(json.dumps(line), flush=True)


def bench_proj(args):
    """The layer's input projections at the prefill shape: Y = x W^T with x [16384, 2048] and
    the stacked weight W [3 d + 4 N, d] (q, dt_K, dt_V, Bm_K, Cm_K, Bm_V, Cm_V), bf16."""
    import torch
    import ssm_compressed_chunked_amd as att
    from workloads import PREFILL_CONFIGS, make_projection
    cfg = PREFILL_CONFIGS["prefill_bf16"]
    T, d, N = cfg.T, cfg.d, cfg.N
    inp = make_projection(T, d, N, seed=cfg.seed)
    x, w = inp.x.cuda(), inp.w.cuda()
    outs = [torch.empty((T, wd), dtype=torch.bfloat16, device="cuda") for wd in inp.widths]
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        att.input_proj(x, w, inp.widths, outs=outs, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        att.input_proj(x, w, inp.widths, outs=outs, stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        att.input_proj(x, w, inp.widths, outs=outs, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    n_out = sum(inp.widths)
    flop = 2.0 * T * d * n_out
    tflops = flop / (us * 1e-6) / 1e12
    traffic = measured_traffic("proj_gemm_kernel", ["proj_gemm.hip", "common.h"], args.workload)
    mp = measured_peaks(want_copy=False)
    if mp.get("mfma_bf16_TFLOPs"):
        mp["proj_frac_of_mfma"] = round(tflops / mp["mfma_bf16_TFLOPs"], 4)
    print(json.dumps({
        "metric": "input projections TFLOP/s (x W^T, bf16)", "value": round(tflops, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "proj_bf16", "T": T, "d": d, "n_out": n_out,
                   "segments": inp.widths},
        "roofline": {"bound": "mfma", "kernel": "proj_gemm_kernel + proj_tail_kernel (one call)", "achieved": round(tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "avg_launch_us": round(us, 2)},
        "measured_peaks": mp}), flush=True)


def bench_layer(args):
    """One layer from its input x at the prefill shape: the input projections (x W^T on the
    matrix cores) followed by the KV-SSM forward (segmentation, scan, attention)."""
    import torch
    import ssm_compressed_chunked_amd as att
    from workloads import PREFILL_CONFIGS, make_prefill, make_projection
    cfg = PREFILL_CONFIGS["prefill_bf16"]
    T, d, H, hd, N = cfg.T, cfg.d, cfg.H, cfg.hd, cfg.N
    pj = make_projection(T, d, N, seed=cfg.seed)
    par = {k: v.cuda() for k, v in make_prefill(cfg.with_(B=1, n=256)).param.items()}
    x, w = pj.x.cuda(), pj.w.cuda()
    seq_cu_h = (np.arange(cfg.B + 1) * cfg.n).astype(np.int32)
    seq_cu = torch.from_numpy(seq_cu_h).cuda()
    n = att.count_chunks(seq_cu_h, cfg.P, cfg.layer_idx)
    widths = pj.widths
    proj = [torch.empty((T, wd), dtype=torch.bfloat16, device="cuda") for wd in widths]
    q, dtk, dtv, bmk, cmk, bmv, cmv = proj
    chunk_cu = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    token_chunk = torch.empty(T, dtype=torch.int32, device="cuda")
    is_end = torch.empty(T, dtype=torch.uint8, device="cuda")
    y_k, y_v = torch.empty_like(x), torch.empty_like(x)
    kb = torch.empty((n, d), dtype=x.dtype, device="cuda")
    vb = torch.empty_like(kb)
    out = torch.empty((T, H, hd), dtype=x.dtype, device="cuda")
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        att.input_proj(x, w, widths, outs=proj, stream=stream)
        att.chunk_boundaries(seq_cu, T, cfg.P, cfg.layer_idx, n, chunk_cu, token_chunk, is_end,
                             stream=stream)
        att.kvssm_scan(x, dtk, dtv, bmk, cmk, bmv, cmv, par["A_k"], par["A_v"], par["D_k"],
                       par["D_v"], par["bias_k"], par["bias_v"], chunk_cu, y_k=y_k, y_v=y_v,
                       kb=kb, vb=vb, stream=stream)
        att.chunk_attn_fwd(q.view(T, H, hd), y_k.view(T, H, hd), y_v.view(T, H, hd),
                           kb.view(n, H, hd), vb.view(n, H, hd), seq_cu, chunk_cu, token_chunk,
                           cfg.n, cfg.L, att.MASK_TEST, out=out, lse=lse, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(json.dumps({
        "metric": "tokens/sec, input projections + KV-SSM forward", "value": round(T * args.steps / wall, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "layer_bf16", "B": cfg.B, "n": cfg.n, "d_model": d, "heads": H,
                   "head_dim": hd, "N": N, "P": cfg.P, "L": cfg.L}}), flush=True)


def cpu_baseline_train(cfg, inp, dout, T_full, scan_budget_s=3.0, attn_budget_s=8.0):
    """The oracle's forward and backward on a bounded sample of the training workload: both
    scans and their backward over a whole-chunk prefix of sequence 0 (all channels), and the
    attention forward and backward of sequence 0 for as many heads as fit in about
    attn_budget_s; scaled to the whole batch like cpu_baseline."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    f = {k: inp.f64(k) for k in list(inp.act) + list(inp.param)}
    chunk_cu, tc, ie = oracle.segment(inp.seq_cu, cfg.P, cfg.layer_idx)
    s0, s1 = int(inp.seq_cu[0]), int(inp.seq_cu[1])
    rng = np.random.default_rng(0)

    def scan_prefix(n_tok):
        n_tok = int(chunk_cu[np.searchsorted(chunk_cu, min(n_tok, s1))])
        cu = chunk_cu[chunk_cu <= n_tok]
        t0 = time.perf_counter()
        for tag in ("k", "v"):
            args = (f["x"][:n_tok], f[f"dt_{tag}"][:n_tok], f[f"bias_{tag}"], f[f"A_{tag}"],
                    f[f"bm_{tag}"][:n_tok], f[f"cm_{tag}"][:n_tok], f[f"D_{tag}"], cu)
            oracle.selective_scan(*args)
            oracle.selective_scan_backward(*args, rng.standard_normal((n_tok, cfg.d)))
        return n_tok, time.perf_counter() - t0

    n_scan, t_scan = scan_prefix(256)
    if t_scan < scan_budget_s and n_scan < s1:
        n_scan, t_scan = scan_prefix(int(n_scan * scan_budget_s / max(t_scan, 1e-3)))
    H, hd = cfg.H, cfg.hd
    t_attn, heads = 0.0, 0
    n = s1 - s0
    while heads < H and t_attn < attn_budget_s:
        q = f["q"][s0:s1].reshape(-1, H, hd)[:, heads:heads + 1]
        k = rng.standard_normal((n, 1, hd))
        v = rng.standard_normal((n, 1, hd))
        g = dout[s0:s1, heads:heads + 1].to(dtype=__import__("torch").float64).numpy()
        t0 = time.perf_counter()
        oracle.chunk_attention(q, k, v, [0, n], tc[s0:s1] - tc[s0], ie[s0:s1], cfg.L, cfg.mode)
        oracle.chunk_attention_backward(q, k, v, [0, n], tc[s0:s1] - tc[s0], ie[s0:s1], cfg.L,
                                        cfg.mode, g)
        t_attn += time.perf_counter() - t0
        heads += 1
    n_pairs = (len(inp.seq_cu) - 1) * H
    est = t_scan * (T_full / n_scan) + t_attn / heads * n_pairs
    return {"value": T_full / est, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"oracle forward + backward of both scans over tokens 0..{n_scan - 1} of sequence 0 "
                       f"(all {cfg.d} channels: {t_scan:.2f} s) scaled by {T_full / n_scan:.2f}; oracle attention "
                       f"forward + backward of sequence 0, heads 0..{heads - 1} ({n} rows each: {t_attn:.2f} s) "
                       f"scaled to {n_pairs} sequence-head pairs; estimated {est:.1f} s per step")}


# minimal VALU slots per state update of the scan backward: the forward recompute (decay
# multiply, v_exp_f32, input multiply, state FMA), g h for dCm, and the reverse step (dh FMA,
# dBm multiply, du FMA, decay recomputed (multiply and v_exp_f32), dh e, w = dh e h_prev, dA and
# ddelta FMAs), plus one add each for the channel sums of dCm and dBm
SLOTS_PER_UPDATE_BWD = (3.0 + EXP_SLOTS) + 1.0 + (8.0 + EXP_SLOTS) + 2.0


def bench_train(args):
    """One training step of the KV-SSM path at the M_train workload (bf16, B=4, n=2048,
    d=1024, 16 heads x 64, N=16, P=8, L=64, layer 3): segmentation, both scans, the attention
    with its LSE, then the attention backward and the scan backward for a seeded output
    gradient. Phase times come from HIP events on the launch stream."""
    import torch
    import ssm_compressed_chunked_amd as att
    from ssm_compressed_chunked_amd.pipeline import prefill_forward
    from workloads import PREFILL_CONFIGS, make_output_grad, make_prefill
    cfg = PREFILL_CONFIGS["train_bf16"]
    T, d, H, hd, N = cfg.T, cfg.d, cfg.H, cfg.hd, cfg.N
    inp = make_prefill(cfg)
    act = {k: v.cuda() for k, v in inp.act.items()}
    par = {k: v.cuda() for k, v in inp.param.items()}
    act["seq_cu"] = torch.from_numpy(inp.seq_cu).cuda()
    dout_h = make_output_grad((T, H, hd), cfg.dtype, seed=42)
    dout = dout_h.cuda()
    stream = torch.cuda.current_stream()
    ws = att.chunk_attn_bwd_workspace(T, H, hd, att.count_chunks(inp.seq_cu, cfg.P, cfg.layer_idx),
                                      act["q"].dtype)

    def step(ev=None):
        stream = torch.cuda.current_stream()
        if ev is not None:
            ev[0].record(stream)
        res = prefill_forward(act, par, inp.seq_cu, H, hd, cfg.P, cfg.layer_idx, cfg.L,
                              att.MASK_TRAIN, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        lay, sc, n = res["layout"], res["scan"], res["layout"].n_chunks
        ga = att.chunk_attn_bwd(act["q"].view(T, H, hd), sc["y_k"].view(T, H, hd),
                                sc["y_v"].view(T, H, hd), sc["kb"].view(n, H, hd),
                                sc["vb"].view(n, H, hd), res["seq_cu"], lay.chunk_cu,
                                lay.token_chunk, res["max_len"], cfg.L, att.MASK_TRAIN,
                                res["out"], res["lse"], dout, workspace=ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        att.kvssm_scan_bwd(act["x"], act["dt_k"], act["dt_v"], act["bm_k"], act["cm_k"],
                           act["bm_v"], act["cm_v"], par["A_k"], par["A_v"], par["D_k"],
                           par["D_v"], par["bias_k"], par["bias_v"], lay.chunk_cu,
                           ga["dk"].view(T, d), ga["dv"].view(T, d), gkb=ga["dkb"].view(n, d),
                           gvb=ga["dvb"].view(n, d), stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    # The same step captured once as a HIP graph (the step makes about twenty allocations and a
    # dozen launches through Python, which can take as long as the GPU work) and replayed K
    # times; tests/test_gpu_graph.py checks the replays against eager steps.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    for _ in range(min(args.warmup, 50)):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    fwd_ms, abwd_ms, sbwd_ms = (float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
                                for i in range(3))
    updates = 2 * T * d * N
    alu_peak = VALU_SLOTS_PER_S / 1e12
    ach = SLOTS_PER_UPDATE_BWD * updates / (sbwd_ms * 1e-3) / 1e12
    traffic = measured_traffic("kvssm_scan_bwd_kernel", ["kvssm_scan_bwd.hip", "common.h"], args.workload)
    line = {
        "metric": "tokens/sec, KV-SSM forward + backward (training step)",
        "value": round(T * args.steps / wall, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "train_step_bf16", "B": cfg.B, "n": cfg.n, "d_model": d,
                   "heads": H, "head_dim": hd, "N": N, "P": cfg.P, "L": cfg.L,
                   "layer_idx": cfg.layer_idx, "mask": "M_train+window"},
        "roofline": {"bound": "alu", "kernel": "kvssm_scan_bwd_kernel", "achieved": round(ach, 3),
                     "peak": round(alu_peak, 3), "unit": "T VALU-slot/s", "frac": round(ach / alu_peak, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "work_per_launch": f"{updates} state updates x {SLOTS_PER_UPDATE_BWD} slots",
                     "avg_launch_us": round(sbwd_ms * 1e3, 2)},
        "phases_us": {"forward": round(fwd_ms * 1e3, 2), "attention_backward": round(abwd_ms * 1e3, 2),
                      "scan_backward": round(sbwd_ms * 1e3, 2)},
        "timing": "K replays of the step captured as a HIP graph",
        "eager_ms_per_step": round(eager_wall * 1e3 / args.steps, 4),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_train(cfg, inp, dout_h, T)
    print(json.dumps(line), flush=True)


def measured_peaks(want_copy=True, want_mfma=True) -> dict:
    """The denominators measured on this machine, reported beside the vendor peaks: the bandwidth
    of a plain 512 MiB device copy (read plus write bytes over the event-timed copy) and of a
    read-only stream over 2 GiB (the probe library's streaming-read kernel), and the
    bf16 matrix-core rate of the issue probe's MFMA loop (v_mfma_f32_32x32x16_bf16 chains,
    two waves on every SIMD, 32 768 FLOP per instruction) over its event-timed launch."""
    import ctypes
    import torch
    out = {}
    stream = torch.cuda.current_stream()
    if want_copy:
        nbytes = 512 << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        out["copy_GBps"] = round(2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del src, dst
        # a read-only stream over 2 GiB (the probe library's streaming-read kernel): the
        # denominator of kernels that mostly read
        if os.path.exists(PROBE_LIB):
            lib = ctypes.CDLL(PROBE_LIB)
            lib.attamba_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
            big = torch.ones(4 * nbytes // 4, dtype=torch.float32, device="cuda")
            blocks = torch.cuda.get_device_properties(0).multi_processor_count * 8
            sink = torch.empty(256 * blocks, dtype=torch.float32, device="cuda")

            def read_once():
                rc = lib.attamba_probe_read_stream(big.data_ptr(), 4 * nbytes, sink.data_ptr(),
                                                   blocks, ctypes.c_void_p(stream.cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"read-stream probe failed ({rc})")
            for _ in range(3):
                read_once()
            e0.record(stream)
            for _ in range(reps):
                read_once()
            e1.record(stream)
            torch.cuda.synchronize()
            out["read_GBps"] = round(4 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
            del big, sink
    if want_mfma:
        if not os.path.exists(PROBE_LIB):
            out["mfma_bf16_TFLOPs"] = None
            out["mfma_note"] = f"{os.path.basename(PROBE_LIB)} not built"
        else:
            lib = ctypes.CDLL(PROBE_LIB)
            lib.attamba_probe_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p]
            lib.attamba_probe_ops_per_iter.argtypes = [ctypes.c_int]
            op, W = 4, 2                       # the MFMA loop; two waves per SIMD
            blocks = torch.cuda.get_device_properties(0).multi_processor_count * W
            vin = torch.full((192,), 0.75, dtype=torch.float32, device="cuda")
            rows = (ctypes.c_float * 32)(*([0.5] * 32))
            probe_out = torch.zeros(6 * 4 * blocks, dtype=torch.int64, device="cuda")
            sink = torch.empty(256 * blocks, dtype=torch.float32, device="cuda")
            iters = PROBE_ITERS[op]

            def launch():
                rc = lib.attamba_probe_issue(op, blocks, iters, 0.3, vin.data_ptr(), rows,
                                             probe_out.data_ptr(), sink.data_ptr(),
                                             ctypes.c_void_p(stream.cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"probe launch failed ({rc})")
            for _ in range(2):
                launch()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 3
            e0.record(stream)
            for _ in range(reps):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            mfmas = blocks * 4 * lib.attamba_probe_ops_per_iter(op) * iters * reps
            out["mfma_bf16_TFLOPs"] = round(mfmas * 32768.0 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    return out


def bench_copy(args):
    """A plain device copy of 512 MiB: the reference point that scales rocprofv3's FETCH_SIZE
    and WRITE_SIZE counters to bytes (the copy moves exactly 512 MiB each way per launch)."""
    import torch
    nbytes = 512 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gbps = 2 * nbytes * args.steps / wall / 1e9
    print(json.dumps({"metric": "device copy", "bytes_each_way": nbytes, "steps": args.steps,
                      "GBps_read_plus_write": round(gbps, 1)}), flush=True)


PROBE_OPS = {0: "v_fma_f32 VOP3 (VGPR operands)", 1: "v_fma_f32 VOP3 (one SGPR operand)",
             2: "v_mul_f32 VOP2 (VGPR operands)", 3: "v_exp_f32 VOP3 (negated source)",
             4: "v_mfma_f32_32x32x16_bf16",
             5: "scan state update (v_mul, v_exp, v_mul with SGPR, v_fmac, v_fmac with SGPR)",
             6: "v_fmac_f32 VOP2 (VGPR operands)", 7: "v_fmac_f32 VOP2 (one SGPR operand)",
             8: "v_add_f32 VOP2 (VGPR operands)", 9: "v_exp_f32 VOP1 + v_mul_f32 VOP2 (VGPR) pair",
             10: "v_fmamk_f32 VOP2 (literal operand)", 11: "v_cvt_pk_bf16_f32 + v_perm_b32 (two VOP3)",
             12: "v_dot2 bf16 pairs, f32 accumulator",
             13: "v_exp_f32 VOP3 + independent v_fmac_f32 VOP2 pair",
             14: "v_mfma_f32_32x32x16_bf16 + 8 independent v_fmac_f32 VOP2 (per MFMA)",
             15: "v_mfma_f32_32x32x16_bf16 + 8 independent v_exp_f32 (per MFMA)",
             16: "v_mfma_f32_32x32x16_bf16 + 8 independent v_fma_f32 VOP3 (per MFMA)",
             17: "v_mul_f32 VOP2 with a DPP row-broadcast operand",
             18: "v_fmac_f32 VOP2 with a DPP row-broadcast operand",
             19: "scan state update with DPP row-broadcast row operands (v_mul, v_exp, v_mul_dpp, v_fmac, v_fmac_dpp)"}
PROBE_ITERS = {0: 20000, 1: 20000, 2: 20000, 3: 8000, 4: 2000, 5: 1000, 6: 20000, 7: 20000,
               8: 20000, 9: 8000, 10: 20000, 11: 20000, 12: 20000, 13: 8000, 14: 2000, 15: 2000,
               16: 2000, 17: 20000, 18: 20000, 19: 1000}


def probe_per_simd(rec, ops_per_wave, W):
    """rec: one row per wave (clock before, after, real time before, after, HW_ID, XCC_ID).
    Groups the waves by SIMD (XCC, shader engine, shader array, CU, SIMD: HW_ID bits 4..15),
    keeps the SIMDs that held exactly W waves that all ran side by side (every start before
    every end, on that SIMD's shader clock), and returns the median over them of the SIMD's busy
    span divided by the instructions its waves issued."""
    rec = rec.astype(np.int64)
    key = (rec[:, 5] & 0xF) * 4096 + ((rec[:, 4] >> 4) & 0xFFF)
    spans, counts = [], {}
    for k in np.unique(key):
        g = rec[key == k]
        counts[len(g)] = counts.get(len(g), 0) + 1
        if len(g) == W and g[:, 0].max() < g[:, 1].min():
            spans.append((g[:, 1].max() - g[:, 0].min()) / (W * ops_per_wave))
    dclk = (rec[:, 1] - rec[:, 0]).astype(np.float64)
    dreal = (rec[:, 3] - rec[:, 2]).astype(np.float64)
    return {"clocks_per_instr_per_simd": round(float(np.median(spans)), 3) if spans else None,
            "simds_used": len(spans), "waves_per_simd_histogram": {str(k): v for k, v in sorted(counts.items())},
            "clock_GHz": float(np.median(dclk / (dreal * 10.0)))}


def bench_valu_issue(args):
    """Issue cost of the instructions the scan and the attention are made of: shader clocks per
    wave64 instruction per SIMD, with W = 1, 2, 4, 8 waves per SIMD, each wave running
    independent chains (libattamba_probe.so, read from the kernel's own s_memtime clock). Also
    the scan's whole state update in FMA slots, the figure its instruction-issue roofline uses."""
    import ctypes
    import torch
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is missing: run the build first")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.attamba_probe_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.attamba_probe_ops_per_iter.argtypes = [ctypes.c_int]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(0)
    vin = torch.from_numpy(np.concatenate([rng.uniform(0.5, 1.0, 128), np.full(64, 0.3)])
                           .astype(np.float32)).cuda()
    rows = (ctypes.c_float * 32)(*rng.uniform(-1.0, 1.0, 32).astype(np.float32).tolist())
    stream = torch.cuda.current_stream()
    res, clock_ghz = {}, []
    for op, name in PROBE_OPS.items():
        per_iter = lib.attamba_probe_ops_per_iter(op)
        res[name] = {}
        for W in (1, 2, 4, 8):
            blocks = n_cu * W            # 4-wave workgroups: W waves on every SIMD
            out = torch.zeros(6 * 4 * blocks, dtype=torch.int64, device="cuda")
            sink = torch.empty(256 * blocks, dtype=torch.float32, device="cuda")
            for _ in range(2):           # the first run ramps the clocks
                rc = lib.attamba_probe_issue(op, blocks, PROBE_ITERS[op], 0.3, vin.data_ptr(),
                                             rows, out.data_ptr(), sink.data_ptr(),
                                             ctypes.c_void_p(stream.cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"probe launch failed ({rc})")
                torch.cuda.synchronize()
            r = probe_per_simd(out.cpu().numpy().reshape(-1, 6), per_iter * PROBE_ITERS[op], W)
            clock_ghz.append(r.pop("clock_GHz"))
            res[name][f"W{W}"] = r
    def clk(op, w="W4"):
        return res[PROBE_OPS[op]][w]["clocks_per_instr_per_simd"]

    def ratio(a, b):
        return None if a is None or b is None else round(a / b, 3)

    fma = clk(0)
    derived = {
        "fma_vop3_clocks_W4": fma,
        "fmac_vop2_clocks_W4": clk(6),
        "mul_vop2_clocks_W4": clk(2),
        "exp_vop1_clocks_W4": None if clk(9) is None or clk(2) is None else round(clk(9) - clk(2), 3),
        "fmamk_literal_clocks_W4": clk(10),
        "cvt_pk_bf16_clocks_W4": clk(11),
        "dot2_bf16_clocks_W4": clk(12),
        "exp_plus_fmac_pair_clocks_W4": clk(13),
        "mfma_plus_8_fmac_clocks_W1": clk(14, "W1"),
        "mfma_plus_8_fmac_clocks_W2": clk(14, "W2"),
        "mfma_plus_8_exp_clocks_W2": clk(15, "W2"),
        "mfma_plus_8_vop3_fma_clocks_W2": clk(16, "W2"),
        "sgpr_operand_fma_slots_W4": ratio(clk(1), fma),
        "exp_vop3_slots_W4": ratio(clk(3), fma),
        "scan_update_clocks_W4": clk(5),
        "mul_dpp_clocks_W4": clk(17),
        "fmac_dpp_clocks_W4": clk(18),
        "scan_update_dpp_clocks_W2": clk(19, "W2"),
        "scan_update_clocks_W2": clk(5, "W2"),
        "scan_update_slots_W4": ratio(clk(5), fma),
        "mfma_32x32x16_clocks_W4": clk(4),
        "slots_per_update_used_by_prefill_line": SLOTS_PER_UPDATE,
    }
    print(json.dumps({"metric": "issue clocks per wave64 instruction per SIMD", "unit": "clocks",
                      "n_gpus": 1, "data": "synthetic", "config": {"workload": "valu_issue",
                      "compute_units": n_cu, "waves_per_simd": [1, 2, 4, 8]},
                      "shader_clock_GHz": round(float(np.median(clock_ghz)), 3),
                      "results": res, "derived": derived}), flush=True)


def att_ends_before(x, P, o):
    if x <= 0:
        return 0
    if o == 0:
        return x // P
    return (x - o) // P + 1 if x >= o else 0


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path would "
              "shard by batch, head or sequence, with no exchange beyond one all-gather of the "
              "boundary states and a halo of the last L keys)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.workload == "copy":
        bench_copy(args)
    elif args.workload == "valu_issue":
        bench_valu_issue(args)
    elif args.workload == "proj_bf16":
        bench_proj(args)
    elif args.workload == "layer_bf16":
        bench_layer(args)
    elif args.workload == "train_step_bf16":
        bench_train(args)
    elif args.workload.startswith("decode"):
        bench_decode(args)
    else:
        bench_prefill(args)


if __name__ == "__main__":
    main()
