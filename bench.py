#!/usr/bin/env python
"""Benchmark of the Dory token forward on one MI355X.

Workloads (``--config``), all on seeded synthetic bf16 Dory-2B weights and
seeded tokens:

* ``decode`` (default): batch-1 decode at context 4096, loops 4, last_loop, fp32
  cache.  Set-up: a 4096-token prompt in calls of 512 through the prefill path.
  A step is one decode token: one call of the whole forward (input block, 4
  passes of the recurrent block, output block, head).
* ``q8``: the same decode with the q8_2f cache, full_window 8192, at context
  32768 (prompt of 32768 tokens in calls of 512).
* ``prefill``: per_loop, loops 8; a step is one 8192-token prompt in 16 calls
  of 512 rows (logits of the last call only), the cache reset before each.
* ``batch``: 64 sequences, each prefilled to 8192 tokens (last_loop, loops 4);
  a step is one batched decode call with one token per sequence and a loop
  count per (sequence, step) drawn uniformly from 1..16.
* ``gate``: the ``decode`` workload with the confidence-gated early exit on
  (dory.rs ``Gate::Conf``, threshold ``--gate``, 0.7 by default): every token
  runs one or two passes as the gate decides; a token that reads out waits for
  its read-out on the host, so the host clock times the steps.  No CPU
  baseline (the oracle's decode sample is not gated).

Timed: ``--steps`` steps after ``--warmup`` untimed ones, bracketed by device
synchronisation and HIP events on the stream the library launches on.  One JSON
line on stdout; progress on stderr.

The roofline entry is for the workload's dominant kernel, launched on its own
(dory_stage_bench) over the sub-layers' weights in turn on the same stream and
timed with HIP events: the gate|up GEMV (decode, q8), the gate|up GEMM at 512
rows (prefill), decode attention over the batch's 64 rows (batch).  The CPU
baseline is the oracle on the host cores on a bounded sample of the workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
METRIC = "decode tokens/s (all loops) + achieved HBM GB/s, 1×MI355X, Dory-2B ctx 4096"
CSRC = os.path.join(ROOT, "looped_normalized_gpt_amd", "csrc")
TRAFFIC = {  # committed counter runs: file, kernel source it was taken on (with the shared headers)
    "decode": ("gemv_gateup_2b_traffic.json", "gemv.hip"),
    "q8": ("gemv_gateup_2b_traffic.json", "gemv.hip"),
    "prefill": ("gemm_gateup_2b_traffic.json", "gemm.hip"),
    "batch": ("attn_dec_batch64_traffic.json", "attn.hip"),
}
TRAFFIC_HEADERS = ("device.h", "internal.h")
# the profiler's mean duration of each workload's roofline kernel, from the
# committed rocprofv3 runs of this script (profiles/*_kernels.md)
ROCPROF = "roofline_rocprof.json"


def sources_digest(src):
    """sha256 over a kernel source and the headers every kernel includes."""
    h = hashlib.sha256()
    for f in (src,) + TRAFFIC_HEADERS:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def n_ord(cfg):
    return sum(1 for ch in cfg["pattern"] if ch != "-")


def kv_row_bytes(cfg):
    """Bytes of one cached position of one layer (all kv heads, K and V)."""
    nk, hd = cfg["nk"], cfg["hd"]
    if cfg.get("kv_encoding", "f32") == "q8_2f":
        return nk * (hd + 4 * ((hd + 31) // 32) + hd + 4)
    return nk * hd * 4 * 2


def visible(cfg, kind, pos):
    win = cfg["window"] if kind == "S" else (cfg.get("full_window") or 1 << 60)
    return min(win, pos + 1)


def sublayer_weight_bytes(cfg, kind):
    H, F, Q, KV = cfg["hidden"], cfg["ffn"], cfg["nh"] * cfg["hd"], cfg["nk"] * cfg["hd"]
    wb = 2 if cfg["weight_dtype"] == "bf16" else 4
    if kind == "-":
        return 3 * F * H * wb + (2 * F + H) * 4
    return (2 * Q + 2 * KV) * H * wb + H * Q * wb + (2 * Q + H) * 4


def passes(cfg, loops):
    n_in, n_rec, n_out = cfg["n_in"], cfg["n_rec"], cfg["n_out"]
    return list(range(n_in)) + \
           [n_in + j for _ in range(loops) for j in range(n_rec)] + \
           [n_in + n_rec + j for j in range(n_out)]


def token_bytes(cfg, pos, loops):
    """Algorithmic HBM bytes of one batch-1 decode token at position pos: every
    weight byte once per sub-layer pass, every visible cache row once, the scale
    vectors, the cache row written, the head."""
    H, V = cfg["hidden"], cfg["vocab"]
    wb = 2 if cfg["weight_dtype"] == "bf16" else 4
    rb = kv_row_bytes(cfg)
    total = 0
    for li in passes(cfg, loops):
        kind = cfg["pattern"][li]
        total += sublayer_weight_bytes(cfg, kind)
        if kind != "-":
            total += visible(cfg, kind, pos) * rb + rb
    return total + V * H * wb + V * 4


def batch_step_bytes(cfg, pos, loops_row):
    """Algorithmic bytes of one batched decode step: the weights of every
    sub-layer pass once (the recurrent block once per loop of the longest row),
    and per row its own visible cache rows and written row; the head once."""
    H, V = cfg["hidden"], cfg["vocab"]
    wb = 2 if cfg["weight_dtype"] == "bf16" else 4
    rb = kv_row_bytes(cfg)
    total = sum(sublayer_weight_bytes(cfg, cfg["pattern"][li]) for li in passes(cfg, max(loops_row)))
    for L in loops_row:
        for li in passes(cfg, L):
            kind = cfg["pattern"][li]
            if kind != "-":
                total += visible(cfg, kind, pos) * rb + rb
    return total + V * H * wb + V * 4 * len(loops_row)


def prefill_flops(cfg, T, loops):
    """Projection GEMM flops of one T-row call (2 flop per multiply-add)."""
    H, F, Q, KV, V = cfg["hidden"], cfg["ffn"], cfg["nh"] * cfg["hd"], cfg["nk"] * cfg["hd"], cfg["vocab"]
    f = 0
    for li in passes(cfg, loops):
        if cfg["pattern"][li] == "-":
            f += 2 * T * 3 * F * H
        else:
            f += 2 * T * ((2 * Q + 2 * KV) * H + H * Q)
    return f


def traffic_entry(mode):
    """HBM bytes per launch of the dominant kernel from the committed counter
    runs, or None when there are none or the kernel source or the headers it
    includes changed since."""
    fname, src = TRAFFIC[mode]
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("sources_sha256") != sources_digest(src):
        return None
    return t.get("bytes_per_launch")


def rocprof_entry(mode):
    """The profiler's mean launch time of the workload's roofline kernel (its
    stage-benchmark launches in a rocprofv3 --kernel-trace run of this script),
    or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", ROCPROF)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f).get(mode)
    if not t or t.get("sources_sha256") != sources_digest(TRAFFIC[mode][1]):
        return None
    return {"us_per_launch": t["us_per_launch"], "launches": t["launches"], "summary": t["summary"]}


def measured_peaks():
    """Practical peaks of this GPU (dory_probe): one streaming read of a 2 GiB
    buffer (8x the 256 MB Infinity Cache) with 16-byte nontemporal loads, the
    same read of 46 MB slices rotating over the buffer (the size of the largest
    decode GEMV, ramp and drain included), and a bf16 MFMA loop from registers
    (v_mfma_f32_32x32x16_bf16, two waves per SIMD)."""
    import torch
    from looped_normalized_gpt_amd import dory
    stream = torch.cuda.current_stream()
    sink = torch.zeros(16, dtype=torch.float32, device="cuda")
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    slice_b = 46137344
    slices = [buf[i * slice_b:(i + 1) * slice_b] for i in range(8)]

    def rate(launch, reps):
        for i in range(3):
            launch(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        work = sum(launch(i) for i in range(reps))
        e1.record(stream)
        torch.cuda.synchronize()
        return work / (e0.elapsed_time(e1) * 1e-3)

    big = rate(lambda i: dory.probe("stream", buf=buf, sink=sink, stream=stream), 10)
    small = rate(lambda i: dory.probe("stream", buf=slices[i % 8], sink=sink, stream=stream), 64)
    mfma = rate(lambda i: dory.probe("mfma", iters=20000, sink=sink, stream=stream), 5)
    del buf, slices
    torch.cuda.empty_cache()
    return {"hbm_gbs": round(big / 1e9, 1), "hbm_gbs_46MB_reads": round(small / 1e9, 1),
            "bf16_mfma_tflops": round(mfma / 1e12, 1),
            "how": "dory_probe: one 2 GiB streaming read (16-byte nontemporal loads), 46 MB reads rotating over "
                   "8 slices, and a loop of v_mfma_f32_32x32x16_bf16 from registers; HIP events"}


def launch_floor(cfg, ctx, loops, sliding_merged=True):
    """A measured ceiling for a decode token made of one kernel per step: the
    probe's streaming read (dory_probe) timed back to back at the size of each
    kernel of the token (each projection's weights, each attention's cache rows,
    a 64 KB read for each split merge launched on its own: the full layers', and
    the sliding layers' unless they merge inside the attention kernel), buffers
    rotating past the Infinity Cache, summed over the token's kernels.  What a
    kernel costs beyond its read at that size is its own excess."""
    import torch
    from looped_normalized_gpt_amd import dory
    stream = torch.cuda.current_stream()
    sink = torch.zeros(16, dtype=torch.float32, device="cuda")
    H, F, Q, KV, V = cfg["hidden"], cfg["ffn"], cfg["nh"] * cfg["hd"], cfg["nk"] * cfg["hd"], cfg["vocab"]
    rb = kv_row_bytes(cfg)
    sizes = {"qkvg GEMV": (2 * Q + 2 * KV) * H * 2, "O GEMV": H * Q * 2, "gate|up GEMV": 2 * F * H * 2,
             "down GEMV": H * F * 2, "head GEMV": V * H * 2,
             "sliding attention": visible(cfg, "S", ctx) * rb, "full attention": visible(cfg, "*", ctx) * rb,
             "merge": 65536}
    pool = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    us = {}
    reps = 32
    for name, b in sizes.items():
        b = (b + 255) // 256 * 256
        nbuf = max(2, min(64, (512 << 20) // b))
        views = [pool[(i * b) % ((1 << 30) - b):][:b] for i in range(nbuf)]
        for i in range(4):
            dory.probe("stream", buf=views[i % nbuf], sink=sink, stream=stream)
        torch.cuda.synchronize()
        # the reads captured back to back in one HIP graph, as the decode
        # token's kernels are (host launches would be the bound for small ones)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            for i in range(reps):
                dory.probe("stream", buf=views[i % nbuf], sink=sink, stream=cs)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(4):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us[name] = round(e0.elapsed_time(e1) * 1e3 / (4 * reps), 2)
        del g
    del pool
    torch.cuda.empty_cache()
    n_attn = sum(1 for ch in cfg["pattern"] if ch != "-")
    per = {"qkvg GEMV": 0, "O GEMV": 0, "gate|up GEMV": 0, "down GEMV": 0, "sliding attention": 0,
           "full attention": 0, "merge": 0, "head GEMV": 1}
    for li in passes(cfg, loops):
        kind = cfg["pattern"][li]
        if kind == "-":
            per["gate|up GEMV"] += 1
            per["down GEMV"] += 1
        else:
            per["qkvg GEMV"] += 1
            per["O GEMV"] += 1
            if kind != "S" or not sliding_merged:
                per["merge"] += 1
            per["sliding attention" if kind == "S" else "full attention"] += 1
    floor = sum(us[k] * n for k, n in per.items())
    return {"us_per_read": us, "launches_per_token": per, "token_floor_us": round(floor, 1),
            "token_floor_tokens_per_s": round(1e6 / floor, 1),
            "how": "dory_probe streaming reads of each kernel's byte count, 32 back to back in a captured HIP "
                   "graph per size, buffers rotating over 512 MB; summed over the kernels of one token"}


def roofline_extra(roof, mode, peaks):
    """Adds the fraction against the measured peak and the profiler's launch
    time to a roofline entry."""
    meas = peaks["hbm_gbs"] if roof["bound"] == "hbm" else peaks["bf16_mfma_tflops"]
    roof["measured_peak"] = meas
    roof["frac_of_measured_peak"] = round(roof["achieved"] / meas, 4)
    rp = rocprof_entry(mode)
    roof["rocprof"] = rp
    if rp:
        work = roof.get("bytes_per_launch") or roof.get("flops_per_launch")
        scale = 1e9 if roof["bound"] == "hbm" else 1e12
        roof["achieved_at_rocprof_time"] = round(work / (rp["us_per_launch"] * 1e-6) / scale, 1)
    return roof


def vendor_gemm_tflops(M, N, K, reps=100):
    """Reference point, not part of the path: torch.mm (hipBLASLt) on an
    M x N x K bf16 product with a contiguous [K][N] right operand, rotating over
    8 weight copies so they stream from HBM as the library's weights do."""
    import torch
    A = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
    Ws = [torch.randn(K, N, device="cuda", dtype=torch.bfloat16) for _ in range(8)]
    for i in range(16):
        torch.mm(A, Ws[i % 8])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        torch.mm(A, Ws[i % 8])
    e1.record()
    torch.cuda.synchronize()
    return 2 * M * N * K / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e12


def vendor_gemv_us(N, K, reps=200):
    """Reference point, not part of the path: torch.mv (the vendor GEMV) of a
    bf16 [N][K] matrix by a bf16 vector, rotating over 8 matrices so each launch
    streams its weights from HBM."""
    import torch
    x = torch.randn(K, device="cuda", dtype=torch.bfloat16)
    Ws = [torch.randn(N, K, device="cuda", dtype=torch.bfloat16) for _ in range(8)]
    for i in range(16):
        torch.mv(Ws[i % 8], x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        torch.mv(Ws[i % 8], x)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del Ws
    return us


def time_stage(dory, g, stage, reps, stream):
    import torch
    dory.stage_bench(g, stage, min(reps, 40), stream)   # warm
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    dory.stage_bench(g, stage, reps, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


# ------------------------------------------------------------------ CPU baseline

def _cores():
    return int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count())


def cpu_decode(cfg, w, context, loops_of, budget_s, what, threads=0):
    """The oracle decoding single tokens after its cache is loaded with
    `context` synthetic rows; loops_of(i) gives token i's loop count.  threads:
    the oracle's OpenMP threads (0: all the host's).  At least one token, then
    as many as fit the budget."""
    from looped_normalized_gpt_amd import synth
    from oracle import oracle as O
    used = O.set_threads(threads)
    o = O.Oracle(cfg, w, max_ctx=context + 40)
    no = n_ord(cfg)
    k, v = synth.make_kv_rows(no * context, cfg["nk"], cfg["hd"], cfg["hidden"], seed=4)
    shp = (no, 1, context, cfg["nk"], cfg["hd"])
    o.kv_load(k.reshape(shp), v.reshape(shp))
    del k, v
    toks = synth.make_tokens(32, cfg["vocab"], seq=9)
    n, t0 = 0, time.perf_counter()
    while n < 32:
        o.forward(toks[n:n + 1], loops_of(n), "last_loop")
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    o.close()
    O.set_threads(0)
    return {"value": round(n / dt, 4), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{n} {what} at context {context}, the oracle's cache loaded with {context} synthetic rows, "
                      f"{dt:.1f} s on {used} thread(s) of {os.cpu_count()} host cores"}


def cpu_prefill(cfg, w, rows, loops, threads=0):
    from looped_normalized_gpt_amd import synth
    from oracle import oracle as O
    used = O.set_threads(threads)
    o = O.Oracle(cfg, w, max_ctx=rows + 8)
    toks = synth.make_tokens(rows, cfg["vocab"], seq=9)
    t0 = time.perf_counter()
    o.forward(toks, loops, "per_loop")
    dt = time.perf_counter() - t0
    o.close()
    O.set_threads(0)
    return {"value": round(rows / dt, 4), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"one {rows}-row prompt call of Dory-2B (per_loop, loops {loops}) from position 0, {dt:.1f} s "
                      f"on {used} thread(s) of {os.cpu_count()} host cores"}


# ------------------------------------------------------------------ workloads

def prompt(g, cfg, n, loops, mode, seq=0, chunk=512, tok_seed=None, last_logits=False):
    from looped_normalized_gpt_amd import synth
    toks = synth.make_tokens(n, cfg["vocab"], seq=seq if tok_seed is None else tok_seed)
    for c in range(0, n, chunk):
        g.forward(toks[c:min(c + chunk, n)], loops, mode, seq=seq, logits=(last_logits and c + chunk >= n))


def run_decode(args, q8, gate=None):
    import numpy as np
    import torch

    from looped_normalized_gpt_amd import dory, synth
    cfg = synth.config("2b", kv_encoding="q8_2f", full_window=8192) if q8 else synth.config("2b")
    ctx = args.context or (32768 if q8 else 4096)
    K, W, loops = args.steps or 256, 16 if args.warmup is None else args.warmup, 4
    log(f"bench: Dory-2B weights; decode at context {ctx}{' (q8_2f cache)' if q8 else ''}")
    w = synth.make_weights(cfg)
    g = dory.Dory(cfg, w, max_ctx=ctx + W + K + 8, max_chunk=512)
    toks = synth.make_tokens(ctx + W + K, cfg["vocab"])
    stream = torch.cuda.current_stream()
    log(f"bench: prompt of {ctx} tokens in calls of 512")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for c in range(0, ctx, 512):
        g.forward(toks[c:min(c + 512, ctx)], loops, "last_loop", logits=(c + 512 >= ctx))
        if c % 8192 == 0 and c:
            log(f"bench:   {c} tokens")
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t0

    logits = torch.empty(cfg["vocab"], dtype=torch.float32, device="cuda")
    if gate is not None:
        # the confidence-gated early exit on every one-row call (its passes
        # replace `loops`); a call with a read-out waits for it on the host
        g.set_gate(gate)
    for i in range(W):
        g.forward(toks[ctx + i:ctx + i + 1], loops, "last_loop", logits=logits)
    torch.cuda.synchronize()
    log(f"bench: {K} timed decode steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(W, W + K):
        g.forward(toks[ctx + i:ctx + i + 1], loops, "last_loop", logits=logits)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms = ev0.elapsed_time(ev1) / K
    if gate is not None:
        ms = wall_ms / K   # the read-outs wait on the host: the host clock is the one that counts
        gstats = g.gate_stats()
    assert torch.isfinite(logits).all().item(), "non-finite logits"
    tok_s = 1000.0 / ms
    bytes_tok = float(np.mean([token_bytes(cfg, ctx + i, loops) for i in range(W, W + K)]))
    gbs = bytes_tok * tok_s / 1e9

    log("bench: dominant kernel (gate|up GEMV) and the other stages")
    H, F = cfg["hidden"], cfg["ffn"]
    gu_bytes = 2 * F * H * 2 + H * 4 + F * 4
    gu_us = time_stage(dory, g, "gateup", args.stage_reps, stream)
    stages = {st: round(time_stage(dory, g, st, 96, stream), 2) for st in ("qkvg", "attn", "o", "down", "head")}
    stages["gateup"] = round(gu_us, 2)
    sliding_merged = g.xcd_merge()
    g.close()
    gu_gbs = gu_bytes / (gu_us * 1e-6) / 1e9
    log("bench: the vendor GEMV on the gate|up shape (reference only)")
    v_us = vendor_gemv_us(2 * F, H)
    vendor = {"us": round(v_us, 2), "gbps": round(2 * F * H * 2 / (v_us * 1e-6) / 1e9, 1),
              "what": "torch.mv, bf16 [11264][2048] x bf16 vector (no SwiGLU)"}

    log("bench: measured peaks and the per-launch floor of a token")
    peaks = measured_peaks()
    floor = launch_floor(cfg, ctx, loops, sliding_merged)
    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        log("bench: CPU baseline (oracle), all host cores and one core")
        # q8: the windows (1024 sliding, 8192 full) cap the rows a token reads, so
        # a context just past 8192 costs the oracle what 32768 does
        cctx = 8200 if q8 else ctx
        what = f"decode tokens of Dory-2B (loops {loops}, last_loop{', q8_2f' if q8 else ''})"
        cpu = cpu_decode(cfg, w, cctx, lambda i: loops, 20.0, what)
        cpu1 = cpu_decode(cfg, w, cctx, lambda i: loops, 15.0, what, threads=1)
    if gate is not None:
        metric = f"gated decode tokens/s (confidence gate {gate}), 1×MI355X, Dory-2B ctx {ctx}"
        workload = (f"Dory-2B decode, batch 1, context {ctx}, confidence-gated early exit at top probability "
                    f"{gate} (one or two passes), last_loop, fp32 KV cache, bf16 weights with fp32 arithmetic")
    elif q8:
        metric = "q8_2f long-context decode tokens/s (all loops) + achieved HBM GB/s, 1×MI355X, Dory-2B ctx 32768"
        workload = (f"Dory-2B decode, batch 1, context {ctx}, loops 4, last_loop, q8_2f KV cache "
                    f"(full_window 8192), bf16 weights with fp32 arithmetic")
    else:
        metric = METRIC
        workload = (f"Dory-2B decode, batch 1, context {ctx}, loops 4, last_loop, fp32 KV cache, "
                    f"bf16 weights with fp32 arithmetic")
    out = {
        "metric": metric, "value": round(tok_s, 2), "unit": "tokens/s", "steps": K, "warmup": W,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": workload, "context": ctx, "loops": loops, "kv_mode": "last_loop",
                   "kv_encoding": cfg["kv_encoding"], "weights": "bf16", "parallelism": "none (one GPU)"},
        "hbm_gbps_algorithmic": round(gbs, 1), "bytes_per_token": int(bytes_tok),
        "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "wall_ms_per_step": round(wall_ms / K, 4),
        "prefill_tokens_per_s": round(ctx / prefill_s, 1), "stage_us": stages, "vendor_gemv_same_shape": vendor,
        "roofline": roofline_extra({"kernel": "k_gemv gate|up + SwiGLU (bf16 [2x5632][2048])", "bound": "hbm",
                                    "achieved": round(gu_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(gu_gbs / PEAK_HBM_GBS, 4),
                                    "traffic": traffic_entry("q8" if q8 else "decode"),
                                    "bytes_per_launch": gu_bytes, "us_per_launch": round(gu_us, 3)},
                                   "q8" if q8 else "decode", peaks),
        "measured_peaks": peaks,
        "hbm_frac_of_measured_peak": round(gbs / peaks["hbm_gbs"], 4),
        "launch_floor": floor,
        "cpu_baseline": cpu,
        "cpu_baseline_one_core": cpu1,
    }
    if gate is not None:
        # passes per token follow the gate's decisions, not `loops`: the byte
        # count above assumes 4 loops and is not reported for this workload
        tokens, one, _, rate = gstats
        for k in ("hbm_gbps_algorithmic", "bytes_per_token", "hbm_frac_of_peak", "hbm_frac_of_measured_peak"):
            out.pop(k)
        out["config"]["loops"] = "1 or 2 (gated)"
        out["gate"] = {"threshold": gate, "tokens": tokens, "one_pass": one, "exit_rate": round(rate, 4),
                       "note": "synthetic weights: top probabilities stay far below the threshold, so no token "
                               "exits; the exit rate falls and 1 token in 8 reads out after its first pass"}
    return out


def run_prefill(args):
    import torch

    from looped_normalized_gpt_amd import dory, synth
    cfg = synth.config("2b")
    n = args.context or 8192
    K, W, loops, chunk = args.steps or 2, 1 if args.warmup is None else args.warmup, 8, 512
    log(f"bench: Dory-2B weights; prefill of {n} tokens, per_loop, loops {loops}")
    w = synth.make_weights(cfg)
    g = dory.Dory(cfg, w, max_ctx=n + 8, max_chunk=chunk)
    stream = torch.cuda.current_stream()
    for i in range(W):
        g.reset()
        prompt(g, cfg, n, loops, "per_loop", last_logits=True)
    torch.cuda.synchronize()
    log(f"bench: {K} timed prompts")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        g.reset()
        prompt(g, cfg, n, loops, "per_loop", last_logits=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms = ev0.elapsed_time(ev1) / K
    tok_s = n * 1000.0 / ms
    gemm_tflops = prefill_flops(cfg, n, loops) / (ms * 1e-3) / 1e12

    log("bench: stages at 512 rows")
    H, F, Q, KV = cfg["hidden"], cfg["ffn"], cfg["nh"] * cfg["hd"], cfg["nk"] * cfg["hd"]
    shapes = {"gemm_qkvg": (2 * Q + 2 * KV, H), "gemm_o": (H, Q), "gemm_gateup": (2 * F, H), "gemm_down": (H, F)}
    stages, tflops = {}, {}
    for st, (N, Kd) in shapes.items():
        us = time_stage(dory, g, st, args.stage_reps if st == "gemm_gateup" else 96, stream)
        stages[st] = round(us, 2)
        tflops[st] = round(2 * chunk * N * Kd / (us * 1e-6) / 1e12, 1)
    stages["attn_chunk"] = round(time_stage(dory, g, "attn_chunk", 32, stream), 2)
    g.close()
    log("bench: the vendor GEMM on the same shapes (reference only)")
    vendor = {st: round(vendor_gemm_tflops(chunk, N, Kd), 1) for st, (N, Kd) in shapes.items()}
    gu_flops = 2 * chunk * 2 * F * H
    gu_tf = tflops["gemm_gateup"]

    log("bench: measured peaks")
    peaks = measured_peaks()
    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        log("bench: CPU baseline (oracle): one 512-row call on all host cores, 16 rows on one core")
        cpu = cpu_prefill(cfg, w, chunk, loops)
        cpu1 = cpu_prefill(cfg, w, 16, loops, threads=1)
    return {
        "metric": "prefill tokens/s, 1×MI355X, Dory-2B per_loop loops 8, 8192-token prompt in 512-row calls",
        "value": round(tok_s, 1), "unit": "tokens/s", "steps": K, "warmup": W, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"Dory-2B prefill, {n}-token prompt in calls of {chunk}, per_loop, loops {loops}, "
                               f"bf16 MFMA projections (bf16 operands, fp32 accumulation), fp32 attention",
                   "prompt": n, "chunk": chunk, "loops": loops, "kv_mode": "per_loop", "weights": "bf16",
                   "parallelism": "none (one GPU)"},
        "projection_tflops_overall": round(gemm_tflops, 1), "wall_ms_per_step": round(wall_ms / K, 3),
        "stage_us": stages, "stage_tflops": tflops, "vendor_gemm_tflops_same_shapes": vendor,
        "roofline": roofline_extra({"kernel": "k_gemm_mfma2<SwiGLU> gate|up with the SwiGLU epilogue "
                                              "(512 x 11264 x 2048, bf16)",
                                    "bound": "mfma",
                                    "achieved": gu_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                    "frac": round(gu_tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic_entry("prefill"),
                                    "flops_per_launch": gu_flops, "us_per_launch": stages["gemm_gateup"]},
                                   "prefill", peaks),
        "measured_peaks": peaks,
        "stage_frac_of_measured_mfma": {k: round(v / peaks["bf16_mfma_tflops"], 4) for k, v in tflops.items()},
        "cpu_baseline": cpu,
        "cpu_baseline_one_core": cpu1,
    }


def run_batch(args):
    import numpy as np
    import torch

    from looped_normalized_gpt_amd import dory, synth
    cfg = synth.config("2b")
    nseq, ctx = 64, args.context or 8192
    K, W = args.steps or 128, 4 if args.warmup is None else args.warmup
    log(f"bench: Dory-2B weights; {nseq} sequences prefilled to {ctx}")
    w = synth.make_weights(cfg)
    g = dory.Dory(cfg, w, max_ctx=ctx + W + K + 8, max_chunk=512, max_seqs=nseq)
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    for s in range(nseq):
        prompt(g, cfg, ctx, 4, "last_loop", seq=s)
        if s % 8 == 7:
            torch.cuda.synchronize()
            log(f"bench:   {s + 1} sequences prefilled, {time.perf_counter() - t0:.1f} s")
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t0
    loops = synth.make_loops((W + K) * nseq).reshape(W + K, nseq)
    toks = np.stack([synth.make_tokens(W + K, cfg["vocab"], seq=100 + s) for s in range(nseq)], 1)
    seqs = np.arange(nseq, dtype=np.int32)
    logits = torch.empty((nseq, cfg["vocab"]), dtype=torch.float32, device="cuda")
    for i in range(W):
        g.forward_batch(seqs, toks[i], loops[i], "last_loop", logits=logits)
    torch.cuda.synchronize()
    log(f"bench: {K} timed batch steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(W, W + K):
        g.forward_batch(seqs, toks[i], loops[i], "last_loop", logits=logits)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms = ev0.elapsed_time(ev1) / K
    assert torch.isfinite(logits).all().item(), "non-finite logits"
    tok_s = nseq * 1000.0 / ms
    step_bytes = float(np.mean([batch_step_bytes(cfg, ctx + i, loops[i]) for i in range(W, W + K)]))
    gbs = step_bytes * (1000.0 / ms) / 1e9

    log("bench: dominant kernel (decode attention over the 64 rows)")
    # stage 1 cycles the 8 attention sub-layers (S and full alternate); the last
    # call's rows are all at position ctx + W + K - 1
    p = ctx + W + K - 1
    rb = kv_row_bytes(cfg)
    Q = cfg["nh"] * cfg["hd"]
    per_row = [visible(cfg, kind, p) * rb + Q * 4 * 2 + 2 * cfg["nk"] * cfg["hd"] * 4
               for kind in cfg["pattern"] if kind != "-"]
    at_bytes = nseq * float(np.mean(per_row))
    at_us = time_stage(dory, g, "attn", 64, stream)
    stages = {"attn": round(at_us, 2)}
    g.close()
    at_gbs = at_bytes / (at_us * 1e-6) / 1e9

    log("bench: measured peaks")
    peaks = measured_peaks()
    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        log("bench: CPU baseline (oracle), all host cores and one core")
        lp = loops[W:, 0]
        what = "single-sequence decode tokens of Dory-2B (loops drawn from 1..16, last_loop)"
        cpu = cpu_decode(cfg, w, ctx, lambda i: int(lp[i % len(lp)]), 20.0, what)
        cpu1 = cpu_decode(cfg, w, ctx, lambda i: int(lp[i % len(lp)]), 15.0, what, threads=1)
    return {
        "metric": "batched decode tokens/s (64 sequences, all loops) + achieved HBM GB/s, 1×MI355X, Dory-2B ctx 8192",
        "value": round(tok_s, 1), "unit": "tokens/s", "steps": K, "warmup": W, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"Dory-2B batched decode, {nseq} sequences at context {ctx}, last_loop, loops per "
                               f"(sequence, step) uniform in 1..16, fp32 KV cache, bf16 weights",
                   "sequences": nseq, "context": ctx, "kv_mode": "last_loop", "weights": "bf16",
                   "parallelism": "none (one GPU)"},
        "hbm_gbps_algorithmic": round(gbs, 1), "bytes_per_step": int(step_bytes),
        "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "wall_ms_per_step": round(wall_ms / K, 3),
        "prefill_tokens_per_s": round(nseq * ctx / prefill_s, 1), "stage_us": stages,
        "roofline": roofline_extra({"kernel": "k_attn_dec + k_attn_merge over 64 rows (S and full layers alternating)",
                                    "bound": "hbm", "achieved": round(at_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(at_gbs / PEAK_HBM_GBS, 4), "traffic": traffic_entry("batch"),
                                    "bytes_per_launch": int(at_bytes), "us_per_launch": round(at_us, 3)},
                                   "batch", peaks),
        "measured_peaks": peaks,
        "hbm_frac_of_measured_peak": round(gbs / peaks["hbm_gbs"], 4),
        "cpu_baseline": cpu,
        "cpu_baseline_one_core": cpu1,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--config", choices=("decode", "q8", "prefill", "batch", "gate"), default="decode")
    ap.add_argument("--gate", type=float, default=0.7,
                    help="gate workload: the top-probability threshold (dory.rs `--loops auto` default 0.7)")
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--context", type=int, default=None, help="decode context / prompt length")
    ap.add_argument("--stage-reps", type=int, default=400)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="first copy this many MiB device to device 3 times (a known-size kernel for "
                         "calibrating HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe_mb:
        n = args.copy_probe_mb << 18   # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.config in ("decode", "q8"):
        out = run_decode(args, args.config == "q8")
    elif args.config == "gate":
        args.no_cpu_baseline = True   # the oracle's decode sample is not gated
        out = run_decode(args, False, gate=args.gate)
    elif args.config == "prefill":
        out = run_prefill(args)
    else:
        out = run_batch(args)
    out = {"metric": out.pop("metric"), "value": out.pop("value"), "unit": out.pop("unit"), "n_gpus": 1, **out}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
