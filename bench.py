#!/usr/bin/env python
"""Benchmark: Dory-2B decode on one MI355X.

A step is one decode token: one call of the whole forward (input block, 4
passes of the recurrent block, output block, head) for one row at the next
position of a sequence whose cache already holds `--context` positions.
Set-up (not timed): seeded synthetic bf16 weights, a prompt of `--context`
seeded tokens run through the library's prefill path in calls of 512 rows
(last_loop, loops 4), then `--warmup` decode steps.  Timed: `--steps` decode
steps, bracketed by device synchronisation and HIP events on the stream the
library launches on.  Prints one JSON line.

The roofline entry is for the dominant kernel, the gate|up projection GEMV
with its SwiGLU epilogue (40% of a token's bytes): it is launched on its own
over the 20 MLP sub-layers' weights in turn, timed with HIP events on the same
stream, and its algorithmic bytes per launch are divided by the mean launch
time.  The CPU baseline is the oracle on the host cores: a few decode tokens at
the same context, after its cache is loaded with synthetic rows.
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
METRIC = "decode tokens/s (all loops) + achieved HBM GB/s, 1×MI355X, Dory-2B ctx 4096"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_gateup_2b_traffic.json")
GEMV_SRC = os.path.join(ROOT, "looped_normalized_gpt_amd", "csrc", "gemv.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def token_bytes(cfg, pos, loops):
    """Algorithmic HBM bytes of one decode token at position pos: every weight
    byte once, every visible cache row once (K and V, fp32), the scale vectors,
    the cache row written."""
    H, F, V, Q, KV = cfg["hidden"], cfg["ffn"], cfg["vocab"], cfg["nh"] * cfg["hd"], cfg["nk"] * cfg["hd"]
    wb = 2 if cfg["weight_dtype"] == "bf16" else 4
    n_in, n_rec, n_out = cfg["n_in"], cfg["n_rec"], cfg["n_out"]
    seq = [(li, 0) for li in range(n_in)] + [(n_in + j, i) for i in range(loops) for j in range(n_rec)] + \
          [(n_in + n_rec + j, 0) for j in range(n_out)]
    total = 0
    for li, _ in seq:
        kind = cfg["pattern"][li]
        if kind == "-":
            total += 3 * F * H * wb + (2 * F + H) * 4
        else:
            total += (2 * Q + 2 * KV) * H * wb + H * Q * wb + (2 * Q + H) * 4
            win = cfg["window"] if kind == "S" else (cfg.get("full_window") or 1 << 60)
            total += min(win, pos + 1) * KV * 4 * 2 + KV * 4 * 2
    total += V * H * wb + V * 4
    return total


def gateup_bytes(cfg):
    H, F = cfg["hidden"], cfg["ffn"]
    wb = 2 if cfg["weight_dtype"] == "bf16" else 4
    return 2 * F * H * wb + H * 4 + F * 4


def traffic_entry():
    """HBM bytes per launch of the gate|up GEMV from the committed counter runs,
    or None when there are none or the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    src = hashlib.sha256(open(GEMV_SRC, "rb").read()).hexdigest()
    if t.get("gemv_source_sha256") != src:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(cfg, w, context, loops, budget_s=20.0):
    import numpy as np

    from looped_normalized_gpt_amd import synth
    from oracle import oracle as O
    o = O.Oracle(cfg, w, max_ctx=context + 16)
    n_ord = sum(1 for ch in cfg["pattern"] if ch != "-")
    k, v = synth.make_kv_rows(n_ord * context, cfg["nk"], cfg["hd"], cfg["hidden"], seed=4)
    o.kv_load(k.reshape(n_ord, 1, context, cfg["nk"], cfg["hd"]), v.reshape(n_ord, 1, context, cfg["nk"], cfg["hd"]))
    del k, v
    toks = synth.make_tokens(16, cfg["vocab"], seq=9)
    n, t0 = 0, time.perf_counter()
    while n < 16:
        o.forward(toks[n:n + 1], loops, "last_loop")
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count())
    o.close()
    return {"value": round(n / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} decode tokens of Dory-2B (loops {loops}, last_loop) at context {context}, "
                      f"the oracle's cache loaded with {context} synthetic rows, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--context", type=int, default=4096)
    ap.add_argument("--loops", type=int, default=4)
    ap.add_argument("--stage-reps", type=int, default=400)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from looped_normalized_gpt_amd import dory, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = synth.config("2b")
    log("bench: generating Dory-2B weights")
    w = synth.make_weights(cfg)
    K, W, ctx, loops = args.steps, args.warmup, args.context, args.loops
    chunk = 512
    g = dory.Dory(cfg, w, max_ctx=ctx + W + K + 8, max_chunk=chunk)
    toks = synth.make_tokens(ctx + W + K, cfg["vocab"])
    stream = torch.cuda.current_stream()

    log(f"bench: prompt of {ctx} tokens in calls of {chunk}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for c in range(0, ctx, chunk):
        g.forward(toks[c:c + chunk], loops, "last_loop", logits=(c + chunk >= ctx))
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t0

    logits = torch.empty(cfg["vocab"], dtype=torch.float32, device="cuda")
    log(f"bench: {W} warm-up decode steps")
    for i in range(W):
        g.forward(toks[ctx + i:ctx + i + 1], loops, "last_loop", logits=logits)
    torch.cuda.synchronize()

    log(f"bench: {K} timed decode steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(W, W + K):
        g.forward(toks[ctx + i:ctx + i + 1], loops, "last_loop", logits=logits)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms = ev0.elapsed_time(ev1) / K
    assert torch.isfinite(logits).all().item(), "non-finite logits"
    tok_s = 1000.0 / ms
    pos = [ctx + i for i in range(W, W + K)]
    bytes_tok = float(np.mean([token_bytes(cfg, p, loops) for p in pos]))
    gbs = bytes_tok * tok_s / 1e9

    log(f"bench: dominant kernel (gate|up GEMV) x{args.stage_reps}")
    dory.stage_bench(g, "gateup", 40, stream)   # warm the launch path
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    dory.stage_bench(g, "gateup", args.stage_reps, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    gu_us = e0.elapsed_time(e1) * 1e3 / args.stage_reps
    gu_bytes = gateup_bytes(cfg)
    gu_gbs = gu_bytes / (gu_us * 1e-6) / 1e9
    traffic = traffic_entry()

    stages = {}
    for st in ("qkvg", "attn", "o", "down", "head"):
        reps = 100
        e0.record(stream)
        dory.stage_bench(g, st, reps, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        stages[st] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    stages["gateup"] = round(gu_us, 2)
    g.close()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: CPU baseline (oracle)")
        cpu = cpu_baseline(cfg, w, ctx, loops)

    out = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "Dory-2B decode, batch 1, context 4096, loops 4, last_loop, fp32 KV cache, "
                               "bf16 weights with fp32 arithmetic",
                   "context": ctx, "loops": loops, "kv_mode": "last_loop", "kv_encoding": "f32",
                   "weights": "bf16", "parallelism": "none (one GPU)"},
        "hbm_gbps_algorithmic": round(gbs, 1),
        "bytes_per_token": int(bytes_tok),
        "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
        "wall_ms_per_step": round(wall_ms / K, 4),
        "prefill_tokens_per_s": round(ctx / prefill_s, 1),
        "stage_us": stages,
        "roofline": {"kernel": "k_gemv gate|up + SwiGLU (bf16 [2x5632][2048])", "bound": "hbm",
                     "achieved": round(gu_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": gu_bytes, "us_per_launch": round(gu_us, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
