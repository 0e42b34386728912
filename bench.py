#!/usr/bin/env python3
"""Benchmark of the HySparse MQA sparse-attention forward path on one MI355X.

One step = the metric path on one batch of seeded synthetic input:
block scoring fused with causal attention (hs_block_score_fwd), per-token
top-k block selection (hs_topk_blocks) and block-sparse gather attention
(hs_sparse_gather_fwd), at S = 32768, 64 query heads, one latent KV head of
576 columns (value = leading 512), 64-key blocks, top-k 32, learnable sink.
The sliding-window call (hs_swa_fwd) is timed separately and reported next
to the metric, not in it.

Prints ONE JSON line. `value` is tokens/s of the metric path with inputs
resident in HBM; TFLOP/s counts algorithmic (query-head, key) pairs times
2*Dk + 2*Dv. The roofline object covers the dominant kernel (block scoring,
MFMA-bound) with its average launch time measured by HIP events on the
stream it runs on. The CPU baseline is the float64 oracle timed on a bounded
sample of query rows of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_mqa_amd as hs  # noqa: E402
from block_sparse_mqa_amd import inputs  # noqa: E402

METRIC = "TFLOP/s + tokens/s, block-score+top-k+sparse-gather fwd, S=32k, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def causal_pairs(p) -> int:
    """(query-head, key) pairs of causal attention over the allowed keys."""
    S = p.Sq
    if p.doc_start:
        tot = sum(L * (L + 1) // 2 for L in (e - s for s, e in zip(p.doc_start, p.doc_end)))
    else:
        tot = S * (S + 1) // 2
    return tot * p.H


def gather_pairs_from_idx(p, idx_cpu: np.ndarray) -> int:
    """Pairs of the gather: for each token, keys of its selected blocks that
    are allowed (no documents: block j covers [64j, 64j+64))."""
    S, BS = p.Sq, p.block_size
    t = np.arange(S)
    tot = 0
    for k in range(idx_cpu.shape[-1]):
        j = idx_cpu[0, :, k].astype(np.int64)
        ok = j >= 0
        start = j * BS
        n = np.clip(np.minimum(start + BS - 1, t) - start + 1, 0, BS)
        tot += int(np.where(ok, n, 0).sum())
    return tot * p.H


def swa_pairs(p) -> int:
    t = np.arange(p.Sq)
    return int(np.minimum(t + 1, p.window).sum()) * p.H


def flops_per_pair(p) -> int:
    return 2 * p.Dk + 2 * p.Dv


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_baseline(p, budget_s: float, seed: int = 0):
    """Time the oracle (block scores, top-k, gather) on uniformly drawn query
    rows until `budget_s` of CPU time is spent; tokens/s = rows / seconds."""
    from oracle import hysparse_ref as ref
    rng = np.random.default_rng(seed)
    kv64 = p.kv.to(torch.float64).numpy()
    sink = p.sink
    rows_done, spent = 0, 0.0
    while spent < budget_s and rows_done < p.Sq:
        r = int(rng.integers(0, p.Sq))
        t0 = time.perf_counter()
        _, _, bl = ref.block_score(p.q, kv64, sink, p.Dv, p.scale, block_size=p.block_size,
                                   rows=[r])
        own = ref.own_blocks(1, p.Sq, p.Skv, p.block_size, rows=[r])
        idx_r = ref.topk_blocks(bl, own, p.top_k)
        idx = np.full((1, p.Sq, p.top_k), -1, dtype=np.int64)
        idx[0, r] = idx_r[0, 0]
        ref.sparse_gather(p.q, kv64, sink, p.Dv, p.scale, idx, block_size=p.block_size, rows=[r])
        spent += time.perf_counter() - t0
        rows_done += 1
    return {"value": rows_done / spent, "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{rows_done} query rows drawn uniformly from S={p.Sq} "
                      f"(block scores + top-k + gather per row, float64), {spent:.1f} s"}


def counter_traffic(path: str, workload: str, kernel: str):
    """HBM bytes per launch measured by rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (each scaled by the reading of a 1 GiB copy), or None when no record
    exists or the kernel source changed since the counters were taken."""
    import hashlib
    try:
        with open(path) as f:
            rec = json.load(f)[workload][kernel]
        with open(os.path.join(ROOT, rec["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != rec["source_sha256_16"]:
                return None
        return int(rec["bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class Timer:
    """HIP events recorded on the stream the kernels run on."""

    def __init__(self, stream):
        self.stream = stream
        self.pairs = []

    def span(self):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        self.pairs.append((a, b))
        return a, b


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=3, help="named workload (1-5); 3 is the metric's")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one 1 GiB device copy (counter calibration)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured by counters, if recorded")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the path is built and measured on a single "
              "MI355X; multi-GPU runs are not supported.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    p = inputs.config(args.workload)
    dev = torch.device("cuda:0")
    q = p.q.to(dev)
    kv = p.kv.to(dev)
    sink = p.sink.to(dev)
    prob = hs.Problem(p.B, p.Sq, p.Skv, p.H, p.Dk, p.Dv, block_size=p.block_size, scale=p.scale,
                      dtype=p.dtype, kv_lens=p.kv_lens, doc_start=p.doc_start, doc_end=p.doc_end)
    NB = hs.hs_num_blocks(prob)
    tdt = p.torch_dtype
    out = torch.empty((p.B, p.Sq, p.H, p.Dv), dtype=tdt, device=dev)
    lse = torch.empty((p.B, p.Sq, p.H), dtype=torch.float32, device=dev)
    bl = torch.empty((p.B, p.Sq, NB), dtype=torch.float32, device=dev)
    idx = torch.empty((p.B, p.Sq, p.top_k), dtype=torch.int32, device=dev)
    og = torch.empty_like(out)
    lg = torch.empty_like(lse)
    osw = torch.empty_like(out)
    lsw = torch.empty_like(lse)

    def ws_for(op, **kw):
        n = hs.hs_workspace_size(prob, op, **kw)
        return torch.empty((n + 3) // 4, dtype=torch.float32, device=dev) if n else None

    ws1 = ws_for(hs.HS_OP_BLOCK_SCORE)
    ws3 = ws_for(hs.HS_OP_SPARSE_GATHER, top_k=p.top_k)
    ws4 = ws_for(hs.HS_OP_SWA, window=p.window)
    stream = torch.cuda.current_stream(dev)

    def step(tm=None):
        ev = [tm.span() for _ in range(3)] if tm else None
        if ev: ev[0][0].record(stream)
        hs.hs_block_score_fwd(prob, q, kv, sink, out, lse, bl, ws1, stream)
        if ev: ev[0][1].record(stream); ev[1][0].record(stream)
        hs.hs_topk_blocks(prob, bl, p.top_k, idx, stream)
        if ev: ev[1][1].record(stream); ev[2][0].record(stream)
        hs.hs_sparse_gather_fwd(prob, q, kv, sink, idx, p.top_k, og, lg, ws3, stream)
        if ev: ev[2][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tm = Timer(stream)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step(tm)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = start.elapsed_time(stop)
    per = np.array([a.elapsed_time(b) for a, b in tm.pairs]).reshape(args.steps, 3)
    k_ms = per.mean(axis=0)                  # block score, top-k, gather
    ms_per_step = total_ms / args.steps

    # Sliding window, timed on its own (not part of the metric path).
    hs.hs_swa_fwd(prob, q, kv, sink, p.window, osw, lsw, ws4, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(max(1, args.steps // 2)):
        hs.hs_swa_fwd(prob, q, kv, sink, p.window, osw, lsw, ws4, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    swa_ms = e0.elapsed_time(e1) / max(1, args.steps // 2)

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    # Algorithmic work.
    fpp = flops_per_pair(p)
    f_score = causal_pairs(p) * fpp
    idx_cpu = idx.cpu().numpy()
    f_gather = gather_pairs_from_idx(p, idx_cpu) * fpp if p.B == 1 and not p.doc_start else None
    f_swa = swa_pairs(p) * fpp if p.B == 1 and not p.doc_start else None
    tokens = p.B * p.Sq
    tok_s = tokens / (ms_per_step * 1e-3)
    tflops = ((f_score + (f_gather or 0)) / (ms_per_step * 1e-3) / 1e12)
    achieved = f_score / (k_ms[0] * 1e-3) / 1e12

    traffic = counter_traffic(args.traffic_json, p.name, "block_score")

    res = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "tflop_s": round(tflops, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": p.name, "B": p.B, "S": p.Sq, "H": p.H, "Dk": p.Dk, "Dv": p.Dv,
                   "block_size": p.block_size, "top_k": p.top_k, "window": p.window,
                   "sink": True, "parallelism": "single-gpu"},
        "kernels_ms": {"block_score": round(float(k_ms[0]), 4), "topk": round(float(k_ms[1]), 4),
                       "sparse_gather": round(float(k_ms[2]), 4), "swa": round(swa_ms, 4)},
        "kernels_tflop_s": {
            "block_score": round(f_score / (k_ms[0] * 1e-3) / 1e12, 2),
            "sparse_gather": round(f_gather / (k_ms[2] * 1e-3) / 1e12, 2) if f_gather else None,
            "swa": round(f_swa / (swa_ms * 1e-3) / 1e12, 2) if f_swa else None},
        "wall_s_timed": round(wall, 3),
        "roofline": {"kernel": "block_score (hs_block_score_fwd)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(p, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
