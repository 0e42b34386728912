#!/usr/bin/env python3
"""Benchmark of the HySparse MQA sparse-attention forward path on one MI355X.

One step = the metric path on one batch of seeded synthetic input:
block scoring fused with causal attention (hs_block_score_fwd), per-token
top-k block selection (hs_topk_blocks) and block-sparse gather attention
(hs_sparse_gather_fwd), at S = 32768, 64 query heads, one latent KV head of
576 columns (value = leading 512), 64-key blocks, top-k 32, learnable sink.
The sliding-window call (hs_swa_fwd) is timed separately and reported next
to the metric, not in it, and so are the gradient calls of the three
attention operations (the "gradients" object, timed after the metric).

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


def roofline_entry(kernel, flops, compulsory_bytes, ms, traffic=None, **extra):
    """Roofline of one kernel: t_roof = max(flops / MFMA peak, compulsory bytes /
    HBM peak); `achieved` is the rate on the bounding resource over the
    kernel's mean launch time (HIP events on its stream)."""
    t_m = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_h = compulsory_bytes / (PEAK_HBM_GBS * 1e9)
    s = ms * 1e-3
    if t_m >= t_h:
        ach, peak, unit, bound = flops / s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = compulsory_bytes / s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    r = {"kernel": kernel, "bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
         "frac": round(ach / peak, 4), "traffic": traffic, "flop": flops,
         "compulsory_bytes": int(compulsory_bytes), "ms": round(ms, 4)}
    r.update(extra)
    return r


def cpu_baseline(p, budget_s: float, seed: int = 0, group: int = 4):
    """Time the oracle (block scores, top-k, gather; float64) on a bounded
    sample of query rows: groups of `group` consecutive rows at uniformly drawn
    starts, computed by one thread per host core with one BLAS thread each
    (oracle/parallel.py), until about `budget_s` seconds of wall time have
    passed. tokens/s = rows / wall seconds."""
    from oracle import parallel as par
    rng = np.random.default_rng(seed)
    kv64 = p.kv.to(torch.float64).numpy()
    workers = par.default_workers()
    starts = rng.integers(0, max(1, p.Sq - group + 1), size=4096)
    kw = dict(block_size=p.block_size, kv_lens=p.kv_lens, doc_start=p.doc_start,
              doc_end=p.doc_end)

    def fn(rows):
        return par.metric_path_rows(p.q, kv64, p.sink, p.Dv, p.scale, p.top_k, rows, **kw)[3]

    done, t0 = 0, time.perf_counter()
    batch = 2 * workers
    for i in range(0, len(starts), batch):
        rows = np.concatenate([np.arange(s0, s0 + group) for s0 in starts[i:i + batch]])
        for c, _ in par.map_row_chunks(fn, rows, group, workers):
            done += len(c)
        if time.perf_counter() - t0 >= budget_s:
            break
    spent = time.perf_counter() - t0
    return {"value": round(done * p.B / spent, 3), "unit": "tokens/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{done} query rows in groups of {group} consecutive rows at uniformly drawn "
                      f"starts of S={p.Sq} (block scores + top-k + gather per row, float64), "
                      f"{workers} threads x 1 BLAS thread, {spent:.1f} s wall"}


def counter_traffic(path: str, workload: str, kernel: str):
    """HBM bytes per launch measured by rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (each scaled by the reading of a 1 GiB copy), or None when no record
    exists or the kernel's sources (the files listed in the record, hashed in
    order) changed since the counters were taken."""
    import hashlib
    try:
        with open(path) as f:
            rec = json.load(f)[workload][kernel]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest()[:16] != rec["sources_sha256_16"]:
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


# ---------------------------------------------------------------------------
# --suite: every named workload, every kernel, warm and cold, against the
# vendor peaks and the attainable peaks measured by the probe kernels.
# ---------------------------------------------------------------------------

PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector (the fp32 shapes use FMAs, no MFMA)


def host_blocks(p):
    """Per batch entry: valid length L_b, document bounds and block table
    (start, end) in the numbering of block_logit (blocks restart at every
    document start). Host arithmetic for work counting only."""
    out = []
    for b in range(p.B):
        L = p.kv_lens[b] if p.kv_lens else p.Skv
        docs = list(zip(p.doc_start, p.doc_end)) if p.doc_start else [(0, L)]
        blocks = []
        for s0, e0 in docs:
            for st in range(s0, e0, p.block_size):
                blocks.append((st, min(st + p.block_size, e0)))
        out.append((L, docs, blocks))
    return out


def row_key_counts(p, idx_cpu=None):
    """Per (batch, row): allowed keys of causal attention, of the window, of
    the gather over the selected blocks (when indices are given), and the
    distinct KV rows each operation touches per batch entry."""
    causal, window, gather = [], [], []
    kv_rows = {"score": 0, "swa": 0, "gather": 0}
    for b, (L, docs, blocks) in enumerate(host_blocks(p)):
        pos = np.arange(L - p.Sq, L)
        lo = np.zeros_like(pos)
        for s0, e0 in docs:
            m = (pos >= s0) & (pos < e0)
            lo[m] = s0
        causal.append(pos - lo + 1)
        wlo = np.maximum(lo, pos - p.window + 1)
        window.append(pos - wlo + 1)
        kv_rows["score"] += int(pos.max() + 1 - lo.min())
        kv_rows["swa"] += int(pos.max() + 1 - wlo.min())
        if idx_cpu is not None:
            st = np.array([x[0] for x in blocks]); en = np.array([x[1] for x in blocks])
            g = np.zeros(p.Sq, dtype=np.int64)
            used = np.zeros(len(blocks), dtype=bool)   # blocks some row gathers from
            for k in range(idx_cpu.shape[-1]):
                j = idx_cpu[b, :, k].astype(np.int64)
                ok = (j >= 0) & (j < len(blocks))
                jj = np.where(ok, j, 0)
                a = np.maximum(st[jj], lo); e = np.minimum(en[jj] - 1, pos)
                n = np.where(ok, np.clip(e - a + 1, 0, None), 0)
                g += n
                used[jj[n > 0]] = True
            gather.append(g)
            # distinct KV rows of the gathered blocks (each block's rows at most once)
            kv_rows["gather"] += int((en - st)[used].sum())
    cat = lambda x: np.concatenate(x) if x else None
    return cat(causal), cat(window), cat(gather), kv_rows


def median_time(fn, stream, n=20, warm=3, before=None):
    """Median launch time (ms) of fn() over n launches after `warm` warm-ups,
    each bracketed by HIP events on `stream`; before() runs untimed first."""
    for _ in range(warm):
        fn()
    ts = []
    for _ in range(n):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
        a.record(stream); fn(); b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def measure_peaks(dev, stream):
    from block_sparse_mqa_amd import probe
    wg, iters = 2048, 10000
    out = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    t = median_time(lambda: probe.hs_probe_mfma_bf16(wg, iters, out, clocks, stream), stream,
                    n=10, warm=2)
    mfma = probe.hs_probe_mfma_flops(wg, iters) / (t * 1e-3) / 1e12
    cyc, ticks = (int(x) for x in clocks.cpu())
    sclk_ghz = cyc / (ticks / 1e8) / 1e9 if ticks > 0 else None
    nbytes = 2 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    t = median_time(lambda: probe.hs_probe_copy(src, dst, nbytes, stream), stream, n=10, warm=2)
    copy = 2 * nbytes / (t * 1e-3) / 1e9
    del src, dst
    return {"mfma_bf16_tflop_s": round(mfma, 1), "copy_gb_s": round(copy, 1),
            "shader_clock_ghz_under_mfma": None if sclk_ghz is None else round(sclk_ghz, 3),
            "mfma_probe": f"{wg} workgroups x 4 waves x {iters} x 4 chains of v_mfma_f32_32x32x16_bf16",
            "copy_probe": f"{nbytes >> 30} GiB read + {nbytes >> 30} GiB written, 16 B per lane, nontemporal"}


def oracle_time(p, budget_s, seed=0, threads=None, group=4):
    """Oracle (block scores, top-k, gather; float64) on the workload's rows,
    run by `threads` worker threads (default: one per host core) with one BLAS
    thread each: all rows when they fit in `budget_s`, else groups of `group`
    consecutive rows at uniformly drawn starts, with the full-run time
    extrapolated by causal pairs (labelled)."""
    from oracle import parallel as par
    causal, _, _, _ = row_key_counts(p)
    per_row = causal.reshape(p.B, p.Sq).sum(axis=0)       # pairs per row index, all batch entries
    rng = np.random.default_rng(seed)
    order = rng.permutation(np.arange(0, p.Sq, group))
    kv64 = p.kv.to(torch.float64).numpy()
    workers = threads or par.default_workers()
    kw = dict(block_size=p.block_size, kv_lens=p.kv_lens, doc_start=p.doc_start, doc_end=p.doc_end)

    def fn(rows):
        return par.metric_path_rows(p.q, kv64, p.sink, p.Dv, p.scale, p.top_k, rows, **kw)[3]

    done, pairs, t0, last_note = 0, 0, time.perf_counter(), 0.0
    batch = 2 * workers
    for i in range(0, len(order), batch):
        rows = np.concatenate([np.arange(s0, min(p.Sq, s0 + group)) for s0 in order[i:i + batch]])
        for c, _ in par.map_row_chunks(fn, rows, group, workers):
            done += len(c)
            pairs += int(per_row[c].sum())
        spent = time.perf_counter() - t0
        if spent - last_note >= 30.0:
            last_note = spent
            print(f"[oracle] {p.name}: {done}/{p.Sq} rows, {spent:.0f} s", file=sys.stderr,
                  flush=True)
        if spent >= budget_s:
            break
    spent = time.perf_counter() - t0
    full = done == p.Sq
    est_full_s = spent if full else spent * float(per_row.sum()) / max(pairs, 1)
    return {"tokens_s": round(done * p.B / spent, 3), "rows": done * p.B, "seconds": round(spent, 2),
            "full": full, "full_run_s": round(est_full_s, 1),
            "full_run_s_is": "measured" if full else "extrapolated by causal pairs from the sample",
            "threads": workers}


def suite_config(c, dev, stream, peaks, oracle_budget):
    p = inputs.config(c)
    q, kv, sink = p.q.to(dev), p.kv.to(dev), p.sink.to(dev)
    prob = hs.Problem(p.B, p.Sq, p.Skv, p.H, p.Dk, p.Dv, block_size=p.block_size, scale=p.scale,
                      dtype=p.dtype, kv_lens=p.kv_lens, doc_start=p.doc_start, doc_end=p.doc_end)
    NB = hs.hs_num_blocks(prob)
    tdt = p.torch_dtype
    out = torch.empty((p.B, p.Sq, p.H, p.Dv), dtype=tdt, device=dev)
    lse = torch.empty((p.B, p.Sq, p.H), dtype=torch.float32, device=dev)
    bl = torch.empty((p.B, p.Sq, NB), dtype=torch.float32, device=dev)
    idx = torch.empty((p.B, p.Sq, p.top_k), dtype=torch.int32, device=dev)

    def ws(op, **k):
        n = hs.hs_workspace_size(prob, op, **k)
        return torch.empty((n + 3) // 4, dtype=torch.float32, device=dev) if n else None

    w1, w3, w4 = ws(hs.HS_OP_BLOCK_SCORE), ws(hs.HS_OP_SPARSE_GATHER, top_k=p.top_k), \
        ws(hs.HS_OP_SWA, window=p.window)
    calls = {
        "block_score": lambda: hs.hs_block_score_fwd(prob, q, kv, sink, out, lse, bl, w1, stream),
        "topk": lambda: hs.hs_topk_blocks(prob, bl, p.top_k, idx, stream),
        "score_topk_fused": lambda: hs.hs_block_score_topk_fwd(prob, q, kv, sink, p.top_k, out, lse,
                                                               bl, idx, w1, stream),
        "sparse_gather": lambda: hs.hs_sparse_gather_fwd(prob, q, kv, sink, idx, p.top_k, out, lse,
                                                         w3, stream),
        "swa": lambda: hs.hs_swa_fwd(prob, q, kv, sink, p.window, out, lse, w4, stream),
    }
    # both branches of a sliding-window layer in one call (window, then the
    # selected blocks of this workload's own top-k)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    w8 = ws(hs.HS_OP_SWA_SPARSE, top_k=p.top_k, window=p.window)
    calls["swa_sparse"] = lambda: hs.hs_swa_sparse_fwd(prob, q, kv, sink, p.window, idx, p.top_k,
                                                       out2, lse2, out, lse, w8, stream)
    calls["block_score"](); calls["topk"](); torch.cuda.synchronize()
    idx_cpu = idx.cpu().numpy()
    # Gradients of the three attention calls, each from its own forward outputs.
    dout = inputs.make_dout(p, seed=900 + c).to(dev)
    fwd = {}
    for op_name, fn in (("block_score", calls["block_score"]), ("sparse_gather", calls["sparse_gather"]),
                        ("swa", calls["swa"])):
        fn(); torch.cuda.synchronize()
        fwd[op_name] = (out.clone(), lse.clone())
    dq = torch.empty((p.B, p.Sq, p.H, p.Dk), dtype=torch.float32, device=dev)
    dkv = torch.empty((p.B, p.Skv, p.Dk), dtype=torch.float32, device=dev)
    dsink = torch.empty((p.H,), dtype=torch.float32, device=dev)
    wb1, wb3, wb4 = hs.score_bwd_workspace(prob, store_ds=True), \
        hs.sparse_gather_bwd_workspace(prob, p.top_k, store_ds=True), \
        hs.swa_bwd_workspace(prob, p.window, store_ds=True)
    calls["block_score_bwd"] = lambda: hs.hs_block_score_bwd(
        prob, q, kv, sink, *fwd["block_score"], dout, dq, dkv, dsink, wb1, stream)
    calls["sparse_gather_bwd"] = lambda: hs.hs_sparse_gather_bwd(
        prob, q, kv, sink, idx, p.top_k, *fwd["sparse_gather"], dout, dq, dkv, dsink, wb3, stream)
    calls["swa_bwd"] = lambda: hs.hs_swa_bwd(
        prob, q, kv, sink, p.window, *fwd["swa"], dout, dq, dkv, dsink, wb4, stream)
    causal, window, gather, kv_rows = row_key_counts(p, idx_cpu)
    fpp, H, es = 2 * p.Dk + 2 * p.Dv, p.H, (2 if p.dtype == "bf16" else 4)
    qb, ob, lb = p.B * p.Sq * H * p.Dk * es, p.B * p.Sq * H * p.Dv * es, p.B * p.Sq * H * 4
    work = {
        "block_score": (int(causal.sum()) * H * fpp,
                        qb + kv_rows["score"] * p.Dk * es + ob + lb + p.B * p.Sq * NB * 4),
        "topk": (0, p.B * p.Sq * (NB + p.top_k) * 4),
        "score_topk_fused": (int(causal.sum()) * H * fpp,
                             qb + kv_rows["score"] * p.Dk * es + ob + lb + p.B * p.Sq * NB * 4),
        # compulsory bytes: every gathered KV row at most once (the per-token
        # selected rows, reported separately, are served largely from L2 and
        # the MALL)
        "sparse_gather": (int(gather.sum()) * H * fpp,
                          qb + ob + lb + p.B * p.Sq * p.top_k * 4 + kv_rows["gather"] * p.Dk * es),
        "swa": (int(window.sum()) * H * fpp, qb + kv_rows["swa"] * p.Dk * es + ob + lb),
    }
    work["swa_sparse"] = (int(window.sum()) * H * fpp + int(gather.sum()) * H * fpp,
                          qb + max(kv_rows["swa"], kv_rows["gather"]) * p.Dk * es +
                          2 * (ob + lb) + p.B * p.Sq * p.top_k * 4)
    l2_served = {"sparse_gather": qb + ob + lb + int(gather.sum()) * p.Dk * es}
    # Gradients: five contractions per pair (S recomputed, dP, dQ, dK, dV), i.e.
    # 2 (3 Dk + 2 Dv) flops; bytes: q, kv rows, out, dout, lse, dq and dkv in fp32.
    fpb = 2 * (3 * p.Dk + 2 * p.Dv)
    gb = qb + 2 * ob + lb + p.B * p.Sq * H * p.Dk * 4
    work["block_score_bwd"] = (int(causal.sum()) * H * fpb,
                               gb + kv_rows["score"] * p.Dk * (es + 4))
    work["sparse_gather_bwd"] = (int(gather.sum()) * H * fpb,
                                 gb + p.B * p.Sq * p.top_k * 4 + kv_rows["gather"] * p.Dk * (es + 4))
    work["swa_bwd"] = (int(window.sum()) * H * fpb, gb + kv_rows["swa"] * p.Dk * (es + 4))
    peak_f = PEAK_BF16_TFLOPS if p.dtype == "bf16" else PEAK_F32_TFLOPS
    meas_f = peaks["mfma_bf16_tflop_s"] if p.dtype == "bf16" else None
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    rows = {}
    for k, fn in calls.items():
        if k == "sparse_gather":   # indices of this workload's own top-k
            calls["topk"](); torch.cuda.synchronize()
        warm = median_time(fn, stream)
        cold = median_time(fn, stream, n=10, warm=1, before=lambda: scratch.fill_(0.5))
        F, Bts = work[k]
        t_roof = max(F / (peak_f * 1e12), Bts / (PEAK_HBM_GBS * 1e9)) * 1e3
        t_roof_m = max(F / (meas_f * 1e12) if meas_f else 0.0,
                       Bts / (peaks["copy_gb_s"] * 1e9)) * 1e3
        bound = "hbm" if Bts / (PEAK_HBM_GBS * 1e9) >= F / (peak_f * 1e12) else \
            ("mfma" if p.dtype == "bf16" else "alu")
        rows[k] = {"ms_warm": round(warm, 4), "ms_cold": round(cold, 4),
                   "tflop": round(F / 1e12, 4), "gb_alg": round(Bts / 1e9, 4), "bound": bound,
                   "tflop_s": round(F / (warm * 1e-3) / 1e12, 2) if F else None,
                   "gb_s_alg": round(Bts / (warm * 1e-3) / 1e9, 1),
                   "frac_vendor": round(t_roof / warm, 4),
                   "frac_measured_peak": round(t_roof_m / warm, 4) if (meas_f or bound == "hbm") else None}
        if k in l2_served:
            rows[k]["gb_s_per_token_kv_l2_served"] = round(l2_served[k] / (warm * 1e-3) / 1e9, 1)
        print(f"[suite] workload {c} {k}: {rows[k]}", file=sys.stderr, flush=True)
    del scratch, dq, dkv, dout, fwd
    path_ms = rows["block_score"]["ms_warm"] + rows["topk"]["ms_warm"] + rows["sparse_gather"]["ms_warm"]
    res = {"workload": p.name, "dtype": p.dtype, "kernels": rows,
           "metric_path_ms": round(path_ms, 4),
           "fused_path_ms": round(rows["score_topk_fused"]["ms_warm"] + rows["sparse_gather"]["ms_warm"], 4),
           "tokens_s": round(p.B * p.Sq / (path_ms * 1e-3), 1),
           "metric_tflop_s": round((work["block_score"][0] + work["sparse_gather"][0]) /
                                   (path_ms * 1e-3) / 1e12, 2)}
    if oracle_budget > 0:
        res["oracle"] = oracle_time(p, oracle_budget)
        print(f"[suite] workload {c} oracle: {res['oracle']}", file=sys.stderr, flush=True)
        if c in (1, 2):
            res["oracle_1_thread"] = oracle_time(p, min(oracle_budget, 20.0), threads=1)
    return res


def run_suite(args):
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    peaks = measure_peaks(dev, stream)
    print(json.dumps({"suite": "peaks", **peaks}), flush=True)
    results = []
    for c in args.suite_workloads:
        budget = float("inf") if c in (args.oracle_full_for or []) else args.oracle_budget
        r = suite_config(c, dev, stream, peaks, budget)
        results.append(r)
        print(json.dumps({"suite": "workload", **r}), flush=True)
        torch.cuda.empty_cache()
    if args.suite_md:
        write_suite_md(args.suite_md, peaks, results, args)


def write_suite_md(path, peaks, results, args):
    L = ["# Per-workload measurements (all kernels, warm and cold)\n",
         "Command (from the repository root, on one MI355X):\n",
         "```\npython3 bench.py --suite --suite-md " + os.path.relpath(path, ROOT) +
         (" --oracle-full" if args.oracle_full else f" --oracle-budget {args.oracle_budget:g}") +
         (" --oracle-full-for " + " ".join(str(c) for c in args.oracle_full_for)
          if args.oracle_full_for and not args.oracle_full else "") +
         "\n```\n",
         f"Attainable peaks measured by the probe kernels (`include/hs_probe.h`): dense bf16 MFMA "
         f"{peaks['mfma_bf16_tflop_s']:.0f} TFLOP/s ({peaks['mfma_probe']}; shader clock while it ran: "
         f"{peaks['shader_clock_ghz_under_mfma']} GHz by s_memtime against the 100 MHz reference); copy "
         f"{peaks['copy_gb_s']:.0f} GB/s ({peaks['copy_probe']}). Vendor peaks: 2500 TFLOP/s bf16 "
         "MFMA, 157.3 TFLOP/s fp32 vector, 8000 GB/s HBM.\n",
         "Times are medians of 20 launches after 3 warm-ups (warm) and of 10 launches each after "
         "writing a 1 GiB buffer, which evicts the 256 MB MALL and the L2 (cold). f = t_roof / t_warm "
         "with t_roof = max(flops / peak, compulsory bytes / bandwidth); compulsory bytes read "
         "every input and write every output once (the gather's KV rows at most once). The "
         "gather's per-token selected KV rows (each token's rows once, shared by its 64 heads) "
         "are served largely from L2 and the MALL; their rate is listed after the table, not "
         "used as a bound.\n",
         "| Workload | Kernel | Warm ms | Cold ms | TFLOP | Alg. GB | Bound | TFLOP/s | GB/s (alg.) | f vendor | f measured peak |",
         "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in results:
        for k, v in r["kernels"].items():
            fm = "—" if v["frac_measured_peak"] is None else f"{v['frac_measured_peak']:.3f}"
            ts = "—" if v["tflop_s"] is None else f"{v['tflop_s']:.1f}"
            L.append(f"| {r['workload']} | {k} | {v['ms_warm']:.4f} | {v['ms_cold']:.4f} | "
                     f"{v['tflop']:.3f} | {v['gb_alg']:.3f} | {v['bound']} | {ts} | {v['gb_s_alg']:.0f} | "
                     f"{v['frac_vendor']:.3f} | {fm} |")
    L.append("")
    L.append("Gather, per-token selected KV rows (served largely from L2 and the MALL, not HBM "
             "traffic): " + "; ".join(
                 f"{r['workload']} {r['kernels']['sparse_gather']['gb_s_per_token_kv_l2_served']:.0f} GB/s"
                 for r in results if "gb_s_per_token_kv_l2_served" in r["kernels"].get("sparse_gather", {}))
             + ".\n")
    L.append("`*_bwd` are the gradient calls (dq, dkv and the sink gradient) of the three attention "
             "operations, each fed its own forward outputs; their flops are 2 (3 Dk + 2 Dv) per "
             "(query-head, key) pair (score recomputed, dP, dQ, dK, dV) and their bytes count q, the "
             "KV rows, out, dout, lse and the fp32 dq and dkv. With the larger workspaces used here "
             "the bf16 calls store the score gradients and execute exactly the counted flops; the "
             "fp32 shapes recompute the scores and dP in both of their kernels, 1.4 times the "
             "counted flops.\n")
    L.append("`swa_sparse` is `hs_swa_sparse_fwd`: the window and the selected-block branches of a "
             "sliding-window layer in one call (separate outputs), its work the sum of `swa` and "
             "`sparse_gather`.\n")
    L.append("`score_topk_fused` is `hs_block_score_topk_fwd` (block scores and the top-k in one call; "
             "its work is counted as the block score's). Metric path (block score + top-k + gather; "
             "with the fused call in place of the first two) and the float64 oracle on the host:\n")
    L.append("| Workload | Path ms | Path ms, fused | tokens/s | TFLOP/s | Oracle tokens/s | Oracle rows | Oracle full-run s |")
    L.append("|---|---|---|---|---|---|---|---|")
    for r in results:
        o = r.get("oracle")
        if o:
            ot = f"{o['tokens_s']} ({o['threads']} threads)"
            extra = r.get("oracle_1_thread")
            if extra:
                ot += f"; {extra['tokens_s']} (1 thread)"
            orow = f"{o['rows']}{'' if o['full'] else ' (sample)'}"
            ofull = f"{o['full_run_s']} ({o['full_run_s_is']})"
        else:
            ot = orow = ofull = "—"
        L.append(f"| {r['workload']} | {r['metric_path_ms']:.3f} | {r['fused_path_ms']:.3f} | {r['tokens_s']:.0f} | "
                 f"{r['metric_tflop_s']:.1f} | {ot} | {orow} | {ofull} |")
    L.append("")
    with open(path, "w") as f:
        f.write("\n".join(L))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=3, help="named workload (1-5); 3 is the metric's")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gradients", action="store_true",
                    help="skip timing the gradient calls after the metric's timed region")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one 1 GiB device copy (counter calibration)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured by counters, if recorded")
    ap.add_argument("--suite", action="store_true",
                    help="measure every named workload and kernel (warm, cold, rooflines) instead "
                         "of the metric line")
    ap.add_argument("--suite-workloads", type=int, nargs="+", default=[1, 2, 3, 4, 5])
    ap.add_argument("--suite-md", default=None, help="also write the suite as a markdown table")
    ap.add_argument("--oracle-budget", type=float, default=20.0,
                    help="seconds of oracle time per workload in the suite (0 = skip)")
    ap.add_argument("--oracle-full", action="store_true",
                    help="suite: run the oracle over every row of every workload (no sampling; "
                         "the S=32768 workload takes about an hour on 16 cores)")
    ap.add_argument("--oracle-full-for", type=int, nargs="+", default=None,
                    help="suite: run the oracle over every row of these workloads only")
    args = ap.parse_args()
    if args.oracle_full:
        args.oracle_budget = float("inf")

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the path is built and measured on a single "
              "MI355X; multi-GPU runs are not supported.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.suite:
        run_suite(args)
        return

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

    # Gradient calls of the three attention operations, each fed its own
    # forward outputs, timed after (and outside) the metric's timed region.
    grads = None
    if not args.no_gradients:
        dout = inputs.make_dout(p, seed=900 + args.workload).to(dev)
        dq = torch.empty((p.B, p.Sq, p.H, p.Dk), dtype=torch.float32, device=dev)
        dkv = torch.empty((p.B, p.Skv, p.Dk), dtype=torch.float32, device=dev)
        dsink = torch.empty((p.H,), dtype=torch.float32, device=dev)
        wb1 = hs.score_bwd_workspace(prob, store_ds=True)
        stored = wb1.numel() * 4 >= hs.hs_workspace_size(prob, hs.HS_OP_BLOCK_SCORE_BWD_STORE_DS)
        wb3 = hs.sparse_gather_bwd_workspace(prob, p.top_k, store_ds=True)
        stored3 = wb3.numel() * 4 >= hs.hs_workspace_size(prob, hs.HS_OP_SPARSE_GATHER_BWD_STORE_DS,
                                                          top_k=p.top_k)
        wb4 = hs.swa_bwd_workspace(prob, p.window, store_ds=True)
        stored4 = wb4.numel() * 4 >= hs.hs_workspace_size(prob, hs.HS_OP_SWA_BWD_STORE_DS,
                                                          window=p.window)
        gcalls = {
            "block_score_bwd": lambda: hs.hs_block_score_bwd(
                prob, q, kv, sink, out, lse, dout, dq, dkv, dsink, wb1, stream),
            "sparse_gather_bwd": lambda: hs.hs_sparse_gather_bwd(
                prob, q, kv, sink, idx, p.top_k, og, lg, dout, dq, dkv, dsink, wb3, stream),
            "swa_bwd": lambda: hs.hs_swa_bwd(
                prob, q, kv, sink, p.window, osw, lsw, dout, dq, dkv, dsink, wb4, stream)}
        grads = {"ms": {}, "block_score_bwd_dq": "stored dS" if stored else "recomputed dS",
                 "sparse_gather_bwd_dq": "stored dS" if stored3 else "recomputed dS",
                 "swa_bwd_dq": "stored dS" if stored4 else "recomputed dS"}
        for k, fn in gcalls.items():
            fn()
            torch.cuda.synchronize()
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            for _ in range(3):
                fn()
            g1.record(stream)
            torch.cuda.synchronize()
            grads["ms"][k] = round(g0.elapsed_time(g1) / 3, 4)
        del dout, dq, dkv, wb1, wb3, wb4
        torch.cuda.empty_cache()

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

    # Compulsory HBM bytes (each input read once, each output written once).
    es = 2 if p.dtype == "bf16" else 4
    qb = tokens * p.H * p.Dk * es
    ob = tokens * p.H * p.Dv * es
    lb = tokens * p.H * 4
    kvb = p.B * p.Skv * p.Dk * es
    c_score = qb + kvb + ob + lb + tokens * NB * 4
    c_topk = tokens * (NB + p.top_k) * 4
    c_gather = qb + kvb + ob + lb + tokens * p.top_k * 4
    c_swa = qb + kvb + ob + lb
    tr = lambda k: counter_traffic(args.traffic_json, p.name, k)
    rooflines = {
        "block_score": roofline_entry("block_score (hs_block_score_fwd)", f_score, c_score,
                                      float(k_ms[0]), tr("block_score")),
        "topk": roofline_entry("topk (hs_topk_blocks)", 0, c_topk, float(k_ms[1]), tr("topk")),
    }
    if f_gather:
        # Per-token selected KV rows, each token's gather counted once (shared by its
        # heads): bytes the method moves per token, served largely from L2 and the
        # MALL (the whole KV is 37.7 MB), so they are reported, not used as the bound.
        l2 = gather_pairs_from_idx(p, idx_cpu) // p.H * p.Dk * es + qb + ob + lb
        rooflines["sparse_gather"] = roofline_entry(
            "sparse_gather (hs_sparse_gather_fwd)", f_gather, c_gather, float(k_ms[2]),
            tr("sparse_gather"), per_token_kv_bytes_l2_served=int(l2),
            per_token_kv_rate_gb_s=round(l2 / (k_ms[2] * 1e-3) / 1e9, 1))
    if f_swa:
        rooflines["swa"] = roofline_entry("swa (hs_swa_fwd)", f_swa, c_swa, swa_ms, tr("swa"))

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
        "roofline": {k: v for k, v in rooflines["block_score"].items()
                     if k in ("kernel", "bound", "achieved", "peak", "unit", "frac", "traffic")},
        "rooflines": rooflines,
    }
    if grads is not None:
        # 2 (3 Dk + 2 Dv) flops per pair: score recomputed, dP, dQ, dK, dV.
        fpb = 2 * (3 * p.Dk + 2 * p.Dv)
        f_bwd = causal_pairs(p) * fpb
        t = grads["ms"]["block_score_bwd"]
        grads["flop_per_pair"] = fpb
        grads["block_score_bwd_tflop_s"] = round(f_bwd / (t * 1e-3) / 1e12, 2)
        grads["block_score_bwd_frac"] = round(f_bwd / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        # the gather and the window over the same (head, key) pairs as their
        # forward calls (forward flops / (2 Dk + 2 Dv) pairs)
        for name, f_fwd in (("sparse_gather_bwd", f_gather), ("swa_bwd", f_swa)):
            if f_fwd and name in grads["ms"]:
                fb = f_fwd / (2 * (p.Dk + p.Dv)) * fpb
                rate = fb / (grads["ms"][name] * 1e-3) / 1e12
                grads[name + "_tflop_s"] = round(rate, 2)
                grads[name + "_frac"] = round(rate / PEAK_BF16_TFLOPS, 4)
        res["gradients"] = grads
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(p, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
