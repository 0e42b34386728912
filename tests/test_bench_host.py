"""Host-side arithmetic of bench.py, checked on the CPU: the algorithmic pair
counts behind TFLOP/s (against a count of the oracle's allowed-key masks),
the roofline object (bound, achieved rate, fraction), the counter-traffic
record's staleness check, and the single-GPU guard."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_sparse_mqa_amd import inputs  # noqa: E402
from oracle import hysparse_ref as ref  # noqa: E402


def _mask_pairs(kind, p, window=None, block_idx=None):
    """(query head, key) pairs the oracle lets attend, counted entry by entry."""
    n = 0
    for _, _, _, _, _, allowed, _ in ref._chunk_masks(
            kind, p.B, p.Sq, p.Skv, p.H, p.block_size, p.kv_lens, p.doc_start, p.doc_end,
            window, block_idx, np.arange(p.Sq), None):
        n += int(allowed.sum())
    return n * p.H


def _small(S, docs=None, seed=3):
    p = inputs.make(1, S, S, 4, 16, 8, seed=seed, top_k=3, window=37, dtype="f32",
                    name=f"bench_host_{S}")
    if docs is not None:
        starts = np.cumsum([0] + docs[:-1]).tolist()
        p.doc_start, p.doc_end = starts, [s + L for s, L in zip(starts, docs)]
    return p


@pytest.mark.parametrize("S", [1, 63, 64, 200, 333])
def test_causal_and_window_pairs_match_the_oracle_masks(S):
    p = _small(S)
    assert bench.causal_pairs(p) == _mask_pairs("block_score", p)
    assert bench.swa_pairs(p) == _mask_pairs("swa", p, window=p.window)


def test_causal_pairs_with_documents_match_the_oracle_masks():
    p = _small(300, docs=[100, 33, 167])
    assert bench.causal_pairs(p) == _mask_pairs("block_score", p)


@pytest.mark.parametrize("S", [64, 200, 333])
def test_gather_pairs_match_the_oracle_masks(S):
    """Selections with -1 entries, blocks past the row's position and the
    row's own partial block."""
    p = _small(S)
    nb = (S + 63) // 64
    rng = np.random.default_rng(S)
    idx = np.stack([rng.permutation(max(nb, 3))[:3] for _ in range(S)])[None].astype(np.int32)
    idx[idx >= nb] = -1
    idx[0, ::5, 0] = -1
    assert bench.gather_pairs_from_idx(p, idx) == _mask_pairs("gather", p, block_idx=idx)


def test_flops_per_pair_is_two_dk_plus_two_dv():
    p = inputs.make(1, 8, 8, 64, 576, 512, seed=0, top_k=1, window=8, name="fpp")
    assert bench.flops_per_pair(p) == 2176


def test_roofline_entry_takes_the_binding_resource():
    # 2.5 TFLOP in 2 ms: MFMA-bound (1 ms at peak against 0.5 ms for 4 GB)
    r = bench.roofline_entry("k", 2.5e12, 4e9, 2.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1250.0) and r["frac"] == pytest.approx(0.5)
    # 8 GB with little arithmetic in 4 ms: HBM-bound (1 ms at peak)
    r = bench.roofline_entry("k", 1e9, 8e9, 4.0, traffic=123)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["traffic"] == 123
    assert r["achieved"] == pytest.approx(2000.0) and r["frac"] == pytest.approx(0.25)


def test_counter_traffic_is_dropped_when_a_source_changes(tmp_path):
    import hashlib
    src = tmp_path / "kernel.hip"
    src.write_bytes(b"// kernel v1\n")
    rec = {"w": {"k": {"bytes_per_launch": 4096, "sources": [str(src)],
                       "sources_sha256_16": hashlib.sha256(b"// kernel v1\n").hexdigest()[:16]}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    assert bench.counter_traffic(str(path), "w", "k") == 4096
    assert bench.counter_traffic(str(path), "w", "other") is None
    assert bench.counter_traffic(str(path), "other", "k") is None
    src.write_bytes(b"// kernel v2\n")
    assert bench.counter_traffic(str(path), "w", "k") is None
    assert bench.counter_traffic(str(tmp_path / "missing.json"), "w", "k") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""
