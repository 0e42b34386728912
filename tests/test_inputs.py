"""Seeded input recipe: shapes, determinism and the structured workloads."""
import math

import torch

from block_sparse_mqa_amd import inputs


def test_tiny_config_shapes_and_determinism():
    a = inputs.config(1)
    b = inputs.config(1)
    assert a.q.shape == (1, 512, 8, 96) and a.kv.shape == (1, 512, 96)
    assert a.q.dtype == torch.float32 and a.sink.shape == (8,)
    assert torch.equal(a.q, b.q) and torch.equal(a.kv, b.kv) and torch.equal(a.sink, b.sink)
    assert abs(a.scale - 1 / math.sqrt(96)) < 1e-15


def test_packed_document_lengths():
    g = torch.Generator().manual_seed(4)
    lens = inputs.doc_lengths_packed(g)
    assert len(lens) == 8 and sum(lens) == 16384
    assert all(512 <= L <= 4096 for L in lens[:-1]) and 64 <= lens[-1] <= 4096


def test_custom_problem_nan_past_cache_and_scaled_blocks():
    p = inputs.make(2, 1, 200, 4, 16, 8, seed=3, kv_lens=[130, 200])
    assert torch.isnan(p.kv[0, 130:].float()).all() and torch.isfinite(p.kv[0, :130].float()).all()
    assert torch.isfinite(p.kv[1].float()).all()
    s = inputs.make(1, 256, 256, 2, 16, 8, seed=5, scaled_block_every=4, kv_mult=1.0, dtype="f32")
    r = s.kv[0].pow(2).mean(dim=1).view(4, 64).mean(dim=1)
    assert r[0] > 4 * r[1] and r[0] > 4 * r[2] and r[0] > 4 * r[3]
