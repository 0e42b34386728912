"""GPU parity at the documented limits of the C ABI and in the degenerate
cases of the method: 256 batch entries, 64 packed documents, 4096 key blocks
in top-k, top-k 64 end to end, and gather rows whose selection is empty,
out of range or outside the row's allowed keys."""
import numpy as np
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs
from oracle import hysparse_ref as ref

from gpu_common import Dev, assert_close, np64, say, tol_for
from test_gpu_parity import MLA, _run_all

pytestmark = pytest.mark.gpu


def test_max_batch_entries_prefill_chunks():
    """B = 256 (the cap), 8 query rows per entry at the end of caches of
    ragged length: every entry is its own chunked prefill."""
    rng = np.random.default_rng(31)
    lens = [int(x) for x in rng.integers(8, 81, size=256)]
    say(f"[gpu] B=256 chunked prefill, cache lengths {min(lens)}..{max(lens)}")
    p = inputs.make(256, 8, 80, MLA["H"], MLA["Dk"], MLA["Dv"], seed=31, kv_lens=lens, top_k=2,
                    window=20, name="b256_prefill")
    res = _run_all(Dev(p))
    say(f"[gpu] B=256 prefill: {res}")


def test_max_batch_entries_decode_split():
    """B = 256 single-token rows: the decode path with split key ranges."""
    rng = np.random.default_rng(32)
    lens = [int(x) for x in rng.integers(1, 513, size=256)]
    say("[gpu] B=256 decode")
    p = inputs.make(256, 1, 512, MLA["H"], MLA["Dk"], MLA["Dv"], seed=32, kv_lens=lens, top_k=3,
                    window=100, name="b256_decode")
    res = _run_all(Dev(p))
    say(f"[gpu] B=256 decode: {res}")


def test_max_documents():
    """64 packed documents (the cap) of 1..40 rows."""
    rng = np.random.default_rng(33)
    docs = [int(x) for x in rng.integers(1, 41, size=64)]
    S = sum(docs)
    say(f"[gpu] 64 documents, S={S}")
    p = inputs.make(1, S, S, MLA["H"], MLA["Dk"], MLA["Dv"], seed=33, doc_lens=docs, top_k=4,
                    window=30, name="docs64")
    res = _run_all(Dev(p))
    say(f"[gpu] 64 documents: {res}")


def test_topk_max_blocks():
    """NB = 4096 columns (the top-k cap) with K = 1, 33 and 64, ties and -inf."""
    say("[gpu] top-k with 4096 blocks")
    rng = np.random.default_rng(34)
    Sq, Skv = 3, 4096 * 64
    prob = hs.Problem(1, Sq, Skv, 64, 576, 512)
    NB = hs.hs_num_blocks(prob)
    assert NB == 4096
    bl = rng.choice([0.5, -1.0, 3.0, 2.0], size=(1, Sq, NB)).astype(np.float32)
    bl[0, 1] = rng.standard_normal(NB).astype(np.float32)
    bl[0, 2, ::2] = -np.inf
    own = ref.own_blocks(1, Sq, Skv, 64)
    for K in (1, 33, 64):
        idx = hs.topk_blocks(prob, torch.from_numpy(bl).cuda(), K)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref.topk_blocks(bl, own, K)), K


def test_topk64_end_to_end_sampled():
    """top_k = 64 (the cap) through block scores, top-k and the gather."""
    say("[gpu] top-k 64 end to end, S=8192")
    p = inputs.make(1, 8192, 8192, MLA["H"], MLA["Dk"], MLA["Dv"], seed=35, top_k=64,
                    window=256, name="topk64")
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(8192 - 64, 8192),
                                     np.random.default_rng(35).integers(0, 8192, 64)]))
    res = _run_all(Dev(p), rows=rows)
    say(f"[gpu] top-k 64: {res}")


@pytest.mark.parametrize("sink", [True, False])
def test_gather_degenerate_selections(sink):
    """Rows whose selection is all -1 (empty set: only the sink remains),
    holds indices >= NB, or lists blocks after the row (no allowed key)."""
    say(f"[gpu] gather degenerate selections, sink={sink}")
    p = inputs.make(1, 300, 300, MLA["H"], MLA["Dk"], MLA["Dv"], seed=36, top_k=4, window=64,
                    sink=sink, name="gather_degenerate")
    d = Dev(p, sink=sink)
    NB = hs.hs_num_blocks(d.prob)
    rng = np.random.default_rng(36)
    idx = np.full((1, p.Sq, p.top_k), -1, dtype=np.int32)
    for r in range(p.Sq):
        kind = r % 4
        own = r // 64
        if kind == 0:
            continue                                          # empty selection
        if kind == 1:
            idx[0, r, :2] = [own, NB + 3]                     # out of range skipped
        elif kind == 2:
            fut = [j for j in range(own + 1, NB)][:2]         # blocks after the row
            idx[0, r, :len(fut)] = fut
        else:
            c = sorted(set(rng.integers(0, own + 1, size=3).tolist()) | {own})
            idx[0, r, :len(c)] = c[:p.top_k]
    out, lse = hs.sparse_gather(d.prob, d.q, d.kv, d.sink, torch.from_numpy(idx).cuda(), p.top_k)
    torch.cuda.synchronize()
    o_ref, l_ref = ref.sparse_gather(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, idx.astype(np.int64),
                                     **d.kw())
    tol = tol_for(p)
    e_o = assert_close(np64(out), o_ref, tol, "gather out")
    e_l = assert_close(np64(lse), l_ref, tol, "gather lse")
    empty = np64(out)[0, 0::4]
    assert np.all(empty == 0.0), "empty selections must give zero output"
    if not sink:
        assert np.all(np.isneginf(np64(lse)[0, 0::4])), "empty selection without sink: lse = -inf"
    say(f"[gpu] degenerate gather sink={sink}: out {e_o:.2e} lse {e_l:.2e}")
