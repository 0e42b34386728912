"""Seeded random GPU parity cases: ragged shapes the hand-picked cases do not
pin down. Each case draws a kind (one sequence, a batch of entries with their
own cache lengths, packed documents, or single-token decode), its sizes, top-k,
window and whether a sink is passed, then runs the four calls against the
oracle exactly as the fixed cases do, checks that the fused block score +
top-k call writes what the two separate calls write, and checks the gradients
of the three attention calls against the oracle's. The bf16 cases use the
absorbed-MLA shape, the fp32 cases the small shape (8 heads, Dk 96, Dv 64)."""
import numpy as np
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs

from gpu_common import Dev, np64, say
from test_gpu_bwd import _gpu_grads, _grad_close, _oracle_grads
from test_gpu_parity import MLA, _run_all

pytestmark = pytest.mark.gpu

N_BF16, N_F32 = 16, 4


def _draw(i: int):
    rng = np.random.default_rng(7000 + i)
    f32 = i >= N_BF16
    kind = ("single", "batch", "docs", "decode")[i % 4]
    kw = dict(seed=7000 + i, top_k=int(rng.integers(1, 13)), window=int(rng.integers(1, 400)),
              sink=bool(rng.integers(0, 2)), name=f"random_{i}_{kind}")
    cap = 300 if f32 else 700
    if kind == "single":
        S = int(rng.integers(1, cap))
        B, Sq, Skv, lens, docs = 1, S, S, None, None
    elif kind == "batch":
        B = int(rng.integers(2, 5))
        Skv = int(rng.integers(64, cap))
        lens = [int(x) for x in rng.integers(1, Skv + 1, size=B)]
        Sq = int(rng.integers(1, min(lens) + 1))
        docs = None
    elif kind == "docs":
        S = int(rng.integers(2, cap))
        n = int(rng.integers(1, min(8, S) + 1))
        cuts = sorted(rng.choice(np.arange(1, S), size=n - 1, replace=False).tolist()) if n > 1 else []
        edges = [0] + cuts + [S]
        docs = [edges[k + 1] - edges[k] for k in range(n)]
        B, Sq, Skv, lens = 1, S, S, None
    else:
        B = int(rng.integers(2, 9))
        Skv = int(rng.integers(64, 3000))
        lens = [int(x) for x in rng.integers(1, Skv + 1, size=B)]
        Sq, docs = 1, None
    if f32:
        p = inputs.make(B, Sq, Skv, 8, 96, 64, dtype="f32", kv_lens=lens, doc_lens=docs, **kw)
    else:
        p = inputs.make(B, Sq, Skv, MLA["H"], MLA["Dk"], MLA["Dv"], kv_lens=lens, doc_lens=docs,
                        **kw)
    return p


@pytest.mark.parametrize("i", list(range(N_BF16 + N_F32)))
def test_random_case(i):
    p = _draw(i)
    say(f"[gpu] random case {i}: {p.name} B={p.B} Sq={p.Sq} Skv={p.Skv} kv_lens={p.kv_lens} "
        f"docs={None if p.doc_start is None else len(p.doc_start)} top_k={p.top_k} "
        f"window={p.window} sink={p.sink is not None} dtype={p.dtype}")
    d = Dev(p, sink=p.sink is not None)
    res = _run_all(d)
    out, lse, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    fused = hs.block_score_topk(d.prob, d.q, d.kv, d.sink, p.top_k)
    torch.cuda.synchronize()
    for n, f, s in zip(("out", "lse", "block_logit", "block_idx"), fused, (out, lse, bl, idx)):
        assert torch.equal(f, s), f"fused {n} differs from the separate calls"
    dout_cpu = inputs.make_dout(p, seed=7500 + i)
    dout = dout_cpu.cuda()
    idx_cpu = idx.cpu().numpy()
    for op in ("score", "swa", "gather"):
        g = _gpu_grads(d, op, dout, idx, p.top_k)
        torch.cuda.synchronize()
        w = _oracle_grads(d, op, dout_cpu, idx_cpu)
        for k, name in enumerate(("dq", "dkv", "dsink")):
            if w[k] is None:
                assert g[k] is None
            else:
                res[f"{op}_{name}"] = _grad_close(np64(g[k]), w[k], p.dtype, f"{op} {name}")
    say(f"[gpu] random case {i}: {res}")
