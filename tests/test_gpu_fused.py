"""GPU checks of hs_block_score_topk_fwd, the block scores and the per-token
top-k in one call. It runs the same kernels as hs_block_score_fwd followed by
hs_topk_blocks, so its outputs are compared bit for bit with those two calls;
its selection is also compared exactly with the oracle's top-k on the same
fp32 block scores. Covered: split decode (the top-k runs inside the merge
launch) with few and many blocks per row, a short prefill that splits too,
a prefill that does not split (the top-k kernel follows), the fp32 shape,
and paged decode with device lengths inside a captured graph."""
import numpy as np
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs
from oracle import hysparse_ref as ref

from gpu_common import Dev, say
from test_gpu_paged import _paged
from test_gpu_parity import MLA

pytestmark = pytest.mark.gpu


def _check_same(fused, separate, own, K, tag):
    names = ("out", "lse", "block_logit", "block_idx")
    for n, f, s in zip(names, fused, separate):
        assert torch.equal(f, s), f"{tag}: fused {n} differs from the separate calls"
    want = ref.topk_blocks(separate[2].cpu().numpy().astype(np.float64), own, K)
    assert np.array_equal(fused[3].cpu().numpy(), want), f"{tag}: selection differs from the oracle"


CASES = {
    # name: (B, Sq, Skv, kv_lens, top_k, dtype)
    "decode_split_NB79": (16, 1, 5000, "rand", 8, "bf16"),
    "decode_split_NB625": (4, 1, 40000, "rand", 32, "bf16"),
    "prefill_split": (2, 48, 3000, [3000, 1000], 4, "bf16"),
    "prefill_nosplit": (1, 1024, 1024, None, 16, "bf16"),
    "tiny_f32": (1, 512, 512, None, 4, "f32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_matches_separate_calls(name):
    B, Sq, Skv, lens, K, dtype = CASES[name]
    say(f"[gpu] fused score+top-k {name}")
    if lens == "rand":
        lens = [int(x) for x in np.random.default_rng(51).integers(1, Skv + 1, size=B)]
    if dtype == "f32":
        p = inputs.make(B, Sq, Skv, 8, 96, 64, dtype="f32", seed=52, kv_lens=lens, top_k=K,
                        name=name)
    else:
        p = inputs.make(B, Sq, Skv, MLA["H"], MLA["Dk"], MLA["Dv"], seed=52, kv_lens=lens,
                        top_k=K, name=name)
    d = Dev(p)
    split = hs.hs_workspace_size(d.prob, hs.HS_OP_BLOCK_SCORE) > 0
    out, lse, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, K)
    fused = hs.block_score_topk(d.prob, d.q, d.kv, d.sink, K)
    torch.cuda.synchronize()
    _check_same(fused, (out, lse, bl, idx), d.own(), K, name)
    say(f"[gpu] fused {name}: split={split}, NB={hs.hs_num_blocks(d.prob)}, identical")


def test_fused_paged_device_lengths_in_graph():
    """The merge launch reads device lengths for the own block: a captured
    graph of the fused call replayed at new lengths matches the separate calls."""
    say("[gpu] fused score+top-k, paged, device lengths, captured graph")
    B, cap, K = 8, 2048, 6
    rng = np.random.default_rng(53)
    p = inputs.make(B, 1, cap, MLA["H"], MLA["Dk"], MLA["Dv"], seed=53, kv_lens=[cap] * B,
                    top_k=K, name="fused_paged")
    pool, pt = _paged(p, seed=54)
    pool, pt = pool.cuda(), pt.cuda()
    q, sink = p.q.cuda(), p.sink.cuda()
    lens_dev = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    prob = hs.Problem(B, 1, cap, p.H, p.Dk, p.Dv, page_table=pt, kv_lens_device=lens_dev)
    NB = hs.hs_num_blocks(prob)
    out = torch.empty((B, 1, p.H, p.Dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 1, p.H), dtype=torch.float32, device="cuda")
    bl = torch.empty((B, 1, NB), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, 1, K), dtype=torch.int32, device="cuda")
    ws = hs._workspace(prob, hs.HS_OP_BLOCK_SCORE)
    assert ws is not None, "decode must take the split path here"

    def fused_call():
        hs.hs_block_score_topk_fwd(prob, q, pool, sink, K, out, lse, bl, idx, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fused_call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        fused_call()
    torch.cuda.synchronize()
    for rep in range(3):
        lens = [int(x) for x in rng.integers(1, cap + 1, size=B)]
        lens_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        idx.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone(), bl.clone(), idx.clone())
        o2, l2, b2 = hs.block_score(prob, q, pool, sink)
        i2 = hs.topk_blocks(prob, b2, K)
        torch.cuda.synchronize()
        own = ref.own_blocks(B, 1, cap, 64, kv_lens=lens)
        _check_same(got, (o2, l2, b2, i2), own, K, f"replay {rep}")
        say(f"[gpu] fused graph replay {rep} lengths {min(lens)}..{max(lens)}: identical")


@pytest.mark.parametrize("name", list(CASES))
def test_normalised_block_scores(name):
    """The optional block_prob output: equal to the oracle's block_prob on the
    GPU's own block scores and lse (same inputs, rounding of exp only), and to
    the oracle's from its own float64 scores within the block-score and lse
    tolerances; the fused call's other outputs are unchanged by it."""
    B, Sq, Skv, lens, K, dtype = CASES[name]
    say(f"[gpu] normalised block scores {name}")
    if lens == "rand":
        lens = [int(x) for x in np.random.default_rng(53).integers(1, Skv + 1, size=B)]
    if dtype == "f32":
        p = inputs.make(B, Sq, Skv, 8, 96, 64, dtype="f32", seed=54, kv_lens=lens, top_k=K,
                        name=name)
    else:
        p = inputs.make(B, Sq, Skv, MLA["H"], MLA["Dk"], MLA["Dv"], seed=54, kv_lens=lens,
                        top_k=K, name=name)
    d = Dev(p)
    plain = hs.block_score_topk(d.prob, d.q, d.kv, d.sink, K)
    out, lse, bl, idx, pr = hs.block_score_topk(d.prob, d.q, d.kv, d.sink, K, with_prob=True)
    torch.cuda.synchronize()
    for n, a, b in zip(("out", "lse", "block_logit", "block_idx"), (out, lse, bl, idx), plain):
        assert torch.equal(a, b), f"{name}: {n} changed by the block_prob output"
    got = pr.cpu().numpy().astype(np.float64)
    same = ref.block_prob(bl.cpu().numpy(), lse.cpu().numpy())
    e_same = float(np.abs(got - same).max())
    assert e_same <= 1e-5, e_same
    rows = None if p.B * p.Sq <= 4096 else np.arange(0, p.Sq, 7)
    _, l_ref, b_ref = ref.block_score(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, rows=rows, **d.kw())
    want = ref.block_prob(b_ref, l_ref)
    sel = slice(None) if rows is None else rows
    e_ref = float(np.abs(got[:, sel] - want).max())
    assert e_ref <= 1e-3, e_ref
    assert (got >= 0).all() and (got <= 1 + 1e-6).all()
    say(f"[gpu] block_prob {name}: vs own scores {e_same:.2e}, vs oracle {e_ref:.2e}")
