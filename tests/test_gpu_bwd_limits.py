"""GPU parity of the gradient calls at the documented limits of the C ABI:
256 batch entries, 64 packed documents, and a gather over 4096 key blocks
with top-k 64 (the size of the per-tile row-count table)."""
import numpy as np
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs

from gpu_common import Dev, np64, say
from test_gpu_bwd import _gpu_grads, _grad_close, _oracle_grads
from test_gpu_parity import MLA

pytestmark = pytest.mark.gpu


def _all_ops(p, seed, ops=("score", "swa", "gather")):
    d = Dev(p)
    dout_cpu = inputs.make_dout(p, seed=seed)
    dout = dout_cpu.cuda()
    _, _, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    torch.cuda.synchronize()
    idx_cpu = idx.cpu().numpy()
    res = {}
    for op in ops:
        g = _gpu_grads(d, op, dout, idx, p.top_k)
        torch.cuda.synchronize()
        w = _oracle_grads(d, op, dout_cpu, idx_cpu)
        for k, name in enumerate(("dq", "dkv", "dsink")):
            res[f"{op}_{name}"] = _grad_close(np64(g[k]), w[k], p.dtype, f"{op} {name}")
    return res


def test_gradients_max_batch_entries():
    """B = 256 (the cap), 8 query rows per entry at the end of caches of
    ragged length; rows of kv past each length get zero gradient."""
    rng = np.random.default_rng(61)
    lens = [int(x) for x in rng.integers(8, 81, size=256)]
    say(f"[gpu] gradients B=256, cache lengths {min(lens)}..{max(lens)}")
    p = inputs.make(256, 8, 80, MLA["H"], MLA["Dk"], MLA["Dv"], seed=61, kv_lens=lens, top_k=2,
                    window=20, name="b256_grad")
    res = _all_ops(p, seed=62)
    say(f"[gpu] gradients B=256: {max(res.values()):.2e} worst")


def test_gradients_max_documents():
    """64 packed documents (the cap) of 1..40 rows."""
    rng = np.random.default_rng(63)
    docs = [int(x) for x in rng.integers(1, 41, size=64)]
    S = sum(docs)
    say(f"[gpu] gradients, 64 documents, S={S}")
    p = inputs.make(1, S, S, MLA["H"], MLA["Dk"], MLA["Dv"], seed=63, doc_lens=docs, top_k=4,
                    window=30, name="docs64_grad")
    res = _all_ops(p, seed=64)
    say(f"[gpu] gradients 64 documents: {max(res.values()):.2e} worst")


def test_gather_gradients_max_blocks_and_topk():
    """Eight query rows at the end of a 4096-block cache (the row-list table's
    cap), each selecting 64 blocks (the top-k cap): 63 chosen at random plus
    its own block."""
    say("[gpu] gather gradients, 4096 blocks, top-k 64")
    L = 4096 * 64
    p = inputs.make(1, 8, L, MLA["H"], MLA["Dk"], MLA["Dv"], seed=65, kv_lens=[L], top_k=64,
                    window=64, name="gather_4096_blocks")
    d = Dev(p)
    rng = np.random.default_rng(66)
    idx = np.empty((1, 8, 64), dtype=np.int32)
    for r in range(8):
        own = (L - 8 + r) // 64
        others = rng.choice(np.arange(own), size=63, replace=False)
        idx[0, r] = np.sort(np.append(others, own))
    idx_dev = torch.from_numpy(idx).cuda()
    dout_cpu = inputs.make_dout(p, seed=67)
    g = _gpu_grads(d, "gather", dout_cpu.cuda(), idx_dev, 64)
    torch.cuda.synchronize()
    w = _oracle_grads(d, "gather", dout_cpu, idx)
    errs = [_grad_close(np64(g[k]), w[k], "bf16", f"gather {n}")
            for k, n in enumerate(("dq", "dkv", "dsink"))]
    say(f"[gpu] gather gradients, 4096 blocks: {max(errs):.2e} worst")
