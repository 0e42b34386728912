"""GPU parity of paged KV: the key blocks of each entry live in shuffled pages
of a pool (one 64-row block per page) and the four calls must equal the
oracle on the logical, contiguous cache. Unused pages hold NaN, so a read of
a wrong page shows up as a NaN or an error."""
import numpy as np
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs
from oracle import hysparse_ref as ref

from gpu_common import assert_close, check_topk_margin, np64, say, tol_for
from test_gpu_parity import MLA

pytestmark = pytest.mark.gpu


def _paged(p, seed, spare=7):
    """Pool [n_pages, 64, Dk] and page table [B, max_pages] for problem p."""
    B, Skv, BS = p.B, p.Skv, p.block_size
    max_pages = (Skv + BS - 1) // BS
    n_pages = B * max_pages + spare
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_pages)[:B * max_pages].reshape(B, max_pages)
    pool = torch.full((n_pages, BS, p.Dk), float("nan"), dtype=torch.bfloat16)
    for b in range(B):
        L = p.kv_lens[b] if p.kv_lens else Skv
        for j in range((L + BS - 1) // BS):
            rows = p.kv[b, j * BS:min((j + 1) * BS, L)]
            pool[perm[b, j], :rows.shape[0]] = rows
    return pool, torch.from_numpy(perm.astype(np.int32))


@pytest.mark.parametrize("case", ["decode", "chunked_prefill"])
def test_paged_kv_matches_contiguous(case):
    say(f"[gpu] paged KV {case}")
    if case == "decode":
        lens = [int(x) for x in np.random.default_rng(41).integers(1, 3000, size=12)]
        p = inputs.make(12, 1, 3000, MLA["H"], MLA["Dk"], MLA["Dv"], seed=41, kv_lens=lens,
                        top_k=5, window=300, name="paged_decode")
    else:
        lens = [700, 333, 1100]
        p = inputs.make(3, 200, 1100, MLA["H"], MLA["Dk"], MLA["Dv"], seed=42, kv_lens=lens,
                        top_k=4, window=150, name="paged_prefill")
    pool, pt = _paged(p, seed=43)
    pool, pt = pool.cuda(), pt.cuda()
    q, sink = p.q.cuda(), p.sink.cuda()
    prob = hs.Problem(p.B, p.Sq, p.Skv, p.H, p.Dk, p.Dv, kv_lens=p.kv_lens, page_table=pt)
    out, lse, bl = hs.block_score(prob, q, pool, sink)
    idx = hs.topk_blocks(prob, bl, p.top_k)
    og, lg = hs.sparse_gather(prob, q, pool, sink, idx, p.top_k)
    osw, lsw = hs.swa(prob, q, pool, sink, p.window)
    torch.cuda.synchronize()
    kw = dict(block_size=p.block_size, kv_lens=p.kv_lens)
    tol = tol_for(p)
    o_ref, l_ref, b_ref = ref.block_score(p.q, p.kv, p.sink, p.Dv, p.scale, **kw)
    res = {"out": assert_close(np64(out), o_ref, tol, "paged out"),
           "lse": assert_close(np64(lse), l_ref, tol, "paged lse"),
           "block_logit": assert_close(np64(bl), b_ref, 2e-4, "paged block_logit")}
    own = ref.own_blocks(p.B, p.Sq, p.Skv, p.block_size, p.kv_lens)
    idx_np = idx.cpu().numpy()
    assert np.array_equal(idx_np, ref.topk_blocks(bl.cpu().numpy(), own, p.top_k))
    res["exact_rows"] = check_topk_margin(idx_np, b_ref, own, p.top_k)
    og_ref, lg_ref = ref.sparse_gather(p.q, p.kv, p.sink, p.Dv, p.scale, idx_np, **kw)
    res["gather_out"] = assert_close(np64(og), og_ref, tol, "paged gather out")
    res["gather_lse"] = assert_close(np64(lg), lg_ref, tol, "paged gather lse")
    os_ref, ls_ref = ref.swa(p.q, p.kv, p.sink, p.Dv, p.scale, p.window, **kw)
    res["swa_out"] = assert_close(np64(osw), os_ref, tol, "paged swa out")
    res["swa_lse"] = assert_close(np64(lsw), ls_ref, tol, "paged swa lse")
    say(f"[gpu] paged {case}: {res}")
