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


def _decode_reference(p, lens, NB):
    """Oracle results for lengths `lens`; block_logit padded with -inf to the
    NB columns the capacity gives (the ABI writes -inf past each entry's blocks)."""
    kw = dict(block_size=p.block_size, kv_lens=lens)
    o, l, b = ref.block_score(p.q, p.kv, p.sink, p.Dv, p.scale, **kw)
    pad = np.full(b.shape[:-1] + (NB - b.shape[-1],), -np.inf)
    b = np.concatenate([b, pad], axis=-1)
    os_, ls = ref.swa(p.q, p.kv, p.sink, p.Dv, p.scale, p.window, **kw)
    return o, l, b, os_, ls


@pytest.mark.parametrize("layout", ["paged", "in_place"])
def test_device_lengths_and_graph_replay(layout):
    """Lengths in device memory, read at run time: one captured graph of the
    decode calls replayed with different lengths matches the oracle each time,
    for a paged pool and for an in-place cache [B, capacity, Dk]."""
    say(f"[gpu] {layout} KV with device lengths, captured graph")
    B, cap = 8, 2048
    rng = np.random.default_rng(44)
    full = [cap] * B
    p = inputs.make(B, 1, cap, MLA["H"], MLA["Dk"], MLA["Dv"], seed=44, kv_lens=full, top_k=4,
                    window=200, name="paged_devlen")
    q, sink = p.q.cuda(), p.sink.cuda()
    lens_dev = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    if layout == "paged":
        pool, pt = _paged(p, seed=45)
        pool, pt = pool.cuda(), pt.cuda()
        prob = hs.Problem(B, 1, cap, p.H, p.Dk, p.Dv, page_table=pt, kv_lens_device=lens_dev)
    else:
        pool = p.kv.cuda()
        prob = hs.Problem(B, 1, cap, p.H, p.Dk, p.Dv, kv_lens_device=lens_dev)
    NB = hs.hs_num_blocks(prob)
    assert NB == cap // 64
    out = torch.empty((B, 1, p.H, p.Dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 1, p.H), dtype=torch.float32, device="cuda")
    bl = torch.empty((B, 1, NB), dtype=torch.float32, device="cuda")
    osw, lsw = torch.empty_like(out), torch.empty_like(lse)
    ws1 = hs._workspace(prob, hs.HS_OP_BLOCK_SCORE)
    ws4 = hs._workspace(prob, hs.HS_OP_SWA, window=p.window)

    def calls():
        hs.hs_block_score_fwd(prob, q, pool, sink, out, lse, bl, ws1)
        hs.hs_swa_fwd(prob, q, pool, sink, p.window, osw, lsw, ws4)

    tol = tol_for(p)
    # eager first, at full length
    calls()
    torch.cuda.synchronize()
    o, l, b, os_, ls = _decode_reference(p, full, NB)
    assert_close(np64(out), o, tol, "eager out")
    assert_close(np64(bl), b, 2e-4, "eager block_logit")
    # capture once, replay with other lengths
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        calls()                      # warm the side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        lens = [int(x) for x in rng.integers(1, cap + 1, size=B)]
        lens_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o, l, b, os_, ls = _decode_reference(p, lens, NB)
        e = {"out": assert_close(np64(out), o, tol, f"replay {rep} out"),
             "lse": assert_close(np64(lse), l, tol, f"replay {rep} lse"),
             "block_logit": assert_close(np64(bl), b, 2e-4, f"replay {rep} block_logit"),
             "swa_out": assert_close(np64(osw), os_, tol, f"replay {rep} swa out"),
             "swa_lse": assert_close(np64(lsw), ls, tol, f"replay {rep} swa lse")}
        say(f"[gpu] graph replay {rep} lengths {min(lens)}..{max(lens)}: {e}")


def test_paged_window_and_sparse_call():
    """hs_swa_sparse_fwd on a paged pool runs the two operations one after the
    other; both outputs must equal the separate paged calls bit for bit and
    the oracle on the contiguous cache."""
    lens = [700, 333, 1100]
    p = inputs.make(3, 200, 1100, MLA["H"], MLA["Dk"], MLA["Dv"], seed=44, kv_lens=lens,
                    top_k=4, window=150, name="paged_swa_sparse")
    say("[gpu] paged KV window-and-sparse call")
    pool, pt = _paged(p, seed=45)
    pool, pt = pool.cuda(), pt.cuda()
    q, sink = p.q.cuda(), p.sink.cuda()
    prob = hs.Problem(p.B, p.Sq, p.Skv, p.H, p.Dk, p.Dv, kv_lens=p.kv_lens, page_table=pt)
    _, _, bl = hs.block_score(prob, q, pool, sink)
    idx = hs.topk_blocks(prob, bl, p.top_k)
    ow, lw, og, lg = hs.swa_sparse(prob, q, pool, sink, p.window, idx, p.top_k)
    sw = hs.swa(prob, q, pool, sink, p.window)
    sg = hs.sparse_gather(prob, q, pool, sink, idx, p.top_k)
    torch.cuda.synchronize()
    for g, w, n in zip((ow, lw, og, lg), (*sw, *sg), ("out_swa", "lse_swa", "out_sparse",
                                                      "lse_sparse")):
        assert torch.equal(g, w), n
    kw = dict(block_size=p.block_size, kv_lens=p.kv_lens)
    idx_np = idx.cpu().numpy()
    os_ref, ls_ref = ref.swa(p.q, p.kv, p.sink, p.Dv, p.scale, p.window, **kw)
    og_ref, lg_ref = ref.sparse_gather(p.q, p.kv, p.sink, p.Dv, p.scale, idx_np, **kw)
    tol = tol_for(p)
    e = [assert_close(np64(ow), os_ref, tol, "swa out"), assert_close(np64(lw), ls_ref, tol, "swa lse"),
         assert_close(np64(og), og_ref, tol, "sparse out"),
         assert_close(np64(lg), lg_ref, tol, "sparse lse")]
    say(f"[gpu] paged window-and-sparse: identical to the separate calls, oracle {max(e):.2e}")
