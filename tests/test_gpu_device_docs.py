"""GPU parity of device-resident document bounds: the packing of a packed
prefill is read from device memory when the kernels run, so one captured
graph serves changing packings. Eager calls must equal the same calls with
host bounds bit for bit (block_logit columns past the packing's blocks are
-inf), and each replay of a graph must match the oracle for the packing it
was given."""
import numpy as np
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs
from oracle import hysparse_ref as ref

from gpu_common import assert_close, check_topk_margin, np64, say, tol_for
from test_gpu_parity import MLA

pytestmark = pytest.mark.gpu

S, CAP, K, W = 300, 8, 3, 40


def _bounds(lens, cap=CAP):
    """Cumulative starts [cap + 1] of a packing, padded with empty documents
    at the end."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return np.concatenate([cu, np.full(cap + 1 - len(cu), cu[-1], np.int32)])


def _docs(cu):
    """Host doc_start / doc_end of the non-empty documents of a bound table."""
    ds = [int(a) for a, b in zip(cu[:-1], cu[1:]) if b > a]
    de = [int(b) for a, b in zip(cu[:-1], cu[1:]) if b > a]
    return ds, de


def _problem(seed):
    return inputs.make(1, S, S, MLA["H"], MLA["Dk"], MLA["Dv"], seed=seed, top_k=K, window=W,
                       name="device_docs")


def test_device_bounds_equal_host_bounds():
    """Eager: the four calls and the one-pass window-and-sparse call with the
    packing on the device equal the calls with the same packing on the host,
    with empty documents between and after the real ones."""
    p = _problem(91)
    q, kv, sink = p.q.cuda(), p.kv.cuda(), p.sink.cuda()
    # empty documents in the middle and at the end
    cu = np.array([0, 70, 71, 71, 134, 234, 234, 300, 300], np.int32)
    ds, de = _docs(cu)
    say(f"[gpu] device document bounds {cu.tolist()}")
    dev = hs.Problem(1, S, S, p.H, p.Dk, p.Dv, scale=p.scale,
                     doc_bounds_device=torch.from_numpy(cu).cuda())
    host = hs.Problem(1, S, S, p.H, p.Dk, p.Dv, scale=p.scale, doc_start=ds, doc_end=de)
    nb_dev, nb_host = hs.hs_num_blocks(dev), hs.hs_num_blocks(host)
    assert nb_dev == (S + 63) // 64 + CAP - 1 and nb_host < nb_dev
    o1, l1, b1 = hs.block_score(dev, q, kv, sink)
    o2, l2, b2 = hs.block_score(host, q, kv, sink)
    i1 = hs.topk_blocks(dev, b1, K)
    i2 = hs.topk_blocks(host, b2, K)
    f1 = hs.block_score_topk(dev, q, kv, sink, K)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(b1[..., :nb_host], b2)
    assert bool(torch.all(torch.isneginf(b1[..., nb_host:])))
    assert torch.equal(i1, i2)
    assert all(torch.equal(x, y) for x, y in zip(f1, (o1, l1, b1, i1)))
    g1 = hs.sparse_gather(dev, q, kv, sink, i1, K)
    g2 = hs.sparse_gather(host, q, kv, sink, i2, K)
    w1 = hs.swa(dev, q, kv, sink, W)
    w2 = hs.swa(host, q, kv, sink, W)
    m1 = hs.swa_sparse(dev, q, kv, sink, W, i1, K)
    m2 = hs.swa_sparse(host, q, kv, sink, W, i2, K)
    torch.cuda.synchronize()
    for n, x, y in (("gather", g1, g2), ("swa", w1, w2), ("swa_sparse", m1, m2)):
        assert all(torch.equal(a, b) for a, b in zip(x, y)), n
    say("[gpu] device document bounds equal host bounds")


def test_device_bounds_graph_replay():
    """One captured graph of block score, top-k, gather and window, replayed
    with three packings (one document; many short ones; a one-row document),
    matches the oracle each time; eager work runs between the replays."""
    p = _problem(92)
    q, kv, sink = p.q.cuda(), p.kv.cuda(), p.sink.cuda()
    cu_dev = torch.from_numpy(_bounds([S])).cuda()
    prob = hs.Problem(1, S, S, p.H, p.Dk, p.Dv, scale=p.scale, doc_bounds_device=cu_dev)
    NB = hs.hs_num_blocks(prob)
    out = torch.empty((1, S, p.H, p.Dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, S, p.H), dtype=torch.float32, device="cuda")
    bl = torch.empty((1, S, NB), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, S, K), dtype=torch.int32, device="cuda")
    og, lg = torch.empty_like(out), torch.empty_like(lse)
    ow, lw = torch.empty_like(out), torch.empty_like(lse)

    def calls():
        hs.hs_block_score_fwd(prob, q, kv, sink, out, lse, bl, None)
        hs.hs_topk_blocks(prob, bl, K, idx)
        hs.hs_sparse_gather_fwd(prob, q, kv, sink, idx, K, og, lg, None)
        hs.hs_swa_fwd(prob, q, kv, sink, W, ow, lw, None)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                      # warm the side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    tol = tol_for(p)
    for rep, lens in enumerate(([S], [40, 33, 64, 1, 65, 50, 47], [299, 1])):
        cu = _bounds(lens)
        cu_dev.copy_(torch.from_numpy(cu))
        out.zero_()
        idx.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ds, de = _docs(cu)
        kw = dict(block_size=64, doc_start=ds, doc_end=de)
        o, l, b = ref.block_score(p.q, p.kv, p.sink, p.Dv, p.scale, **kw)
        nbp = b.shape[-1]
        got_bl = np64(bl)
        assert np.all(np.isneginf(got_bl[..., nbp:])), f"replay {rep}: columns past the packing"
        own = ref.own_blocks(1, S, S, 64, None, ds, de)
        exact = check_topk_margin(idx.cpu().numpy(), b, own, K)
        # the gather is checked on the GPU's own selection
        go, gl = ref.sparse_gather(p.q, p.kv, p.sink, p.Dv, p.scale, idx.cpu().numpy(), **kw)
        wo, wl = ref.swa(p.q, p.kv, p.sink, p.Dv, p.scale, W, **kw)
        e = {"out": assert_close(np64(out), o, tol, f"replay {rep} out"),
             "lse": assert_close(np64(lse), l, tol, f"replay {rep} lse"),
             "block_logit": assert_close(got_bl[..., :nbp], b, 2e-4, f"replay {rep} block_logit"),
             "gather": assert_close(np64(og), go, tol, f"replay {rep} gather out"),
             "gather_lse": assert_close(np64(lg), gl, tol, f"replay {rep} gather lse"),
             "swa": assert_close(np64(ow), wo, tol, f"replay {rep} swa out"),
             "swa_lse": assert_close(np64(lw), wl, tol, f"replay {rep} swa lse")}
        say(f"[gpu] graph replay {rep} with {len(ds)} documents: exact top-k rows {exact:.2f}, {e}")
        # eager work between replays
        hs.swa(prob, q, kv, sink, W)
        torch.cuda.synchronize()
