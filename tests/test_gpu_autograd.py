"""GPU checks of the autograd functions (block_sparse_mqa_amd.autograd): a
backward pass through them must deliver exactly the library's gradients
(rounded to the inputs' dtype), the block scores and selection must not
require gradients, lse carries its gradient into the kernels, and gradients
of two calls sharing q and kv must add."""
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import autograd as hsa
from block_sparse_mqa_amd import inputs

from gpu_common import np64, say
from test_gpu_parity import MLA

pytestmark = pytest.mark.gpu


def _leaves(p):
    q = p.q.cuda().requires_grad_(True)
    kv = p.kv.cuda().requires_grad_(True)
    sink = p.sink.cuda().requires_grad_(True)
    return q, kv, sink


def test_autograd_matches_library_gradients():
    p = inputs.make(1, 200, 200, MLA["H"], MLA["Dk"], MLA["Dv"], seed=81, top_k=3, window=70,
                    name="autograd")
    prob = hs.Problem(1, 200, 200, p.H, p.Dk, p.Dv, scale=p.scale)
    dout = inputs.make_dout(p, seed=82).cuda()
    q, kv, sink = _leaves(p)

    out, lse, bl, idx = hsa.block_score_attention(q, kv, sink, prob, p.top_k)
    assert out.requires_grad and lse.requires_grad and not bl.requires_grad
    assert not idx.requires_grad and idx.dtype == torch.int32
    (gq, gkv, gs) = torch.autograd.grad(out, (q, kv, sink), dout)
    with torch.no_grad():
        dq, dkv, dsink = hs.block_score_bwd(prob, q, kv, sink, out, lse, dout)
    torch.cuda.synchronize()
    assert gq.dtype == q.dtype and gkv.dtype == kv.dtype and gs.dtype == torch.float32
    assert torch.equal(gq, dq.to(q.dtype)) and torch.equal(gkv, dkv.to(kv.dtype))
    assert torch.equal(gs, dsink)

    og, lg = hsa.sparse_gather_attention(q, kv, sink, idx, prob, p.top_k)
    (gq, gkv, gs) = torch.autograd.grad(og, (q, kv, sink), dout)
    with torch.no_grad():
        dq, dkv, dsink = hs.sparse_gather_bwd(prob, q, kv, sink, idx, p.top_k, og, lg, dout)
    assert torch.equal(gq, dq.to(q.dtype)) and torch.equal(gkv, dkv.to(kv.dtype))
    assert torch.equal(gs, dsink)

    ow, lw = hsa.sliding_window_attention(q, kv, sink, prob, p.window)
    (gq, gkv, gs) = torch.autograd.grad(ow, (q, kv, sink), dout)
    with torch.no_grad():
        dq, dkv, dsink = hs.swa_bwd(prob, q, kv, sink, p.window, ow, lw, dout)
    assert torch.equal(gq, dq.to(q.dtype)) and torch.equal(gkv, dkv.to(kv.dtype))
    assert torch.equal(gs, dsink)
    say("[gpu] autograd functions deliver the library's gradients")


def test_autograd_gradients_accumulate_over_branches():
    """A window branch and a gather branch reading the same q and kv (as the
    two branches of a layer would): backward through their sum gives the sum
    of the two calls' gradients, and a sink without requires_grad gets none."""
    p = inputs.make(1, 150, 150, MLA["H"], MLA["Dk"], MLA["Dv"], seed=83, top_k=2, window=40,
                    name="autograd_sum")
    prob = hs.Problem(1, 150, 150, p.H, p.Dk, p.Dv, scale=p.scale)
    dout = inputs.make_dout(p, seed=84).cuda()
    q = p.q.cuda().requires_grad_(True)
    kv = p.kv.cuda().requires_grad_(True)
    sink = p.sink.cuda()                                   # no gradient asked
    _, _, _, idx = hsa.block_score_attention(q, kv, sink, prob, p.top_k)
    og, lg = hsa.sparse_gather_attention(q, kv, sink, idx, prob, p.top_k)
    ow, lw = hsa.sliding_window_attention(q, kv, sink, prob, p.window)
    ((og.float() + ow.float()) * dout.float()).sum().backward()
    with torch.no_grad():
        a = hs.sparse_gather_bwd(prob, q, kv, sink, idx, p.top_k, og, lg, dout)
        b = hs.swa_bwd(prob, q, kv, sink, p.window, ow, lw, dout)
    torch.cuda.synchronize()
    want_q = a[0].to(q.dtype).float() + b[0].to(q.dtype).float()
    want_kv = a[1].to(kv.dtype).float() + b[1].to(kv.dtype).float()
    assert torch.allclose(q.grad.float(), want_q, rtol=1e-2, atol=1e-3)
    assert torch.allclose(kv.grad.float(), want_kv, rtol=1e-2, atol=1e-3)
    say("[gpu] autograd gradients accumulate over branches")


def test_sliding_window_layer_gradients():
    """The layer function (both branches from one forward call) gives the
    gradients of the two separate functions summed, in fp32 before rounding
    to the inputs' dtype, and a branch left out of the loss costs no gradient
    call of its own."""
    p = inputs.make(1, 180, 180, MLA["H"], MLA["Dk"], MLA["Dv"], seed=85, top_k=3, window=50,
                    name="layer_fn")
    prob = hs.Problem(1, 180, 180, p.H, p.Dk, p.Dv, scale=p.scale)
    q, kv, sink = _leaves(p)
    with torch.no_grad():
        _, _, _, idx = hsa.block_score_attention(q, kv, sink, prob, p.top_k)
    d1 = inputs.make_dout(p, seed=86).cuda()
    d2 = inputs.make_dout(p, seed=87).cuda()
    ow, lw, og, lg = hsa.sliding_window_layer(q, kv, sink, idx, prob, p.window, p.top_k)
    gq, gkv, gs = torch.autograd.grad((ow, og), (q, kv, sink), (d1, d2))
    with torch.no_grad():
        a = hs.swa_bwd(prob, q, kv, sink, p.window, ow, lw, d1)
        b = hs.sparse_gather_bwd(prob, q, kv, sink, idx, p.top_k, og, lg, d2)
    torch.cuda.synchronize()
    assert torch.equal(gq, (a[0] + b[0]).to(q.dtype))
    assert torch.equal(gkv, (a[1] + b[1]).to(kv.dtype))
    assert torch.equal(gs, a[2] + b[2])
    # only the window branch in the loss
    ow, lw, og, lg = hsa.sliding_window_layer(q, kv, sink, idx, prob, p.window, p.top_k)
    gq1, = torch.autograd.grad(ow, (q,), d1)
    assert torch.equal(gq1, a[0].to(q.dtype))
    say("[gpu] sliding-window layer function: gradients of both branches")


def test_loss_using_lse_gets_its_gradient():
    """A loss that uses lse (a log-sum-exp weighting of branches would):
    autograd passes dlse to the kernels, giving exactly the library's
    gradients with dlse, and those match the float64 oracle's gradient of
    sum(dout * out) + sum(w * lse) for all three operations."""
    from oracle import hysparse_ref as ref
    from test_gpu_bwd import _grad_close
    p = inputs.make(1, 130, 130, MLA["H"], MLA["Dk"], MLA["Dv"], seed=83, top_k=2, window=70,
                    name="autograd_lse")
    prob = hs.Problem(1, 130, 130, p.H, p.Dk, p.Dv, scale=p.scale)
    dout = inputs.make_dout(p, seed=84).cuda()
    w = torch.randn((1, 130, p.H), generator=torch.Generator().manual_seed(85)).cuda()
    q, kv, sink = _leaves(p)
    out, lse, bl, idx = hsa.block_score_attention(q, kv, sink, prob, p.top_k)
    ow, lw = hsa.sliding_window_attention(q, kv, sink, prob, p.window)
    og, lg = hsa.sparse_gather_attention(q, kv, sink, idx, prob, p.top_k)
    kw = dict(block_size=64)
    cases = (("score", out, lse, lambda d: ref.block_score_bwd(p.q, p.kv, p.sink, p.Dv, p.scale,
                                                               d, dlse=w.cpu(), **kw)),
             ("swa", ow, lw, lambda d: ref.swa_bwd(p.q, p.kv, p.sink, p.Dv, p.scale, p.window, d,
                                                   dlse=w.cpu(), **kw)),
             ("gather", og, lg, lambda d: ref.sparse_gather_bwd(p.q, p.kv, p.sink, p.Dv, p.scale,
                                                                idx.cpu().numpy(), d,
                                                                dlse=w.cpu(), **kw)))
    errs = {}
    for name, o, l, oracle_fn in cases:
        loss = (o.float() * dout.float()).sum() + (l * w).sum()
        gq, gkv, gs = torch.autograd.grad(loss, (q, kv, sink))
        with torch.no_grad():
            if name == "score":
                lib = hs.block_score_bwd(prob, q, kv, sink, o, l, dout, dlse=w)
            elif name == "swa":
                lib = hs.swa_bwd(prob, q, kv, sink, p.window, o, l, dout, dlse=w)
            else:
                lib = hs.sparse_gather_bwd(prob, q, kv, sink, idx, p.top_k, o, l, dout, dlse=w)
        torch.cuda.synchronize()
        assert torch.equal(gq, lib[0].to(q.dtype)) and torch.equal(gkv, lib[1].to(kv.dtype))
        assert torch.equal(gs, lib[2])
        want = oracle_fn(dout.cpu())
        errs[name] = [_grad_close(np64(a), b, "bf16", f"{name} {n}")
                      for a, b, n in zip(lib, want, ("dq", "dkv", "dsink"))]
    say(f"[gpu] gradients with dlse vs oracle: {errs}")


def test_stored_score_gradients_through_autograd():
    """store_ds=True routes each function's backward through the stored
    score-gradient workspace: the gradients equal the library's stored-form
    calls exactly, and dkv and dsink equal the recomputing form's bit for
    bit while dq stays within the rounding of the stored bf16 dS."""
    p = inputs.make(1, 260, 260, MLA["H"], MLA["Dk"], MLA["Dv"], seed=88, top_k=3, window=90,
                    name="autograd_store")
    prob = hs.Problem(1, 260, 260, p.H, p.Dk, p.Dv, scale=p.scale)
    dout = inputs.make_dout(p, seed=89).cuda()
    q, kv, sink = _leaves(p)
    with torch.no_grad():
        _, _, _, idx = hsa.block_score_attention(q, kv, sink, prob, p.top_k)

    def run(store):
        out, lse, _, _ = hsa.block_score_attention(q, kv, sink, prob, p.top_k, store_ds=store)
        og, lg = hsa.sparse_gather_attention(q, kv, sink, idx, prob, p.top_k, store_ds=store)
        ow, lw = hsa.sliding_window_attention(q, kv, sink, prob, p.window, store_ds=store)
        lo_w, _, lo_g, _ = hsa.sliding_window_layer(q, kv, sink, idx, prob, p.window, p.top_k,
                                                    store_ds=store)
        res = [torch.autograd.grad(o, (q, kv, sink), dout) for o in (out, og, ow)]
        res.append(torch.autograd.grad((lo_w, lo_g), (q, kv, sink), (dout, dout)))
        lib = (lambda: hs.block_score_bwd(prob, q, kv, sink, out, lse, dout, store_ds=store),
               lambda: hs.sparse_gather_bwd(prob, q, kv, sink, idx, p.top_k, og, lg, dout,
                                            store_ds=store),
               lambda: hs.swa_bwd(prob, q, kv, sink, p.window, ow, lw, dout, store_ds=store))
        with torch.no_grad():
            want = [f() for f in lib]
        torch.cuda.synchronize()
        for (gq, gkv, gs), (dq, dkv, dsink) in zip(res, want):
            assert torch.equal(gq, dq.to(q.dtype)) and torch.equal(gkv, dkv.to(kv.dtype))
            assert torch.equal(gs, dsink)
        return res

    stored, recomputed = run(True), run(False)
    rel = []
    for (aq, akv, asink), (bq, bkv, bsink) in zip(stored, recomputed):
        assert torch.equal(akv, bkv) and torch.equal(asink, bsink)
        r = float((aq.float() - bq.float()).abs().max() / bq.float().abs().max())
        assert r < 1e-2, r
        rel.append(r)
    say(f"[gpu] stored dS through autograd: dq max rel diff {[f'{r:.1e}' for r in rel]}")
