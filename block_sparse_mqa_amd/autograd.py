"""PyTorch autograd functions over the C ABI.

Each function runs its forward and its gradient in the library's kernels
(hs_block_score_topk_fwd / hs_block_score_bwd, hs_sparse_gather_fwd /
hs_sparse_gather_bwd, hs_swa_fwd / hs_swa_bwd). This mirrors the autograd
layers of the page "HySparse MQA sparse attention (FA4 block scoring + SWA
MQA + block-sparse DSA gather)", section "Core": block scoring trained
through its autograd layer, and the learnable sink's analytic gradient. As in
the review of PaddleFleet PR 1453 (block-score PyLayer comments), gradients
flow to q, the latent kv and the sink only; the block scores and the block
selection are outputs without gradient. lse is differentiable: a loss that
uses it (for instance branches weighted by their log-sum-exp) passes its
gradient to the kernels, which add it exactly (dlse in include/hs.h).

The library computes gradients in fp32. Autograd needs each gradient in its
input's dtype, so bf16 inputs receive the fp32 gradients rounded to bf16.
Nothing else runs outside the kernels.

store_ds (default False) picks the larger gradient workspaces, in which the
key-block pass stores the bf16 score gradients and dq reads them instead of
recomputing the scores (faster, 8 KB per (row, key block) pair; the same
gradients up to the rounding of dS).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (Problem, block_score_topk, hs_block_score_bwd, hs_sparse_gather_bwd, hs_swa_bwd,
               score_bwd_workspace, sparse_gather, sparse_gather_bwd_workspace, swa,
               swa_bwd_workspace, swa_sparse)


def _grads(prob, q, sink, need_sink):
    dq = torch.empty((prob.B, prob.Sq, prob.H, prob.Dk), dtype=torch.float32, device=q.device)
    dkv = torch.empty((prob.B, prob.Skv, prob.Dk), dtype=torch.float32, device=q.device)
    dsink = (torch.empty((prob.H,), dtype=torch.float32, device=q.device)
             if (sink is not None and need_sink) else None)
    return dq, dkv, dsink


def _finish(ctx, q, kv, sink, dq, dkv, dsink):
    gq = dq.to(q.dtype) if ctx.needs_input_grad[0] else None
    gkv = dkv.to(kv.dtype) if ctx.needs_input_grad[1] else None
    gs = dsink if (sink is not None and ctx.needs_input_grad[2]) else None
    return gq, gkv, gs


class BlockScoreTopk(torch.autograd.Function):
    """(out, lse, block_logit, block_idx) of causal attention with block
    scores and the per-token top-k; gradients reach q, kv and the sink."""

    @staticmethod
    def forward(ctx, q, kv, sink, prob: Problem, top_k: int, store_ds: bool = False):
        out, lse, bl, idx = block_score_topk(prob, q, kv, sink, top_k)
        ctx.save_for_backward(q, kv, sink, out, lse)
        ctx.prob, ctx.store_ds = prob, store_ds
        ctx.mark_non_differentiable(bl, idx)
        return out, lse, bl, idx

    @staticmethod
    def backward(ctx, dout, dlse, _dbl, _didx):
        q, kv, sink, out, lse = ctx.saved_tensors
        prob = ctx.prob
        dq, dkv, dsink = _grads(prob, q, sink, ctx.needs_input_grad[2])
        hs_block_score_bwd(prob, q, kv, sink, out, lse, dout.contiguous(), dq, dkv, dsink,
                           score_bwd_workspace(prob, ctx.store_ds), dlse=dlse.contiguous())
        return (*_finish(ctx, q, kv, sink, dq, dkv, dsink), None, None, None)


class SparseGather(torch.autograd.Function):
    """(out, lse) of the block-sparse gather for a given selection; the
    selection itself takes no gradient."""

    @staticmethod
    def forward(ctx, q, kv, sink, block_idx, prob: Problem, top_k: int, store_ds: bool = False):
        out, lse = sparse_gather(prob, q, kv, sink, block_idx, top_k)
        ctx.save_for_backward(q, kv, sink, block_idx, out, lse)
        ctx.prob, ctx.top_k, ctx.store_ds = prob, top_k, store_ds
        return out, lse

    @staticmethod
    def backward(ctx, dout, dlse):
        q, kv, sink, block_idx, out, lse = ctx.saved_tensors
        prob = ctx.prob
        dq, dkv, dsink = _grads(prob, q, sink, ctx.needs_input_grad[2])
        hs_sparse_gather_bwd(prob, q, kv, sink, block_idx, ctx.top_k, out, lse,
                             dout.contiguous(), dq, dkv, dsink,
                             sparse_gather_bwd_workspace(prob, ctx.top_k, ctx.store_ds),
                             dlse=dlse.contiguous())
        return (*_finish(ctx, q, kv, sink, dq, dkv, dsink), None, None, None, None)


class SlidingWindow(torch.autograd.Function):
    """(out, lse) of sliding-window MQA attention."""

    @staticmethod
    def forward(ctx, q, kv, sink, prob: Problem, window: int, store_ds: bool = False):
        out, lse = swa(prob, q, kv, sink, window)
        ctx.save_for_backward(q, kv, sink, out, lse)
        ctx.prob, ctx.window, ctx.store_ds = prob, window, store_ds
        return out, lse

    @staticmethod
    def backward(ctx, dout, dlse):
        q, kv, sink, out, lse = ctx.saved_tensors
        prob = ctx.prob
        dq, dkv, dsink = _grads(prob, q, sink, ctx.needs_input_grad[2])
        hs_swa_bwd(prob, q, kv, sink, ctx.window, out, lse, dout.contiguous(), dq, dkv, dsink,
                   swa_bwd_workspace(prob, ctx.window, ctx.store_ds), dlse=dlse.contiguous())
        return (*_finish(ctx, q, kv, sink, dq, dkv, dsink), None, None, None)


class SlidingWindowLayer(torch.autograd.Function):
    """(out_swa, lse_swa, out_sparse, lse_sparse): both branches of a
    sliding-window layer over a full layer's KV and block selection
    (hs_swa_sparse_fwd). The gradient is the sum of the two branches'
    (hs_swa_bwd and hs_sparse_gather_bwd), each with the gradients its out and
    lse receive; a branch whose outputs receive none is skipped."""

    @staticmethod
    def forward(ctx, q, kv, sink, block_idx, prob: Problem, window: int, top_k: int,
                store_ds: bool = False):
        ow, lw, og, lg = swa_sparse(prob, q, kv, sink, window, block_idx, top_k)
        ctx.save_for_backward(q, kv, sink, block_idx, ow, lw, og, lg)
        ctx.prob, ctx.window, ctx.top_k, ctx.store_ds = prob, window, top_k, store_ds
        ctx.set_materialize_grads(False)
        return ow, lw, og, lg

    @staticmethod
    def backward(ctx, dout_swa, dlw, dout_sparse, dlg):
        q, kv, sink, block_idx, ow, lw, og, lg = ctx.saved_tensors
        prob = ctx.prob
        total = None
        for dout, dl, run in (
                (dout_swa, dlw, lambda g, d, l_: hs_swa_bwd(
                    prob, q, kv, sink, ctx.window, ow, lw, d, *g,
                    swa_bwd_workspace(prob, ctx.window, ctx.store_ds), dlse=l_)),
                (dout_sparse, dlg, lambda g, d, l_: hs_sparse_gather_bwd(
                    prob, q, kv, sink, block_idx, ctx.top_k, og, lg, d, *g,
                    sparse_gather_bwd_workspace(prob, ctx.top_k, ctx.store_ds), dlse=l_))):
            if dout is None and dl is None:
                continue
            g = _grads(prob, q, sink, ctx.needs_input_grad[2])
            d = torch.zeros_like(ow) if dout is None else dout.contiguous()
            run(g, d, None if dl is None else dl.contiguous())
            total = g if total is None else tuple(
                None if a is None else a + b for a, b in zip(total, g))
        if total is None:
            return None, None, None, None, None, None, None, None
        return (*_finish(ctx, q, kv, sink, *total), None, None, None, None, None)


def sliding_window_layer(q, kv, sink: Optional[torch.Tensor], block_idx, prob: Problem,
                         window: int, top_k: int, store_ds: bool = False):
    """Both branches of a sliding-window layer: returns (out_swa, lse_swa,
    out_sparse, lse_sparse); differentiable in q, kv and sink."""
    return SlidingWindowLayer.apply(q, kv, sink, block_idx, prob, window, top_k, store_ds)


def block_score_attention(q, kv, sink: Optional[torch.Tensor], prob: Problem, top_k: int,
                          store_ds: bool = False):
    """Causal attention with sink, its block scores and the top-k selection:
    returns (out, lse, block_logit, block_idx); differentiable in q, kv, sink."""
    return BlockScoreTopk.apply(q, kv, sink, prob, top_k, store_ds)


def sparse_gather_attention(q, kv, sink: Optional[torch.Tensor], block_idx, prob: Problem,
                            top_k: int, store_ds: bool = False):
    """Block-sparse gather attention: returns (out, lse)."""
    return SparseGather.apply(q, kv, sink, block_idx, prob, top_k, store_ds)


def sliding_window_attention(q, kv, sink: Optional[torch.Tensor], prob: Problem, window: int,
                             store_ds: bool = False):
    """Sliding-window MQA attention: returns (out, lse)."""
    return SlidingWindow.apply(q, kv, sink, prob, window, store_ds)
