"""Seeded synthetic inputs for the HySparse MQA path (forward and gradients).

This module only draws random tensors and describes problem shapes. It holds
none of the method's arithmetic: no scores, no softmax, no block scoring, no
selection. Both the CPU oracle (through the tests and the benchmark) and the
HIP path receive exactly the tensors built here.

Workloads (the shapes follow the absorbed-MLA MQA layout that the FlashMLA
sparse-kernel constraints fix on the page "HySparse MQA sparse attention (FA4
block scoring + SWA MQA + block-sparse DSA gather)", section "FlashMLA sparse
kernel constraints": one shared KV head, d_qk = 576 = 512 + 64, d_v = 512 taken
as the leading region of K, h_q = 64):

  1  tiny fp32:   B=1, S=512,   H=8,  Dk=96,  Dv=64,  top_k=4,  window=128
  2  bf16:        B=1, S=4096,  H=64, Dk=576, Dv=512, top_k=16, window=512
  3  bf16 long:   B=1, S=32768, same heads/dims,      top_k=32, window=1024,
                  every 4th key block (j % 4 == 0) scaled by 3
  4  bf16 packed: B=1, S=16384 split into 8 documents, top_k=16, window=512
  5  bf16 decode: B=32, one query token each, cached KV of length
                  U{16384..65536}, top_k=32, window=1024

Recipe (all configs): config c seeds ``torch.Generator().manual_seed(c)``.
Draw order: document or cache lengths (configs 4 and 5), then q, then kv, then
the sink. q and kv are drawn in fp32 in chunks of at most 1024 rows, then cast
to the storage dtype with round-to-nearest-even. q ~ N(0, 1). kv ~ N(0, 1) for
config 1 and N(0, 1) * 4 / sqrt(576) for the others. sink ~ N(0, 1), stored
fp32. KV rows past a sequence's valid length are filled with NaN so that any
read of them shows up in the outputs.

Upstream gradients for the gradient calls (``make_dout``): dout ~ N(0, 1) of
the output's shape [B, Sq, H, Dv], drawn from its own generator seeded with
the given seed, in fp32 chunks of 1024 rows, cast to the storage dtype.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

CHUNK_ROWS = 1024


@dataclass
class Problem:
    """One seeded workload: shapes, scalars and the host-resident tensors."""

    name: str
    dtype: str                      # "f32" or "bf16": storage type of q, kv, out
    B: int
    Sq: int
    Skv: int
    H: int
    Dk: int
    Dv: int
    block_size: int
    top_k: int
    window: int
    scale: float
    kv_lens: Optional[List[int]] = None     # per-batch valid KV length (decode)
    doc_start: Optional[List[int]] = None   # packed documents, B == 1 only
    doc_end: Optional[List[int]] = None
    q: torch.Tensor = field(default=None, repr=False)     # [B, Sq, H, Dk]
    kv: torch.Tensor = field(default=None, repr=False)    # [B, Skv, Dk]
    sink: torch.Tensor = field(default=None, repr=False)  # [H] float32

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x if dtype == "f32" else x.to(torch.bfloat16)


def _draw_rows(g, rows: int, inner: tuple, mult: float, dtype: str,
               row_scale=None) -> torch.Tensor:
    """Draw [rows, *inner] N(0,1)*mult in fp32 chunks of CHUNK_ROWS rows.

    ``row_scale`` optionally maps a row index range to a per-row fp32 factor
    (used for the scaled key blocks of the long-context workload)."""
    out = torch.empty((rows,) + inner, dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
    for r0 in range(0, rows, CHUNK_ROWS):
        r1 = min(rows, r0 + CHUNK_ROWS)
        x = torch.randn((r1 - r0,) + inner, generator=g, dtype=torch.float32)
        if mult != 1.0:
            x.mul_(mult)
        if row_scale is not None:
            f = row_scale(r0, r1)
            x.mul_(f.view((r1 - r0,) + (1,) * len(inner)))
        out[r0:r1] = _cast(x, dtype)
    return out


def doc_lengths_packed(g, total: int = 16384, n_docs: int = 8, lo: int = 512,
                       hi: int = 4096, min_last: int = 64) -> List[int]:
    """Document lengths for the packed workload.

    Rejection-sample n_docs integers uniform in [lo, hi] until the first
    n_docs-1 leave at least ``min_last`` rows and all n_docs reach ``total``;
    the last one is then trimmed so that the lengths sum to ``total``."""
    while True:
        L = torch.randint(lo, hi + 1, (n_docs,), generator=g).tolist()
        head = sum(L[:-1])
        if head <= total - min_last and head + L[-1] >= total:
            L[-1] = total - head
            return L


def make(B, Sq, Skv, H, Dk, Dv, *, dtype="bf16", seed=0, block_size=64, top_k=16,
         window=512, scale=None, kv_mult=None, kv_lens=None, doc_lens=None,
         sink=True, scaled_block_every=0, name="custom") -> Problem:
    """Generic seeded problem.

    kv_lens: per-batch valid lengths (rows past them are NaN); doc_lens: packed
    document lengths for B == 1 (they must sum to Sq == Skv)."""
    g = torch.Generator().manual_seed(seed)
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if kv_mult is None:
        kv_mult = 1.0 if dtype == "f32" else 4.0 / math.sqrt(Dk)
    doc_start = doc_end = None
    if doc_lens is not None:
        assert B == 1 and sum(doc_lens) == Sq == Skv
        doc_start, doc_end, s = [], [], 0
        for L in doc_lens:
            doc_start.append(s)
            doc_end.append(s + L)
            s += L
    q = _draw_rows(g, B * Sq, (H, Dk), 1.0, dtype).view(B, Sq, H, Dk)
    kv = torch.empty((B, Skv, Dk), dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
    row_scale = None
    if scaled_block_every:
        def row_scale(r0, r1, bs=block_size, every=scaled_block_every):
            idx = torch.arange(r0, r1)
            return torch.where((idx // bs) % every == 0, 3.0, 1.0).to(torch.float32)
    for b in range(B):
        L = Skv if kv_lens is None else kv_lens[b]
        if L > 0:
            kv[b, :L] = _draw_rows(g, L, (Dk,), kv_mult, dtype, row_scale)
        if L < Skv:
            kv[b, L:] = float("nan")
    sk = torch.randn((H,), generator=g, dtype=torch.float32) if sink else None
    return Problem(name=name, dtype=dtype, B=B, Sq=Sq, Skv=Skv, H=H, Dk=Dk, Dv=Dv,
                   block_size=block_size, top_k=top_k, window=window, scale=float(scale),
                   kv_lens=list(kv_lens) if kv_lens is not None else None,
                   doc_start=doc_start, doc_end=doc_end, q=q, kv=kv, sink=sk)


def config(c: int) -> Problem:
    """The five named workloads, seeded with their own number."""
    if c == 1:
        return make(1, 512, 512, 8, 96, 64, dtype="f32", seed=1, top_k=4, window=128,
                    scale=1.0 / math.sqrt(96), name="tiny_f32_S512_H8_D96")
    if c == 2:
        return make(1, 4096, 4096, 64, 576, 512, seed=2, top_k=16, window=512,
                    name="mla_S4096_H64_D576")
    if c == 3:
        return make(1, 32768, 32768, 64, 576, 512, seed=3, top_k=32, window=1024,
                    scaled_block_every=4, name="mla_S32768_H64_D576_topk32")
    if c == 4:
        g = torch.Generator().manual_seed(4)
        lens = doc_lengths_packed(g)
        # Lengths come first in the draw order; continue with the same generator.
        return _make_with_generator(g, 4, lens)
    if c == 5:
        g = torch.Generator().manual_seed(5)
        lens = torch.randint(16384, 65536 + 1, (32,), generator=g).tolist()
        return _make_decode_with_generator(g, lens)
    raise ValueError(f"unknown workload {c}")


def _make_with_generator(g, seed, lens) -> Problem:
    S = sum(lens)
    H, Dk, Dv = 64, 576, 512
    q = _draw_rows(g, S, (H, Dk), 1.0, "bf16").view(1, S, H, Dk)
    kv = _draw_rows(g, S, (Dk,), 4.0 / math.sqrt(Dk), "bf16").view(1, S, Dk)
    sink = torch.randn((H,), generator=g, dtype=torch.float32)
    ds, de, s = [], [], 0
    for L in lens:
        ds.append(s)
        de.append(s + L)
        s += L
    return Problem(name="packed_8docs_S16384", dtype="bf16", B=1, Sq=S, Skv=S, H=H, Dk=Dk,
                   Dv=Dv, block_size=64, top_k=16, window=512, scale=1.0 / math.sqrt(Dk),
                   doc_start=ds, doc_end=de, q=q, kv=kv, sink=sink)


def _make_decode_with_generator(g, lens) -> Problem:
    B, Skv, H, Dk, Dv = len(lens), 65536, 64, 576, 512
    q = _draw_rows(g, B, (H, Dk), 1.0, "bf16").view(B, 1, H, Dk)
    kv = torch.empty((B, Skv, Dk), dtype=torch.bfloat16)
    for b, L in enumerate(lens):
        kv[b, :L] = _draw_rows(g, L, (Dk,), 4.0 / math.sqrt(Dk), "bf16")
        kv[b, L:] = float("nan")
    sink = torch.randn((H,), generator=g, dtype=torch.float32)
    return Problem(name="decode_B32_L16k-64k", dtype="bf16", B=B, Sq=1, Skv=Skv, H=H, Dk=Dk,
                   Dv=Dv, block_size=64, top_k=32, window=1024, scale=1.0 / math.sqrt(Dk),
                   kv_lens=list(lens), q=q, kv=kv, sink=sink)


def make_dout(p: Problem, seed: int) -> torch.Tensor:
    """Seeded upstream gradient of the attention output: [B, Sq, H, Dv]."""
    g = torch.Generator().manual_seed(seed)
    d = _draw_rows(g, p.B * p.Sq, (p.H, p.Dv), 1.0, p.dtype)
    return d.view(p.B, p.Sq, p.H, p.Dv)
