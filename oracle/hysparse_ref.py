"""Float64 reference of the HySparse MQA path: the forward operations and the
gradients of the three attention operations (test infrastructure only).

Sources (the pages this restates, cited by title and section):

* "HySparse MQA sparse attention (FA4 block scoring + SWA MQA + block-sparse DSA
  gather)" (PaddleFleet pull request 1470), sections "What" and "Core", and the
  per-file overview table (rows for block_score_fa4.py, pipeline.py,
  swa_attn.py, windowed_mqa_attn*.py and block_sparse_mqa_dsa.py): the method
  is three cooperating structures -- causal full attention fused with a scaled
  per-key-block score, per-token top-k block selection, and block-sparse gather
  attention -- plus a sliding-window MQA branch, each with an optional
  learnable per-head attention sink.
* Same page, section "FlashMLA sparse kernel constraints": absorbed-MLA MQA
  layout, one shared KV head, V is the leading d_v columns of the latent K.
* Review of PaddleFleet pull request 1453, comments on the block-score PyLayer
  (inputs include a document mask and ``block_bos``, the per-block start row):
  blocks restart at each document's first row and never cross a document.
* Blog page on the unified sparse-attention dispatcher, section on choosing a
  sparse scheme in the model config (decode builds the mask against key length
  = cache + current token): a decode token sits at the last cache row.

Notation: row r of batch b sits at absolute position p = L_b - Sq + r, where
L_b is the valid KV length. The allowed key set of position p is
A(p) = {i : doc_start(p) <= i <= p}. Scores are s[h, i] = scale * q[h] . k[i]
over all Dk columns; values are v[i] = k[i, :Dv].

attend(S) with sink sigma_h (-inf when absent):
    m = max(sigma_h, max_{i in S} s[h, i])
    l = exp(sigma_h - m) + sum_{i in S} exp(s[h, i] - m)
    out[h] = sum_{i in S} exp(s[h, i] - m) v[i] / l,   lse[h] = m + ln l
and out = 0, lse = -inf when S is empty and there is no sink.

Readings taken where the pages are silent (each listed in the design notes):
the block score is max over heads of the per-head natural-log log-sum-exp of
the scaled scores over the block's allowed keys, without the sink; top-k
always keeps the token's own block, orders others by (score desc, index asc),
emits indices ascending and pads with -1; the window holds W keys including
the token itself; partial blocks at a document or sequence end are real,
shorter blocks.

Rows are processed in independent chunks (each row's result is computed from
its own definition; chunking only bounds memory). All arithmetic is float64
on the exact input values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# Positions, documents and blocks.
# ---------------------------------------------------------------------------
@dataclass
class BlockTable:
    """Blocks of one batch entry, numbered globally in document order.

    start[j], end[j]: the key rows [start, end) of block j.
    doc_of_block[j]: document index of block j.
    doc_start/doc_end: the documents tiling [0, L).
    """

    start: np.ndarray
    end: np.ndarray
    doc_of_block: np.ndarray
    doc_start: np.ndarray
    doc_end: np.ndarray

    @property
    def nb(self) -> int:
        return int(self.start.shape[0])

    def block_of_key(self, L: int) -> np.ndarray:
        """Block id of every key row 0..L-1."""
        out = np.full(L, -1, dtype=np.int64)
        for j in range(self.nb):
            out[self.start[j]:self.end[j]] = j
        return out

    def doc_start_of(self, pos: np.ndarray) -> np.ndarray:
        """Start row of the document holding each position."""
        d = np.searchsorted(self.doc_start, pos, side="right") - 1
        return self.doc_start[d]


def block_table(L: int, block_size: int, doc_start: Optional[Sequence[int]] = None,
                doc_end: Optional[Sequence[int]] = None) -> BlockTable:
    """Tile each document [s_d, e_d) into blocks of ``block_size`` rows that
    restart at s_d (the per-block start row, ``block_bos``); the last block of a
    document may be shorter. Without documents there is one document [0, L)."""
    if doc_start is None:
        ds, de = [0], [L]
    else:
        ds, de = list(doc_start), list(doc_end)
    st, en, dob = [], [], []
    for d, (s, e) in enumerate(zip(ds, de)):
        m = 0
        while s + m * block_size < e:
            st.append(s + m * block_size)
            en.append(min(s + (m + 1) * block_size, e))
            dob.append(d)
            m += 1
    return BlockTable(np.array(st, dtype=np.int64), np.array(en, dtype=np.int64),
                      np.array(dob, dtype=np.int64), np.array(ds, dtype=np.int64),
                      np.array(de, dtype=np.int64))


def _valid_len(b: int, Skv: int, kv_lens) -> int:
    return Skv if kv_lens is None else int(kv_lens[b])


def num_blocks(B: int, Skv: int, block_size: int, kv_lens=None, doc_start=None,
               doc_end=None) -> int:
    """Columns of block_logit: the largest block count over the batch."""
    return max(block_table(_valid_len(b, Skv, kv_lens), block_size, doc_start, doc_end).nb
               for b in range(B))


# ---------------------------------------------------------------------------
# Attention over an explicit allowed-key mask.
# ---------------------------------------------------------------------------
def _to64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """s[r, h, i] = scale * sum_d q[r, h, d] * k[i, d]."""
    return scale * np.einsum("rhd,id->rhi", q_rows, k, optimize=True)


def _attend_masked(s: np.ndarray, allowed: np.ndarray, v: np.ndarray,
                   sink: Optional[np.ndarray]):
    """attend() for a chunk of rows.

    s: [R, H, n] scores, allowed: [R, n] bool, v: [n, Dv], sink: [H] or None.
    Returns out [R, H, Dv], lse [R, H]."""
    R, H, n = s.shape
    sm = np.where(allowed[:, None, :], s, NEG_INF)
    m = sm.max(axis=2) if n > 0 else np.full((R, H), NEG_INF)
    if sink is not None:
        m = np.maximum(m, sink[None, :])
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.where(allowed[:, None, :], np.exp(sm - m_safe[:, :, None]), 0.0)
    l = e.sum(axis=2)
    if sink is not None:
        l = l + np.exp(sink[None, :] - m_safe)
    num = np.einsum("rhi,id->rhd", e, v, optimize=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(finite[:, :, None], num / np.where(l > 0, l, 1.0)[:, :, None], 0.0)
        lse = np.where(finite, m_safe + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return out, lse


def attend_subset(q_row: np.ndarray, k: np.ndarray, Dv: int, scale: float, keys,
                  sink=None):
    """attend() of one query row ([H, Dk]) over an explicit list of key rows.
    Used by the merge identity and the closed-form pins."""
    q_row = _to64(q_row)
    k = _to64(k)
    keys = np.asarray(list(keys), dtype=np.int64)
    sk = None if sink is None else _to64(sink)
    s = _scores(q_row[None], k[keys], scale)
    allowed = np.ones((1, len(keys)), dtype=bool)
    out, lse = _attend_masked(s, allowed, k[keys, :Dv], sk)
    return out[0], lse[0]


def merge_partials(outs: List[np.ndarray], lses: List[np.ndarray]):
    """Combine attend() results over disjoint key sets (each computed with no
    sink) into the result over their union: weights exp(lse_i - lse)."""
    lse_all = np.stack(lses)                       # [P, H]
    m = lse_all.max(axis=0)
    fin = np.isfinite(m)
    ms = np.where(fin, m, 0.0)
    w = np.where(np.isfinite(lse_all), np.exp(lse_all - ms), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(fin, ms + np.log(np.where(tot > 0, tot, 1.0)), NEG_INF)
    out = sum(w[i][:, None] * outs[i] for i in range(len(outs)))
    out = np.where(fin[:, None], out / np.where(tot > 0, tot, 1.0)[:, None], 0.0)
    return out, lse


# ---------------------------------------------------------------------------
# The four operations.
# ---------------------------------------------------------------------------
def _prepare(q, kv, sink, Dv):
    """Inputs stay as given (numpy or torch); rows are converted to float64
    only when used, so sampled rows of a large problem stay cheap."""
    sk = None if sink is None else _to64(sink)
    B, Sq, H, Dk = q.shape
    assert kv.shape[0] == B and kv.shape[2] == Dk and Dv <= Dk
    return q, kv, sk


def _row_chunks(rows: np.ndarray, chunk: int):
    for i in range(0, len(rows), chunk):
        yield rows[i:i + chunk]


def _chunk_masks(kind, B, Sq, Skv, H, block_size, kv_lens, doc_start, doc_end, window,
                 block_idx, rows_sel, chunk):
    """Allowed-key masks of the requested operation, one chunk of query rows
    at a time: yields (b, rr, L, kmin, kmax, allowed [len(rr), kmax-kmin],
    block id of each key in [kmin, kmax))."""
    R = len(rows_sel)
    for b in range(B):
        L = _valid_len(b, Skv, kv_lens)
        bt = block_table(L, block_size, doc_start, doc_end)
        blk_of_key = bt.block_of_key(L)
        # Bound the [rows, H, keys] float64 score array to about 2e7 entries.
        ch = chunk or max(1, int(2e7 // (H * max(1, L))))
        for rr in _row_chunks(np.arange(R), ch):
            pos = L - Sq + rows_sel[rr]                       # absolute positions
            lo = bt.doc_start_of(pos)                         # document start
            hi = pos                                          # causal limit
            kmin, kmax = int(lo.min()), int(hi.max()) + 1
            keys = np.arange(kmin, kmax)
            allowed = (keys[None, :] >= lo[:, None]) & (keys[None, :] <= hi[:, None])
            if kind == "swa":
                allowed &= keys[None, :] >= (pos - window + 1)[:, None]
            elif kind == "gather":
                sel = block_idx[b, rows_sel[rr]]              # [r, K]
                kb = blk_of_key[kmin:kmax]                    # block of each key
                member = np.zeros(allowed.shape, dtype=bool)
                for t in range(sel.shape[1]):
                    j = sel[:, t]
                    ok = (j >= 0) & (j < bt.nb)
                    member |= ok[:, None] & (kb[None, :] == j[:, None])
                allowed &= member
            yield b, rr, L, kmin, kmax, allowed, blk_of_key[kmin:kmax]


def _op(kind, q, kv, sink, Dv, scale, block_size, kv_lens=None, doc_start=None,
        doc_end=None, window=None, block_idx=None, rows=None, chunk=None):
    """Shared driver: for each batch entry and chunk of query rows, build the
    allowed-key mask of the requested operation and attend over it."""
    q, kv, sk = _prepare(q, kv, sink, Dv)
    B, Sq, H, Dk = q.shape
    Skv = kv.shape[1]
    rows_sel = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows_sel)
    NB = num_blocks(B, Skv, block_size, kv_lens, doc_start, doc_end)
    out = np.zeros((B, R, H, Dv))
    lse = np.full((B, R, H), NEG_INF)
    blog = np.full((B, R, NB), NEG_INF) if kind == "score" else None
    k_entry, k_b = None, -1
    for b, rr, L, kmin, kmax, allowed, kb in _chunk_masks(
            kind, B, Sq, Skv, H, block_size, kv_lens, doc_start, doc_end, window, block_idx,
            rows_sel, chunk):
        if b != k_b:
            k_entry, k_b = _to64(kv[b, :L]), b
        k = k_entry
        v = k[:, :Dv]
        s = _scores(_to64(q[b, rows_sel[rr]]), k[kmin:kmax], scale)
        o, ls = _attend_masked(s, allowed, v[kmin:kmax], sk)
        out[b, rr] = o
        lse[b, rr] = ls
        if kind == "score":
            # block_logit[p, j] = max_h ln sum_{i in blk j, i in A(p)} exp(s[h, i])
            for j in np.unique(kb):
                cols = kb == j
                a = allowed[:, cols]                          # [r, n_j]
                sj = np.where(a[:, None, :], s[:, :, cols], NEG_INF)
                mj = sj.max(axis=2)                           # [r, H]
                fin = np.isfinite(mj)
                mjs = np.where(fin, mj, 0.0)
                with np.errstate(divide="ignore"):
                    lj = np.where(fin, mjs + np.log(np.exp(sj - mjs[:, :, None]).sum(axis=2)),
                                  NEG_INF)
                blog[b, rr, j] = lj.max(axis=1)
    return out, lse, blog


def block_score(q, kv, sink, Dv, scale, block_size=64, kv_lens=None, doc_start=None,
                doc_end=None, rows=None):
    """Causal full attention with sink plus per-block scores.

    Returns out [B,R,H,Dv], lse [B,R,H] (natural log, sink included) and
    block_logit [B,R,NB] (sink excluded; -inf for blocks with no allowed key)."""
    return _op("score", q, kv, sink, Dv, scale, block_size, kv_lens, doc_start, doc_end,
               rows=rows)


def swa(q, kv, sink, Dv, scale, window, block_size=64, kv_lens=None, doc_start=None,
        doc_end=None, rows=None):
    """Sliding-window attention: keys in A(p) with i >= p - window + 1."""
    out, lse, _ = _op("swa", q, kv, sink, Dv, scale, block_size, kv_lens, doc_start,
                      doc_end, window=window, rows=rows)
    return out, lse


def sparse_gather(q, kv, sink, Dv, scale, block_idx, block_size=64, kv_lens=None,
                  doc_start=None, doc_end=None, rows=None):
    """Attention over the union of the selected blocks intersected with A(p).

    block_idx: [B, Sq, K] int; entries < 0 or >= NB are skipped; the entries of
    a row are taken as a set."""
    bi = np.asarray(block_idx.cpu() if hasattr(block_idx, "cpu") else block_idx,
                    dtype=np.int64)
    out, lse, _ = _op("gather", q, kv, sink, Dv, scale, block_size, kv_lens, doc_start,
                      doc_end, block_idx=bi, rows=rows)
    return out, lse


# ---------------------------------------------------------------------------
# Gradients of the three attention operations.
# ---------------------------------------------------------------------------
def _op_bwd(kind, q, kv, sink, Dv, scale, dout, block_size, kv_lens=None, doc_start=None,
            doc_end=None, window=None, block_idx=None, chunk=None, rows=None, dlse=None):
    """Gradients of L = sum(dout * out) + sum(dlse * lse) for one attention
    operation (dlse optional: [B, Sq, H], or the rows' when rows is given).

    The pages train through these kernels: page "HySparse MQA sparse attention
    ...", section "Core" (block scoring with gradients routed through the
    autograd layer, the analytic gradient of the learnable per-head sink) and
    the per-file table rows for windowed_mqa_attn*.py and
    block_sparse_mqa_dsa.py (forward and backward kernels); review of
    PaddleFleet PR 1453, block-score PyLayer comments (the backward returns
    gradients for q, k and v only: block_logit and the block table get none).

    For one row and head, with P_i = exp(s_i - lse) over the allowed set,
    P_sink = exp(sigma - lse) and out = sum_i P_i v_i, the chain rule gives
        dP_i  = dout . v_i,          Dsum = dout . out = sum_i P_i dP_i,
        dL/ds_i    = P_i (dP_i - Dsum),
        dL/dsigma  = -P_sink Dsum   (the sink enters the normaliser only),
    and through s_i = scale q . k_i:
        dq   = scale sum_i dL/ds_i k_i,
        dk_i = scale sum_{rows, heads} dL/ds_i q,   dv_i = sum_{rows, heads} P_i dout.
    The latent row kv_i serves as both key and value (value = its leading Dv
    columns), so dkv_i = dk_i + [dv_i, 0]. An incoming gradient of lse adds
    dL/ds_i += dlse P_i (d lse / d s_i = P_i) and dL/dsigma += dlse P_sink, so
    both formulas hold with Dsum replaced by Dsum - dlse. Returns dq [B,Sq,H,Dk],
    dkv [B,Skv,Dk] (zero past each entry's valid length) and dsink [H]
    (None without a sink).

    rows: optionally only these query rows (dout is then [B, len(rows), H,
    Dv]): dq [B, len(rows), H, Dk] for them, and the dkv and dsink
    contributions of these rows alone (complete for a key that no other row
    attends to)."""
    q, kv, sk = _prepare(q, kv, sink, Dv)
    B, Sq, H, Dk = q.shape
    Skv = kv.shape[1]
    g_all = dout
    dl_all = None if dlse is None else _to64(dlse)
    rows_sel = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    dq = np.zeros((B, len(rows_sel), H, Dk))
    dkv = np.zeros((B, Skv, Dk))
    dsink = None if sk is None else np.zeros(H)
    k_entry, k_b = None, -1
    for b, rr, L, kmin, kmax, allowed, _ in _chunk_masks(
            kind, B, Sq, Skv, H, block_size, kv_lens, doc_start, doc_end, window, block_idx,
            rows_sel, chunk):
        if b != k_b:
            k_entry, k_b = _to64(kv[b, :L]), b
        k = k_entry[kmin:kmax]
        v = k[:, :Dv]
        qr = _to64(q[b, rows_sel[rr]])                        # [r, H, Dk]
        g = _to64(g_all[b, rr])                               # [r, H, Dv]
        s = _scores(qr, k, scale)                             # [r, H, n]
        out, lse = _attend_masked(s, allowed, v, sk)
        fin = np.isfinite(lse)
        lse_s = np.where(fin, lse, 0.0)
        P = np.where(allowed[:, None, :] & fin[:, :, None], np.exp(s - lse_s[:, :, None]), 0.0)
        dP = np.einsum("rhd,id->rhi", g, v, optimize=True)
        Dsum = np.einsum("rhd,rhd->rh", g, out, optimize=True)
        if dl_all is not None:
            Dsum = Dsum - dl_all[b, rr]
        dS = P * (dP - Dsum[:, :, None])
        dq[b, rr] = scale * np.einsum("rhi,id->rhd", dS, k, optimize=True)
        dkv[b, kmin:kmax] += scale * np.einsum("rhi,rhd->id", dS, qr, optimize=True)
        dkv[b, kmin:kmax, :Dv] += np.einsum("rhi,rhd->id", P, g, optimize=True)
        if dsink is not None:
            psink = np.where(fin, np.exp(sk[None, :] - lse_s), 0.0)
            dsink -= (psink * Dsum).sum(axis=0)
    return dq, dkv, dsink


def block_score_bwd(q, kv, sink, Dv, scale, dout, block_size=64, kv_lens=None,
                    doc_start=None, doc_end=None, chunk=None, rows=None, dlse=None):
    """Gradients of the causal attention of block_score (block_logit has none)."""
    return _op_bwd("score", q, kv, sink, Dv, scale, dout, block_size, kv_lens, doc_start,
                   doc_end, chunk=chunk, rows=rows, dlse=dlse)


def swa_bwd(q, kv, sink, Dv, scale, window, dout, block_size=64, kv_lens=None,
            doc_start=None, doc_end=None, chunk=None, rows=None, dlse=None):
    """Gradients of the sliding-window attention."""
    return _op_bwd("swa", q, kv, sink, Dv, scale, dout, block_size, kv_lens, doc_start,
                   doc_end, window=window, chunk=chunk, rows=rows, dlse=dlse)


def sparse_gather_bwd(q, kv, sink, Dv, scale, block_idx, dout, block_size=64, kv_lens=None,
                      doc_start=None, doc_end=None, chunk=None, rows=None, dlse=None):
    """Gradients of the block-sparse gather attention for a fixed selection."""
    bi = np.asarray(block_idx.cpu() if hasattr(block_idx, "cpu") else block_idx,
                    dtype=np.int64)
    return _op_bwd("gather", q, kv, sink, Dv, scale, dout, block_size, kv_lens, doc_start,
                   doc_end, block_idx=bi, chunk=chunk, rows=rows, dlse=dlse)


def own_blocks(B, Sq, Skv, block_size, kv_lens=None, doc_start=None, doc_end=None,
               rows=None) -> np.ndarray:
    """Block id holding each query row's own position: [B, R]."""
    rows_sel = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    own = np.zeros((B, len(rows_sel)), dtype=np.int64)
    for b in range(B):
        L = _valid_len(b, Skv, kv_lens)
        bt = block_table(L, block_size, doc_start, doc_end)
        own[b] = bt.block_of_key(L)[L - Sq + rows_sel]
    return own


def topk_blocks(block_logit, own, top_k: int) -> np.ndarray:
    """Per-row block selection.

    C = {j : block_logit[j] > -inf}. If |C| <= K all of C is kept; otherwise the
    own block plus the first K-1 of C minus own in (score desc, index asc)
    order (the own block is always in C on the real path; were it not, the
    first K of C are kept). Emitted ascending, padded with -1 to K entries. Comparisons are made
    on the values as given (fp32 inputs compare exactly)."""
    bl = np.asarray(block_logit.cpu() if hasattr(block_logit, "cpu") else block_logit)
    own = np.asarray(own, dtype=np.int64)
    lead = bl.shape[:-1]
    flat = bl.reshape(-1, bl.shape[-1])
    own_f = own.reshape(-1)
    res = np.full((flat.shape[0], top_k), -1, dtype=np.int64)
    for r in range(flat.shape[0]):
        row = flat[r]
        cand = [j for j in range(row.shape[0]) if row[j] > NEG_INF]
        if len(cand) <= top_k:
            chosen = cand
        else:
            o = int(own_f[r])
            ranked = sorted(cand, key=lambda j: (-float(row[j]), j))
            if o in cand:
                chosen = [o] + [j for j in ranked if j != o][:top_k - 1]
            else:
                chosen = ranked[:top_k]
        chosen = sorted(chosen)
        res[r, :len(chosen)] = chosen
    return res.reshape(lead + (top_k,))


def block_prob(block_logit, lse) -> np.ndarray:
    """Normalised block scores (page "HySparse MQA sparse attention ...",
    per-file overview row for pipeline.py: the block probabilities are
    recovered as exp(block_logit - lse)).

    Reading: block_logit is one value per (row, block) and lse one per (row,
    head), so the row's normaliser is its largest per-head lse:
        block_prob[b, r, j] = exp(block_logit[b, r, j] - max_h lse[b, r, h]),
    and 0 where block_logit is -inf. With one head this is the page's formula
    and the row sums to the mass the attention puts on keys.

    block_logit [B, R, NB], lse [B, R, H] (natural log, sink included)."""
    bl = np.asarray(block_logit.cpu() if hasattr(block_logit, "cpu") else block_logit,
                    dtype=np.float64)
    ls = np.asarray(lse.cpu() if hasattr(lse, "cpu") else lse, dtype=np.float64)
    lmax = ls.max(axis=-1)[..., None]
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.where(np.isfinite(bl), np.exp(bl - np.where(np.isfinite(lmax), lmax, 0.0)), 0.0)
    return p


def gated_combine(out_swa, out_sparse, gate_swa, gate_sparse) -> np.ndarray:
    """Combination of the two branches of a sliding-window layer (reading: the
    page "HySparse MQA sparse attention ..." calls the method NSA-style, section
    "What", and does not state the rule; NSA combines branch outputs by a gated
    sum with per-token, per-head gates):
        out_mix[b, r, h, :] = gate_swa[b, r, h] * out_swa[b, r, h, :]
                            + gate_sparse[b, r, h] * out_sparse[b, r, h, :].
    out_* [B, R, H, Dv], gates [B, R, H]."""
    a = _to64(out_swa)
    b = _to64(out_sparse)
    ga = _to64(gate_swa)[..., None]
    gb = _to64(gate_sparse)[..., None]
    return ga * a + gb * b
