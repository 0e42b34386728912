"""Helpers shared by the GPU parity tests: move a seeded problem to the
device, call the library, and compare with the float64 oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs
from oracle import hysparse_ref as ref

BF16_TOL = 2e-2
F32_TOL = 1e-4
BLOCK_LOGIT_TOL = 2e-4      # diagnostic: scores of the same inputs
MARGIN = 1e-3               # top-k parity is exact when the k-th gap exceeds this


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class Dev:
    """A seeded problem resident on the GPU."""

    def __init__(self, p: inputs.Problem, sink: bool = True):
        self.p = p
        self.q = p.q.cuda().contiguous()
        self.kv = p.kv.cuda().contiguous()
        self.sink = p.sink.cuda().contiguous() if (sink and p.sink is not None) else None
        self.sink_cpu = p.sink if (sink and p.sink is not None) else None
        self.prob = hs.Problem(p.B, p.Sq, p.Skv, p.H, p.Dk, p.Dv, block_size=p.block_size,
                               scale=p.scale, dtype=p.dtype, kv_lens=p.kv_lens,
                               doc_start=p.doc_start, doc_end=p.doc_end)

    def kw(self):
        p = self.p
        return dict(block_size=p.block_size, kv_lens=p.kv_lens, doc_start=p.doc_start,
                    doc_end=p.doc_end)

    def own(self, rows=None):
        p = self.p
        return ref.own_blocks(p.B, p.Sq, p.Skv, p.block_size, p.kv_lens, p.doc_start, p.doc_end,
                              rows=rows)


def tol_for(p) -> float:
    return F32_TOL if p.dtype == "f32" else BF16_TOL


def np64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got, want, tol, name):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert not np.isnan(got).any(), f"{name}: NaN in GPU result"
    gi, wi = np.isneginf(got), np.isneginf(want)
    assert np.array_equal(gi, wi), f"{name}: -inf pattern differs at {np.argwhere(gi != wi)[:5]}"
    f = ~wi
    if f.any():
        err = np.abs(got[f] - want[f]).max()
        assert err <= tol, f"{name}: max-abs error {err:.3e} > {tol:.1e}"
        return float(err)
    return 0.0


def check_topk_margin(idx_gpu, bl_oracle, own, K):
    """Index parity under the margin rule: exact where the oracle's k-th gap
    exceeds MARGIN; otherwise a valid choice among near-ties: the own block,
    K distinct ascending entries, none more than MARGIN below the cut (the
    oracle's last selected value) and every block more than MARGIN above the
    cut present. Returns the share of rows checked exactly."""
    idx_gpu = np.asarray(idx_gpu)
    rows = idx_gpu.reshape(-1, K)
    blf = bl_oracle.reshape(rows.shape[0], -1)
    ownf = np.asarray(own).reshape(-1)
    want = ref.topk_blocks(blf, ownf, K)
    exact = 0
    for i in range(rows.shape[0]):
        C = np.where(blf[i] > -np.inf)[0]
        if len(C) <= K:
            assert np.array_equal(rows[i], want[i]), (i, rows[i], want[i])
            exact += 1
            continue
        o = ownf[i]
        others = np.array([j for j in C if j != o])
        vals = np.sort(blf[i, others])[::-1]
        kk = K - 1 if o in C else K
        margin = vals[kk - 1] - vals[kk] if kk >= 1 else np.inf
        if margin > MARGIN:
            assert np.array_equal(rows[i], want[i]), (i, rows[i], want[i], margin)
            exact += 1
        else:
            got = rows[i]
            assert np.all(got >= 0) and len(set(got.tolist())) == K and np.all(np.diff(got) > 0)
            if o in C:
                assert o in got
            cut = vals[kk - 1]
            for j in got:
                if j != o:
                    assert blf[i, j] >= cut - MARGIN, (i, j, blf[i, j], cut)
            # every block clearly above the cut must be selected
            clear = others[blf[i, others] > cut + MARGIN]
            assert np.isin(clear, got).all(), (i, clear, got, cut)
    return exact / max(1, rows.shape[0])


def sample_rows(p, n, seed=0):
    """First and last rows, rows around block and document edges, and uniform rows."""
    rng = np.random.default_rng(seed)
    S = p.Sq
    rows = set(range(min(S, 8))) | set(range(max(0, S - 8), S))
    for e in range(64, S, 64 * max(1, S // (64 * 16))):
        rows |= {e - 1, e} if e < S else set()
    if p.doc_start:
        for s0 in p.doc_start[1:]:
            rows |= {s0 - 1, s0, min(S - 1, s0 + 63), min(S - 1, s0 + 64)}
    rest = max(0, n - len(rows))
    rows |= set(rng.integers(0, S, size=rest).tolist())
    return np.array(sorted(rows))
