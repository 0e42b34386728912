"""Pins of the float64 oracle against facts fixed outside the oracle itself.

Each test names what it fixes. None re-implements the oracle's formula:
they use a library routine (torch's scaled_dot_product_attention and
logsumexp) on special cases that reduce to dense causal attention, closed
forms derived by hand, invariants that any correct implementation obeys, and
brute-force enumeration on tiny inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import hysparse_ref as ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-10


def _rand(seed, B, S, H, Dk, Skv=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, H, Dk))
    kv = rng.standard_normal((B, Skv or S, Dk)) * 0.5
    sink = rng.standard_normal(H)
    return q, kv, sink


def _dense_causal_sdpa(q, kv, Dv, scale):
    """Dense causal attention through torch's own SDPA in float64 (MQA: the one
    KV head is expanded over the query heads)."""
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)                    # B,H,S,Dk
    H = qt.shape[1]
    k = torch.from_numpy(kv)[:, None].expand(-1, H, -1, -1)
    v = torch.from_numpy(kv[:, :, :Dv])[:, None].expand(-1, H, -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True,
                                                           scale=scale)
    s = torch.matmul(qt, k.transpose(-1, -2).contiguous()) * scale
    S = s.shape[-1]
    mask = torch.ones(S, S, dtype=torch.bool).tril()
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


# ---------------------------------------------------------------------------
# Hand-worked closed-form example (tests/golden/hand_worked.json).
# ---------------------------------------------------------------------------
def _ev(x):
    return float(eval(x, {"ln": math.log, "inf": math.inf}))  # fixture-only expressions


@pytest.fixture(scope="module")
def gold():
    with open(os.path.join(GOLD, "hand_worked.json")) as f:
        g = json.load(f)
    kv = np.array([[v, _ev(a)] for v, a in g["keys"]], dtype=np.float64)[None]  # [1,4,2]
    q = np.tile(np.array(g["query"], dtype=np.float64), (1, 4, 1, 1))           # [1,4,1,2]
    return g, q, kv


def _same(a, b, tol=TOL):
    """Equal -inf pattern and finite values within tol."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if not np.array_equal(np.isneginf(a), np.isneginf(b)):
        return False
    f = np.isfinite(a)
    return bool(np.allclose(a[f], b[f], atol=tol))


def _close(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    diff = np.abs(np.where(both_inf, 0.0, a) - np.where(both_inf, 0.0, b))
    return bool(np.all(both_inf | (diff <= 1e-12)))


def test_golden_causal_and_block_logit(gold):
    g, q, kv = gold
    out, lse, bl = ref.block_score(q, kv, None, 1, 1.0, block_size=g["block_size"])
    assert _close(out[0, :, 0, 0], [_ev(x) for x in g["causal"]["out"]])
    assert _close(lse[0, :, 0], [_ev(x) for x in g["causal"]["lse"]])
    assert _close(bl[0], [[_ev(x) for x in r] for r in g["causal"]["block_logit"]])


def test_golden_sink(gold):
    g, q, kv = gold
    sink = np.array([_ev(g["causal_sink_ln2"]["sink"])])
    out, lse, _ = ref.block_score(q, kv, sink, 1, 1.0, block_size=g["block_size"])
    assert _close(out[0, :, 0, 0], [_ev(x) for x in g["causal_sink_ln2"]["out"]])
    assert _close(lse[0, :, 0], [_ev(x) for x in g["causal_sink_ln2"]["lse"]])


def test_golden_topk_gather_swa(gold):
    g, q, kv = gold
    _, _, bl = ref.block_score(q, kv, None, 1, 1.0, block_size=2)
    own = ref.own_blocks(1, 4, 4, 2)
    assert ref.topk_blocks(bl, own, 1)[0].tolist() == g["topk_k1"]
    assert ref.topk_blocks(bl, own, 2)[0].tolist() == g["topk_k2"]
    idx = ref.topk_blocks(bl, own, 1)
    out, lse = ref.sparse_gather(q, kv, None, 1, 1.0, idx, block_size=2)
    assert _close(out[0, :, 0, 0], [_ev(x) for x in g["gather_k1"]["out"]])
    assert _close(lse[0, :, 0], [_ev(x) for x in g["gather_k1"]["lse"]])
    out, lse = ref.swa(q, kv, None, 1, 1.0, 2, block_size=2)
    assert _close(out[0, :, 0, 0], [_ev(x) for x in g["swa_w2"]["out"]])
    assert _close(lse[0, :, 0], [_ev(x) for x in g["swa_w2"]["lse"]])


def test_golden_documents(gold):
    g, q, kv = gold
    d = g["docs_0_1_4"]
    bt = ref.block_table(4, 2, d["doc_start"], d["doc_end"])
    assert bt.start.tolist() == d["block_starts"] and bt.end.tolist() == d["block_ends"]
    out, lse, bl = ref.block_score(q, kv, None, 1, 1.0, block_size=2,
                                   doc_start=d["doc_start"], doc_end=d["doc_end"])
    assert _close(out[0, :, 0, 0], [_ev(x) for x in d["out"]])
    assert _close(lse[0, :, 0], [_ev(x) for x in d["lse"]])
    assert _close(bl[0], [[_ev(x) for x in r] for r in d["block_logit"]])


def test_golden_decode(gold):
    g, q, kv = gold
    d = g["decode_lens_3_4"]
    kvb = np.concatenate([kv, kv], axis=0).copy()
    kvb[0, 3] = np.nan                            # past the first cache's length
    qd = np.tile(q[:, :1], (2, 1, 1, 1))          # one new token per sequence
    out, lse, bl = ref.block_score(qd, kvb, None, 1, 1.0, block_size=2, kv_lens=d["kv_lens"])
    assert _close(out[:, 0, 0, 0], [_ev(x) for x in d["out"]])
    assert _close(lse[:, 0, 0], [_ev(x) for x in d["lse"]])
    assert _close(bl[:, 0], [[_ev(x) for x in r] for r in d["block_logit"]])


# ---------------------------------------------------------------------------
# P1 / P2: full coverage equals dense causal attention (library routine).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S,H,Dk,Dv,bs", [(37, 3, 16, 8, 8), (70, 2, 12, 12, 16), (64, 4, 8, 4, 64)])
def test_full_coverage_equals_dense(S, H, Dk, Dv, bs):
    q, kv, _ = _rand(S * 7 + H, 1, S, H, Dk)
    scale = 0.37
    o_ref, l_ref = _dense_causal_sdpa(q, kv, Dv, scale)
    o, l, bl = ref.block_score(q, kv, None, Dv, scale, block_size=bs)
    assert np.allclose(o, o_ref, atol=TOL) and np.allclose(l, l_ref, atol=TOL)
    o, l = ref.swa(q, kv, None, Dv, scale, window=S, block_size=bs)
    assert np.allclose(o, o_ref, atol=TOL) and np.allclose(l, l_ref, atol=TOL)
    NB = bl.shape[-1]
    own = ref.own_blocks(1, S, S, bs)
    idx = ref.topk_blocks(bl, own, NB)                 # K >= NB keeps every finite block
    o, l = ref.sparse_gather(q, kv, None, Dv, scale, idx, block_size=bs)
    assert np.allclose(o, o_ref, atol=TOL) and np.allclose(l, l_ref, atol=TOL)
    # All blocks listed explicitly (including ones past the causal limit).
    idx_all = np.tile(np.arange(NB), (1, S, 1))
    o, l = ref.sparse_gather(q, kv, None, Dv, scale, idx_all, block_size=bs)
    assert np.allclose(o, o_ref, atol=TOL) and np.allclose(l, l_ref, atol=TOL)


# ---------------------------------------------------------------------------
# P3: sink closed form; sink = -inf equals no sink.
# ---------------------------------------------------------------------------
def test_sink_closed_form():
    q, kv, sink = _rand(3, 1, 45, 4, 16)
    Dv, scale = 8, 0.25
    o0, l0, b0 = ref.block_score(q, kv, None, Dv, scale, block_size=16)
    o1, l1, b1 = ref.block_score(q, kv, sink, Dv, scale, block_size=16)
    sig = 1.0 / (1.0 + np.exp(-(l0 - sink[None, None, :])))
    assert np.allclose(o1, o0 * sig[..., None], atol=TOL)
    assert np.allclose(l1, np.logaddexp(l0, sink[None, None, :]), atol=TOL)
    assert np.array_equal(b0, b1)                      # the sink never enters the block score
    oi, li, _ = ref.block_score(q, kv, np.full(4, -np.inf), Dv, scale, block_size=16)
    assert np.allclose(oi, o0, atol=TOL) and np.allclose(li, l0, atol=TOL)
    for fn in (lambda s: ref.swa(q, kv, s, Dv, scale, 7, block_size=16),):
        a0, m0 = fn(None)
        a1, m1 = fn(sink)
        sg = 1.0 / (1.0 + np.exp(-(m0 - sink[None, None, :])))
        assert np.allclose(a1, a0 * sg[..., None], atol=TOL)
        assert np.allclose(m1, np.logaddexp(m0, sink[None, None, :]), atol=TOL)


# ---------------------------------------------------------------------------
# P4: block scores partition the normaliser; max over heads.
# ---------------------------------------------------------------------------
def test_block_logit_partition_and_head_max():
    q, kv, _ = _rand(4, 1, 90, 3, 12)
    scale, bs = 0.4, 16
    _, l0, bl = ref.block_score(q, kv, None, 4, scale, block_size=bs)
    per_head = []
    for h in range(3):
        _, lh, blh = ref.block_score(q[:, :, h:h + 1], kv, None, 4, scale, block_size=bs)
        # With one head the block scores partition that head's normaliser.
        t = torch.from_numpy(blh[0])
        assert np.allclose(torch.logsumexp(t, dim=-1).numpy(), lh[0, :, 0], atol=TOL)
        per_head.append(blh)
    mx = np.maximum.reduce(per_head)
    assert np.array_equal(np.isinf(bl), np.isinf(mx))
    assert np.allclose(bl, mx, atol=TOL)


# ---------------------------------------------------------------------------
# P5: window of one key has a closed form.
# ---------------------------------------------------------------------------
def test_window_one_closed_form():
    q, kv, sink = _rand(5, 1, 33, 2, 10)
    Dv, scale = 6, 0.3
    o, l = ref.swa(q, kv, sink, Dv, scale, 1, block_size=8)
    for t in range(33):
        for h in range(2):
            s = scale * float(q[0, t, h] @ kv[0, t])
            w = 1.0 / (1.0 + math.exp(sink[h] - s))
            assert np.allclose(o[0, t, h], kv[0, t, :Dv] * w, atol=TOL)
            assert abs(l[0, t, h] - np.logaddexp(s, sink[h])) < TOL


# ---------------------------------------------------------------------------
# P6: top_k = 1 gather equals block-diagonal causal attention (each block its
# own document).
# ---------------------------------------------------------------------------
def test_topk_one_is_block_diagonal():
    S, bs = 75, 16
    q, kv, sink = _rand(6, 1, S, 2, 8)
    Dv, scale = 4, 0.5
    _, _, bl = ref.block_score(q, kv, sink, Dv, scale, block_size=bs)
    own = ref.own_blocks(1, S, S, bs)
    idx = ref.topk_blocks(bl, own, 1)
    assert np.array_equal(idx[..., 0], own)
    og, lg = ref.sparse_gather(q, kv, sink, Dv, scale, idx, block_size=bs)
    starts = list(range(0, S, bs))
    ends = [min(s + bs, S) for s in starts]
    ob, lb, _ = ref.block_score(q, kv, sink, Dv, scale, block_size=bs, doc_start=starts,
                                doc_end=ends)
    assert np.allclose(og, ob, atol=TOL) and np.allclose(lg, lb, atol=TOL)


# ---------------------------------------------------------------------------
# P7: decode equals the last prefill row.
# ---------------------------------------------------------------------------
def test_decode_equals_last_prefill_row():
    S, H, Dk, Dv, bs, K, W = 70, 2, 8, 4, 16, 2, 20
    q, kv, sink = _rand(7, 1, S, H, Dk)
    lens = [50, 70, 17]
    kvb = np.full((3, S, Dk), np.nan)
    qd = np.zeros((3, 1, H, Dk))
    for b, L in enumerate(lens):
        kvb[b, :L] = kv[0, :L]
        qd[b, 0] = q[0, L - 1]
    od, ld, bd = ref.block_score(qd, kvb, sink, Dv, 0.3, block_size=bs, kv_lens=lens)
    owd = ref.own_blocks(3, 1, S, bs, kv_lens=lens)
    idd = ref.topk_blocks(bd, owd, K)
    ogd, lgd = ref.sparse_gather(qd, kvb, sink, Dv, 0.3, idd, block_size=bs, kv_lens=lens)
    osd, lsd = ref.swa(qd, kvb, sink, Dv, 0.3, W, block_size=bs, kv_lens=lens)
    for b, L in enumerate(lens):
        op, lp, bp = ref.block_score(q[:, :L], kv[:, :L], sink, Dv, 0.3, block_size=bs)
        assert np.allclose(od[b, 0], op[0, L - 1], atol=TOL)
        assert np.allclose(ld[b, 0], lp[0, L - 1], atol=TOL)
        nb = bp.shape[-1]
        assert _same(bd[b, 0, :nb], bp[0, L - 1])
        assert np.all(np.isneginf(bd[b, 0, nb:]))
        own = ref.own_blocks(1, L, L, bs)
        ip = ref.topk_blocks(bp, own, K)
        assert np.array_equal(idd[b, 0], ip[0, L - 1])
        og, lg = ref.sparse_gather(q[:, :L], kv[:, :L], sink, Dv, 0.3, ip, block_size=bs)
        assert np.allclose(ogd[b, 0], og[0, L - 1], atol=TOL)
        assert np.allclose(lgd[b, 0], lg[0, L - 1], atol=TOL)
        os_, ls_ = ref.swa(q[:, :L], kv[:, :L], sink, Dv, 0.3, W, block_size=bs)
        assert np.allclose(osd[b, 0], os_[0, L - 1], atol=TOL)
        assert np.allclose(lsd[b, 0], ls_[0, L - 1], atol=TOL)
        assert np.all(np.isfinite(od[b])) and np.all(np.isfinite(ogd[b]))


# ---------------------------------------------------------------------------
# P8: packed documents equal per-document runs, concatenated.
# ---------------------------------------------------------------------------
def test_packed_documents_equal_separate_runs():
    lens = [20, 1, 40, 33]
    S, H, Dk, Dv, bs, K, W = sum(lens), 2, 8, 4, 16, 2, 9
    q, kv, sink = _rand(8, 1, S, H, Dk)
    ds = np.cumsum([0] + lens[:-1]).tolist()
    de = np.cumsum(lens).tolist()
    o, l, bl = ref.block_score(q, kv, sink, Dv, 0.3, block_size=bs, doc_start=ds, doc_end=de)
    own = ref.own_blocks(1, S, S, bs, doc_start=ds, doc_end=de)
    idx = ref.topk_blocks(bl, own, K)
    og, lg = ref.sparse_gather(q, kv, sink, Dv, 0.3, idx, block_size=bs, doc_start=ds, doc_end=de)
    osw, lsw = ref.swa(q, kv, sink, Dv, 0.3, W, block_size=bs, doc_start=ds, doc_end=de)
    off = 0
    for s0, e0 in zip(ds, de):
        qs, ks = q[:, s0:e0], kv[:, s0:e0]
        op, lp, bp = ref.block_score(qs, ks, sink, Dv, 0.3, block_size=bs)
        nb = bp.shape[-1]
        assert np.allclose(o[0, s0:e0], op[0], atol=TOL)
        assert np.allclose(l[0, s0:e0], lp[0], atol=TOL)
        assert _same(bl[0, s0:e0, off:off + nb], bp[0])
        rest = np.delete(bl[0, s0:e0], np.s_[off:off + nb], axis=1)
        assert np.all(np.isneginf(rest))                    # no block crosses a document
        ip = ref.topk_blocks(bp, ref.own_blocks(1, e0 - s0, e0 - s0, bs), K)
        shifted = np.where(ip >= 0, ip + off, -1)
        assert np.array_equal(idx[0, s0:e0], shifted[0])
        ogs, lgs = ref.sparse_gather(qs, ks, sink, Dv, 0.3, ip, block_size=bs)
        assert np.allclose(og[0, s0:e0], ogs[0], atol=TOL)
        oss, lss = ref.swa(qs, ks, sink, Dv, 0.3, W, block_size=bs)
        assert np.allclose(osw[0, s0:e0], oss[0], atol=TOL)
        assert np.allclose(lsw[0, s0:e0], lss[0], atol=TOL)
        off += nb
    assert off == bl.shape[-1]


# ---------------------------------------------------------------------------
# P9: brute-force top-k over all subsets, with forced ties.
# ---------------------------------------------------------------------------
def _brute_topk(row, own, K):
    C = [j for j in range(len(row)) if row[j] > -np.inf]
    if len(C) <= K:
        return sorted(C)
    winners = []
    for S in itertools.combinations(C, K):
        if own in C and own not in S:
            continue
        ok = True
        for a in S:
            if a == own:
                continue
            for b in C:
                if b in S:
                    continue
                if not (row[a] > row[b] or (row[a] == row[b] and a < b)):
                    ok = False
        if ok:
            winners.append(sorted(S))
    assert len(winners) == 1, winners
    return winners[0]


def test_topk_brute_force():
    rng = np.random.default_rng(9)
    for trial in range(400):
        NB = int(rng.integers(1, 11))
        K = int(rng.integers(1, 7))
        vals = rng.choice([0.0, 0.5, 1.0, 1.5, -np.inf], size=NB, p=[.25, .25, .2, .15, .15])
        if trial % 3 == 0:
            vals = rng.standard_normal(NB)
        own = int(rng.integers(0, NB))
        if vals[own] == -np.inf:
            vals[own] = rng.standard_normal()
        got = ref.topk_blocks(vals[None], np.array([own]), K)[0]
        exp = _brute_topk(vals, own, K)
        want = np.full(K, -1)
        want[:len(exp)] = exp
        assert np.array_equal(got, want), (vals, own, K, got, want)


def test_topk_ties_from_duplicated_key_blocks():
    # Duplicate key blocks give bit-identical block scores; ties go to the lower index.
    S, bs = 128, 16
    q, kv, _ = _rand(10, 1, S, 2, 8)
    kv[0, 32:48] = kv[0, 0:16]
    kv[0, 64:80] = kv[0, 0:16]
    _, _, bl = ref.block_score(q, kv, None, 4, 0.3, block_size=bs)
    assert np.array_equal(bl[0, 100, 0], bl[0, 100, 2]) and bl[0, 100, 0] == bl[0, 100, 4]
    own = ref.own_blocks(1, S, S, bs)
    idx = ref.topk_blocks(bl, own, 3)
    for t in range(80, S):
        exp = _brute_topk(bl[0, t], own[0, t], 3)
        assert idx[0, t].tolist() == exp


# ---------------------------------------------------------------------------
# P10: merging attention over disjoint key sets.
# ---------------------------------------------------------------------------
def test_merge_identity():
    q, kv, _ = _rand(11, 1, 1, 3, 8, Skv=50)
    keys = np.random.default_rng(1).permutation(50)
    parts = [keys[:7], keys[7:30], keys[30:]]
    res = [ref.attend_subset(q[0, 0], kv[0], 4, 0.5, p) for p in parts]
    o, l = ref.merge_partials([r[0] for r in res], [r[1] for r in res])
    oa, la = ref.attend_subset(q[0, 0], kv[0], 4, 0.5, keys)
    assert np.allclose(o, oa, atol=TOL) and np.allclose(l, la, atol=TOL)


# ---------------------------------------------------------------------------
# P11: corner cases of the tiny fp32 workload's shapes.
# ---------------------------------------------------------------------------
def test_tiny_workload_corners():
    q, kv, sink = _rand(12, 1, 130, 8, 96)
    scale = 1 / math.sqrt(96)
    o, l, bl = ref.block_score(q, kv, sink, 64, scale, block_size=64)
    s00 = scale * q[0, 0] @ kv[0, 0]                     # [H]
    w = 1.0 / (1.0 + np.exp(sink - s00))
    assert np.allclose(o[0, 0], kv[0, 0, :64][None] * w[:, None], atol=TOL)
    assert abs(bl[0, 0, 0] - s00.max()) < TOL
    fin = np.isfinite(bl[0])
    assert np.all(fin[:64].sum(axis=1) == 1)
    assert np.all(fin[64:128].sum(axis=1) == 2) and np.all(fin[128:].sum(axis=1) == 3)
    assert bl.shape[-1] == 3                                # ragged tail is a real block


# ---------------------------------------------------------------------------
# P12: invariances.
# ---------------------------------------------------------------------------
def test_head_permutation_and_scale_invariance():
    q, kv, sink = _rand(13, 1, 40, 5, 8)
    perm = np.array([3, 0, 4, 1, 2])
    o, l, bl = ref.block_score(q, kv, sink, 4, 0.3, block_size=16)
    op, lp, blp = ref.block_score(q[:, :, perm], kv, sink[perm], 4, 0.3, block_size=16)
    assert np.allclose(op, o[:, :, perm], atol=TOL) and np.allclose(lp, l[:, :, perm], atol=TOL)
    assert np.allclose(blp, bl, atol=TOL)
    o2, l2, b2 = ref.block_score(q * 2.0, kv, sink, 4, 0.15, block_size=16)
    assert np.allclose(o2, o, atol=TOL) and np.allclose(l2, l, atol=TOL)
    assert np.allclose(b2, bl, atol=TOL)


def test_block_table_documents():
    bt = ref.block_table(200, 64, [0, 70, 71, 134], [70, 71, 134, 200])
    assert bt.start.tolist() == [0, 64, 70, 71, 134, 198]
    assert bt.end.tolist() == [64, 70, 71, 134, 198, 200]
    assert ref.num_blocks(1, 200, 64, None, [0, 70, 71, 134], [70, 71, 134, 200]) == 6
    assert ref.num_blocks(3, 300, 64, [1, 300, 129]) == 5


def test_block_prob_one_head_is_key_mass():
    """One head: exp(block_logit - lse) summed over the blocks is the
    attention's mass on keys, 1 - exp(sink - lse) (all of it without a sink)."""
    q, kv, sink = _rand(61, 2, 150, 1, 12)
    scale = 0.3
    for sk in (sink, None):
        _, lse, bl = ref.block_score(q, kv, sk, 8, scale)
        p = ref.block_prob(bl, lse)
        mass = p.sum(axis=-1)
        want = np.ones_like(mass) if sk is None else 1.0 - np.exp(sk[0] - lse[..., 0])
        assert np.abs(mass - want).max() < 1e-12
        assert (p >= 0).all() and (p <= 1 + 1e-15).all()


def test_block_prob_many_heads_brute_force():
    """Several heads: block_prob[j] is exp(max_h LSE_h(j) - max_h lse_h), with
    the per-head block log-sum-exp and lse recomputed here key by key from
    q . k (no oracle routine), and -inf blocks give 0."""
    B, S, H, Dk, bs = 1, 70, 3, 5, 16
    q, kv, sink = _rand(62, B, S, H, Dk)
    scale = 0.7
    _, lse, bl = ref.block_score(q, kv, sink, 4, scale, block_size=bs)
    p = ref.block_prob(bl, lse)
    for r in (0, 15, 16, 40, 69):
        s = scale * np.einsum("hd,id->hi", q[0, r], kv[0, :r + 1])          # [H, r+1]
        lse_h = [math.log(math.exp(sink[h]) + sum(math.exp(x) for x in s[h])) for h in range(H)]
        for j in range((S + bs - 1) // bs):
            keys = range(j * bs, min((j + 1) * bs, r + 1))
            if len(keys) == 0:
                assert p[0, r, j] == 0.0
                continue
            blk = max(math.log(sum(math.exp(s[h, i]) for i in keys)) for h in range(H))
            assert abs(p[0, r, j] - math.exp(blk - max(lse_h))) < 1e-12


def test_gated_combine_selects_and_is_linear():
    """Gates (1, 0) and (0, 1) give back each branch; the sum is linear in the
    gates and in each branch (checked against hand-written per-element sums
    on a tiny case)."""
    rng = np.random.default_rng(63)
    a = rng.standard_normal((2, 3, 4, 5))
    b = rng.standard_normal((2, 3, 4, 5))
    one, zero = np.ones((2, 3, 4)), np.zeros((2, 3, 4))
    assert np.array_equal(ref.gated_combine(a, b, one, zero), a)
    assert np.array_equal(ref.gated_combine(a, b, zero, one), b)
    g1 = rng.uniform(size=(2, 3, 4))
    g2 = rng.uniform(size=(2, 3, 4))
    m = ref.gated_combine(a, b, g1, g2)
    for idx in [(0, 0, 0, 0), (1, 2, 3, 4), (0, 1, 2, 3)]:
        want = g1[idx[:3]] * a[idx] + g2[idx[:3]] * b[idx]
        assert abs(m[idx] - want) < 1e-15
    # one branch's full output with equal gates of 1/2 each is its mean
    assert np.allclose(ref.gated_combine(a, a, one / 2, one / 2), a, atol=0, rtol=1e-15)
