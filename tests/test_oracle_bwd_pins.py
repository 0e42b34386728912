"""Pins of the float64 oracle's gradients against facts outside its formula.

The gradient functions are checked against central finite differences of the
forward oracle (itself pinned in test_oracle_pins.py): in random directions
on every operation and mask kind, and entry by entry on a tiny problem. The
dense case is also checked against torch's autograd through its own
scaled_dot_product_attention, and a one-key case against its closed form.
None of these re-types the gradient formula.
"""
import math

import numpy as np
import pytest
import torch

from oracle import hysparse_ref as ref

EPS = 1e-5


def _loss(kind, q, kv, sink, dout, Dv, scale, bs, kw):
    if kind == "score":
        out, _, _ = ref.block_score(q, kv, sink, Dv, scale, block_size=bs, **kw)
    elif kind == "swa":
        out, _ = ref.swa(q, kv, sink, Dv, scale, kw.pop("window"), block_size=bs, **kw)
    else:
        out, _ = ref.sparse_gather(q, kv, sink, Dv, scale, kw.pop("block_idx"), block_size=bs,
                                   **kw)
    return float((out * dout).sum())


def _grads(kind, q, kv, sink, dout, Dv, scale, bs, kw):
    kw = dict(kw)
    if kind == "score":
        return ref.block_score_bwd(q, kv, sink, Dv, scale, dout, block_size=bs, **kw)
    if kind == "swa":
        return ref.swa_bwd(q, kv, sink, Dv, scale, kw.pop("window"), dout, block_size=bs, **kw)
    return ref.sparse_gather_bwd(q, kv, sink, Dv, scale, kw.pop("block_idx"), dout,
                                 block_size=bs, **kw)


def _problem(seed, B, Sq, Skv, H, Dk, Dv, with_sink):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, H, Dk))
    kv = rng.standard_normal((B, Skv, Dk)) * 0.7
    sink = rng.standard_normal(H) if with_sink else None
    dout = rng.standard_normal((B, Sq, H, Dv))
    return rng, q, kv, sink, dout


CASES = {
    # name: (kind, B, Sq, Skv, H, Dk, Dv, bs, sink, extra)
    "score_plain": ("score", 1, 23, 23, 3, 8, 6, 4, True, {}),
    "score_nosink_docs": ("score", 1, 30, 30, 2, 6, 6, 4, False,
                          {"doc_start": [0, 7, 8, 19], "doc_end": [7, 8, 19, 30]}),
    "score_kvlens": ("score", 2, 5, 17, 2, 7, 3, 4, True, {"kv_lens": [17, 9]}),
    "swa_docs": ("swa", 1, 26, 26, 3, 5, 4, 4, True,
                 {"window": 6, "doc_start": [0, 11], "doc_end": [11, 26]}),
    "swa_window1_kvlens": ("swa", 2, 4, 12, 2, 6, 6, 4, False,
                           {"window": 1, "kv_lens": [12, 6]}),
    "gather_mixed": ("gather", 1, 29, 29, 2, 6, 5, 4, True, {"block_idx": "rand"}),
    "gather_docs_nosink": ("gather", 1, 24, 24, 3, 4, 4, 4, False,
                           {"block_idx": "rand", "doc_start": [0, 10], "doc_end": [10, 24]}),
}


def _materialise(name, rng, B, Sq, Skv, bs, extra):
    kw = dict(extra)
    if kw.get("block_idx") == "rand":
        NB = ref.num_blocks(B, Skv, bs, kw.get("kv_lens"), kw.get("doc_start"), kw.get("doc_end"))
        K = 3
        idx = rng.integers(-1, NB + 2, size=(B, Sq, K))    # includes skipped entries
        for b in range(B):
            for r in range(Sq):
                row = list(dict.fromkeys(int(x) for x in idx[b, r]))
                row += [-1] * (K - len(row))
                idx[b, r] = row                            # distinct entries per row
        kw["block_idx"] = idx
    return kw


@pytest.mark.parametrize("name", list(CASES))
def test_gradients_match_directional_finite_differences(name):
    kind, B, Sq, Skv, H, Dk, Dv, bs, with_sink, extra = CASES[name]
    rng, q, kv, sink, dout = _problem(100 + list(CASES).index(name), B, Sq, Skv, H, Dk, Dv, with_sink)
    kw = _materialise(name, rng, B, Sq, Skv, bs, extra)
    scale = 0.41
    dq, dkv, dsink = _grads(kind, q, kv, sink, dout, Dv, scale, bs, kw)
    assert dq.shape == q.shape and dkv.shape == kv.shape
    assert (dsink is None) == (sink is None)
    f = lambda q_, kv_, s_: _loss(kind, q_, kv_, s_, dout, Dv, scale, bs, dict(kw))
    for trial in range(3):
        uq = rng.standard_normal(q.shape)
        ukv = rng.standard_normal(kv.shape)
        fd = (f(q + EPS * uq, kv, sink) - f(q - EPS * uq, kv, sink)) / (2 * EPS)
        assert math.isclose(fd, float((dq * uq).sum()), rel_tol=1e-6, abs_tol=1e-8), (trial, "q")
        fd = (f(q, kv + EPS * ukv, sink) - f(q, kv - EPS * ukv, sink)) / (2 * EPS)
        assert math.isclose(fd, float((dkv * ukv).sum()), rel_tol=1e-6, abs_tol=1e-8), (trial, "kv")
    if sink is not None:
        for h in range(H):
            e = np.zeros(H)
            e[h] = EPS
            fd = (f(q, kv, sink + e) - f(q, kv, sink - e)) / (2 * EPS)
            assert math.isclose(fd, dsink[h], rel_tol=1e-6, abs_tol=1e-9), h
    # rows of kv past an entry's valid length receive nothing
    if "kv_lens" in kw:
        for b, L in enumerate(kw["kv_lens"]):
            assert not np.any(dkv[b, L:])


@pytest.mark.parametrize("kind", ["score", "swa", "gather"])
def test_gradients_entrywise_tiny(kind):
    """Every entry of dq, dkv and dsink against a central difference."""
    rng, q, kv, sink, dout = _problem(11, 1, 6, 6, 2, 3, 2, True)
    bs, scale = 2, 0.9
    kw = {"swa": {"window": 2}, "score": {}, "gather": {}}[kind]
    if kind == "gather":
        kw["block_idx"] = np.array([[[0, -1], [0, -1], [1, 0], [0, 1], [2, -1], [2, 0]]])
    dq, dkv, dsink = _grads(kind, q, kv, sink, dout, 2, scale, bs, kw)
    f = lambda q_, kv_, s_: _loss(kind, q_, kv_, s_, dout, 2, scale, bs, dict(kw))
    for arr, grad, which in ((q, dq, 0), (kv, dkv, 1), (sink, dsink, 2)):
        for ix in np.ndindex(arr.shape):
            e = np.zeros(arr.shape)
            e[ix] = EPS
            args_p = [q, kv, sink]
            args_m = [q, kv, sink]
            args_p[which] = arr + e
            args_m[which] = arr - e
            fd = (f(*args_p) - f(*args_m)) / (2 * EPS)
            assert math.isclose(fd, grad[ix], rel_tol=1e-6, abs_tol=1e-9), (which, ix)


def test_dense_case_matches_torch_autograd():
    """Full-coverage causal attention without a sink is dense causal MQA:
    its gradients equal torch's autograd through scaled_dot_product_attention
    (float64, the one KV head expanded over the query heads; key and value
    both read the latent rows, so their gradients add)."""
    rng, q, kv, _, dout = _problem(5, 1, 41, 41, 3, 10, 7, False)
    scale = 0.33
    qt = torch.from_numpy(q).permute(0, 2, 1, 3).clone().requires_grad_(True)
    kvt = torch.from_numpy(kv).clone().requires_grad_(True)
    H = qt.shape[1]
    k = kvt[:, None].expand(-1, H, -1, -1)
    v = kvt[:, None, :, :7].expand(-1, H, -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True, scale=scale)
    (out * torch.from_numpy(dout).permute(0, 2, 1, 3)).sum().backward()
    dq, dkv, dsink = ref.block_score_bwd(q, kv, None, 7, scale, dout, block_size=8)
    assert dsink is None
    assert np.allclose(dq, qt.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11)
    assert np.allclose(dkv, kvt.grad.numpy(), atol=1e-11)
    # the window covering everything and the gather of every block are the same attention
    dq2, dkv2, _ = ref.swa_bwd(q, kv, None, 7, scale, 41, dout, block_size=8)
    idx = np.tile(np.arange(6), (1, 41, 1))
    dq3, dkv3, _ = ref.sparse_gather_bwd(q, kv, None, 7, scale, idx, dout, block_size=8)
    for a, b in ((dq2, dq), (dkv2, dkv), (dq3, dq), (dkv3, dkv)):
        assert np.allclose(a, b, atol=1e-12)


def test_single_key_closed_form():
    """A row that sees one key and no sink has out = v: the score gradient is
    zero, so dq = 0 and the key row receives dout summed over heads in its
    value columns only."""
    rng, q, kv, _, dout = _problem(8, 1, 1, 1, 4, 6, 4, False)
    dq, dkv, _ = ref.block_score_bwd(q, kv, None, 4, 0.5, dout)
    assert np.allclose(dq, 0, atol=1e-15)
    assert np.allclose(dkv[0, 0, :4], dout[0, 0].sum(axis=0), atol=1e-14)
    assert np.allclose(dkv[0, 0, 4:], 0, atol=1e-15)
    # with a sink sigma: out = a v with a = e^s / (e^s + e^sigma); by hand,
    # dL/dsigma = -a (1 - a) (dout . v) summed over heads' own terms
    sink = rng.standard_normal(4)
    dq, dkv, dsink = ref.block_score_bwd(q, kv, sink, 4, 0.5, dout)
    s = 0.5 * q[0, 0] @ kv[0, 0]
    a = 1.0 / (1.0 + np.exp(sink - s))
    gv = dout[0, 0] @ kv[0, 0, :4]
    assert np.allclose(dsink, -a * (1 - a) * gv, atol=1e-14)
    assert np.allclose(dq[0, 0], (0.5 * a * (1 - a) * gv)[:, None] * kv[0, 0][None, :], atol=1e-14)


def test_empty_selection_gives_zero_gradients():
    """A gather row whose list is empty (or only skipped entries) has no keys:
    with no sink its output is zero and nothing flows back; with a sink the
    output is zero for any sigma, so the sink gradient is zero too."""
    rng, q, kv, sink, dout = _problem(9, 1, 9, 9, 2, 4, 4, True)
    idx = np.full((1, 9, 2), -1)
    idx[0, 4] = [1, 7]                                   # row 4: block 1 and an out-of-range id
    dq, dkv, dsink = ref.sparse_gather_bwd(q, kv, sink, 4, 0.5, idx, dout, block_size=4)
    rows = [r for r in range(9) if r != 4]
    assert not np.any(dq[0, rows])
    assert not np.any(dkv[0, :4]) and not np.any(dkv[0, 5:])
    assert np.any(dkv[0, 4:5])


def test_row_subset_matches_full_run():
    """Restricting the gradient to a set of rows gives those rows' dq exactly,
    and dkv / dsink summed over a partition of the rows equal the full run."""
    rng, q, kv, sink, dout = _problem(21, 1, 37, 37, 2, 5, 4, True)
    full = ref.swa_bwd(q, kv, sink, 4, 0.6, 9, dout, block_size=4)
    a = np.arange(0, 37, 3)
    b = np.setdiff1d(np.arange(37), a)
    pa = ref.swa_bwd(q, kv, sink, 4, 0.6, 9, dout[:, a], block_size=4, rows=a)
    pb = ref.swa_bwd(q, kv, sink, 4, 0.6, 9, dout[:, b], block_size=4, rows=b)
    assert np.allclose(pa[0], full[0][:, a], atol=1e-14)
    assert np.allclose(pb[0], full[0][:, b], atol=1e-14)
    assert np.allclose(pa[1] + pb[1], full[1], atol=1e-12)
    assert np.allclose(pa[2] + pb[2], full[2], atol=1e-12)


def _loss_with_lse(kind, q, kv, sink, dout, dlse, Dv, scale, bs, kw):
    kw = dict(kw)
    if kind == "score":
        out, lse, _ = ref.block_score(q, kv, sink, Dv, scale, block_size=bs, **kw)
    elif kind == "swa":
        out, lse = ref.swa(q, kv, sink, Dv, scale, kw.pop("window"), block_size=bs, **kw)
    else:
        out, lse = ref.sparse_gather(q, kv, sink, Dv, scale, kw.pop("block_idx"), block_size=bs,
                                     **kw)
    fin = np.isfinite(lse)
    return float((out * dout).sum() + (np.where(fin, lse, 0.0) * dlse).sum())


@pytest.mark.parametrize("name", list(CASES))
def test_lse_gradient_matches_finite_differences(name):
    """A loss that also weights lse (as a combination of branches by their
    log-sum-exp would): the gradients with dlse match central differences of
    L = sum(dout * out) + sum(dlse * lse) in random directions, for q, kv and
    the sink."""
    kind, B, Sq, Skv, H, Dk, Dv, bs, with_sink, extra = CASES[name]
    rng, q, kv, sink, dout = _problem(300 + list(CASES).index(name), B, Sq, Skv, H, Dk, Dv,
                                      with_sink)
    kw = _materialise(name, rng, B, Sq, Skv, bs, extra)
    dlse = rng.standard_normal((B, Sq, H))
    scale = 0.37
    kw2 = dict(kw)
    if kind == "score":
        dq, dkv, dsink = ref.block_score_bwd(q, kv, sink, Dv, scale, dout, block_size=bs,
                                             dlse=dlse, **kw2)
    elif kind == "swa":
        dq, dkv, dsink = ref.swa_bwd(q, kv, sink, Dv, scale, kw2.pop("window"), dout,
                                     block_size=bs, dlse=dlse, **kw2)
    else:
        dq, dkv, dsink = ref.sparse_gather_bwd(q, kv, sink, Dv, scale, kw2.pop("block_idx"), dout,
                                               block_size=bs, dlse=dlse, **kw2)
    f = lambda q_, kv_, s_: _loss_with_lse(kind, q_, kv_, s_, dout, dlse, Dv, scale, bs, kw)
    for trial in range(2):
        uq = rng.standard_normal(q.shape)
        ukv = rng.standard_normal(kv.shape)
        fd = (f(q + EPS * uq, kv, sink) - f(q - EPS * uq, kv, sink)) / (2 * EPS)
        assert math.isclose(fd, float((dq * uq).sum()), rel_tol=1e-6, abs_tol=1e-8), (trial, "q")
        fd = (f(q, kv + EPS * ukv, sink) - f(q, kv - EPS * ukv, sink)) / (2 * EPS)
        assert math.isclose(fd, float((dkv * ukv).sum()), rel_tol=1e-6, abs_tol=1e-8), (trial, "kv")
    if sink is not None:
        for h in range(H):
            e = np.zeros(H)
            e[h] = EPS
            fd = (f(q, kv, sink + e) - f(q, kv, sink - e)) / (2 * EPS)
            assert math.isclose(fd, dsink[h], rel_tol=1e-6, abs_tol=1e-9), h
