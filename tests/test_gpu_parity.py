"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Small and medium problems are compared element by element; the long-context
problem is launched at full size (the benchmark's launch configuration) and
compared on sampled rows. The gather is always checked on the indices the GPU
itself selected, so its parity does not depend on near-tie choices."""
import numpy as np
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs
from oracle import hysparse_ref as ref

from gpu_common import (BLOCK_LOGIT_TOL, Dev, assert_close, check_topk_margin, np64, sample_rows,
                        say, tol_for)

pytestmark = pytest.mark.gpu

MLA = dict(H=64, Dk=576, Dv=512)


def _small(name, **kw):
    B = kw.pop("B", 1)
    S = kw.pop("S")
    Skv = kw.pop("Skv", S)
    Sq = kw.pop("Sq", S)
    docs = kw.pop("docs", None)
    return inputs.make(B, Sq, Skv, MLA["H"], MLA["Dk"], MLA["Dv"], name=name, doc_lens=docs, **kw)


SMALL_CASES = {
    "S130_tail": lambda: _small("S130_tail", S=130, seed=11, top_k=2, window=70),
    "S64": lambda: _small("S64", S=64, seed=12, top_k=1, window=1),
    "S1": lambda: _small("S1", S=1, seed=13, top_k=1, window=5),
    "S300_docs": lambda: _small("S300_docs", S=300, seed=14, top_k=2, window=40,
                                docs=[70, 1, 63, 100, 66]),
    "chunked_prefill": lambda: _small("chunked_prefill", B=2, S=0, Sq=70, Skv=200, seed=15,
                                      kv_lens=[200, 150], top_k=3, window=100),
    "decode_small": lambda: _small("decode_small", B=3, S=0, Sq=1, Skv=700, seed=16,
                                   kv_lens=[700, 64, 1], top_k=4, window=129),
    "no_sink": lambda: _small("no_sink", S=190, seed=17, top_k=2, window=64, sink=False),
    "tiny_f32": lambda: inputs.config(1),
}


def _run_all(d: Dev, rows=None):
    """Run the four calls; return GPU results and oracle results on `rows`."""
    p = d.p
    tol = tol_for(p)
    torch.cuda.synchronize()
    out, lse, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    og, lg = hs.sparse_gather(d.prob, d.q, d.kv, d.sink, idx, p.top_k)
    osw, lsw = hs.swa(d.prob, d.q, d.kv, d.sink, p.window)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    res = {}
    o_ref, l_ref, b_ref = ref.block_score(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, rows=rows, **d.kw())
    res["score_out"] = assert_close(np64(out)[:, sel], o_ref, tol, "block_score out")
    res["score_lse"] = assert_close(np64(lse)[:, sel], l_ref, tol, "block_score lse")
    res["block_logit"] = assert_close(np64(bl)[:, sel], b_ref,
                                      BLOCK_LOGIT_TOL if p.dtype == "bf16" else 1e-4, "block_logit")
    # top-k: exact on the GPU's own block scores (identical fp32 inputs) ...
    idx_np = idx.cpu().numpy()
    bl_np = bl.cpu().numpy()
    own = d.own(rows)
    want = ref.topk_blocks(bl_np[:, sel], own, p.top_k)
    assert np.array_equal(idx_np[:, sel], want), "top-k differs on identical inputs"
    # ... and within the margin rule against the oracle's own scores.
    res["exact_rows"] = check_topk_margin(idx_np[:, sel], b_ref, own, p.top_k)
    og_ref, lg_ref = ref.sparse_gather(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, idx_np, rows=rows,
                                       **d.kw())
    res["gather_out"] = assert_close(np64(og)[:, sel], og_ref, tol, "gather out")
    res["gather_lse"] = assert_close(np64(lg)[:, sel], lg_ref, tol, "gather lse")
    os_ref, ls_ref = ref.swa(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, p.window, rows=rows, **d.kw())
    res["swa_out"] = assert_close(np64(osw)[:, sel], os_ref, tol, "swa out")
    res["swa_lse"] = assert_close(np64(lsw)[:, sel], ls_ref, tol, "swa lse")
    return res


@pytest.mark.parametrize("case", list(SMALL_CASES))
def test_small_cases(case):
    say(f"[gpu] small case {case}")
    p = SMALL_CASES[case]()
    res = _run_all(Dev(p, sink=p.sink is not None))
    say(f"[gpu] {case}: {res}")


def test_config2_full():
    say("[gpu] S=4096 H=64 Dk=576 full comparison")
    p = inputs.config(2)
    res = _run_all(Dev(p))
    say(f"[gpu] S=4096: {res}")


def test_tail_tile_S4097_sampled():
    """S = 4097 (a one-row tail block after 64 full blocks) in the launch that
    does not split the key range, at the absorbed-MLA shape: sampled rows,
    including the tail row and the rows around every block edge."""
    say("[gpu] S=4097 one-row tail block, sampled rows")
    p = inputs.make(1, 4097, 4097, MLA["H"], MLA["Dk"], MLA["Dv"], seed=18, top_k=16,
                    window=512, name="S4097_tail")
    rows = sample_rows(p, 200, seed=18)
    assert rows[-1] == 4096
    res = _run_all(Dev(p), rows=rows)
    say(f"[gpu] S=4097: {res}")


def test_config4_packed_documents_sampled():
    say("[gpu] packed 8-document S=16384, sampled rows")
    p = inputs.config(4)
    rows = sample_rows(p, 160, seed=4)
    res = _run_all(Dev(p), rows=rows)
    say(f"[gpu] packed docs: {res}")


def test_config5_decode_full():
    say("[gpu] decode B=32, caches 16k-64k, split key range")
    p = inputs.config(5)
    res = _run_all(Dev(p))
    say(f"[gpu] decode: {res}")


def test_config3_long_context_sampled():
    say("[gpu] S=32768 full-size launch, sampled rows")
    p = inputs.config(3)
    rows = sample_rows(p, 96, seed=3)
    res = _run_all(Dev(p), rows=rows)
    say(f"[gpu] S=32768: {res}")


def test_topk_exact_synthetic():
    """Top-k alone on crafted fp32 scores: forced ties, -inf rows, fewer
    candidates than k, own block not the best, and 1024 columns."""
    say("[gpu] top-k synthetic")
    rng = np.random.default_rng(21)
    B, Skv = 4, 65536
    lens = [65536, 1000, 64, 40000]
    prob = hs.Problem(B, 1, Skv, 64, 576, 512, kv_lens=lens)
    NB = hs.hs_num_blocks(prob)
    assert NB == 1024
    bl = rng.choice([0.0, 0.25, -1.5, 2.0], size=(B, 1, NB)).astype(np.float32)
    bl[1, 0, :] = rng.standard_normal(NB).astype(np.float32)
    for b, L in enumerate(lens):
        bl[b, 0, (L + 63) // 64:] = -np.inf
    bl[3, 0, ::3] = -np.inf
    bl[3, 0, (40000 - 1) // 64] = -7.0          # own block far below the rest
    for K in (1, 4, 32, 64):
        idx = hs.topk_blocks(prob, torch.from_numpy(bl).cuda(), K)
        torch.cuda.synchronize()
        own = ref.own_blocks(B, 1, Skv, 64, lens)
        want = ref.topk_blocks(bl, own, K)
        assert np.array_equal(idx.cpu().numpy(), want), K


def test_topk_exact_adversarial():
    """Top-k on scores built to stress the radix select: neighbours one ulp
    apart (keys that differ only in their lowest bits), +0 and -0 mixed with
    denormals, negative and positive values (the sign bit differs, so every
    digit is searched), long runs of equal values at the cut, one value
    everywhere, and 4096 columns with k = 64. The selection must equal the
    oracle's on the same fp32 scores."""
    say("[gpu] top-k adversarial")
    rng = np.random.default_rng(23)
    B, Skv = 6, 4096 * 64
    prob = hs.Problem(B, 1, Skv, 64, 576, 512)
    NB = hs.hs_num_blocks(prob)
    assert NB == 4096
    one = np.float32(1.0)
    steps = rng.integers(0, 3000, size=NB)
    bl = np.empty((B, 1, NB), np.float32)
    bl[0, 0] = (one + steps.astype(np.float32) * np.finfo(np.float32).eps).astype(np.float32)
    tiny = np.finfo(np.float32).smallest_subnormal
    bl[1, 0] = rng.choice(np.array([0.0, -0.0, tiny, -tiny, 2 * tiny], np.float32), size=NB)
    bl[2, 0] = rng.standard_normal(NB).astype(np.float32) * np.float32(1e3)
    bl[3, 0] = np.where(rng.random(NB) < 0.5, np.float32(3.0), np.float32(-3.0))
    bl[3, 0, rng.choice(NB, 40, replace=False)] = np.float32(5.0)   # 40 above a long tie run
    bl[4, 0] = np.float32(0.75)
    bl[5, 0] = rng.standard_normal(NB).astype(np.float32)
    bl[5, 0, rng.random(NB) < 0.7] = -np.inf
    own = ref.own_blocks(B, 1, Skv, 64, None)
    for K in (1, 2, 33, 64):
        idx = hs.topk_blocks(prob, torch.from_numpy(bl).cuda(), K)
        torch.cuda.synchronize()
        want = ref.topk_blocks(bl, own, K)
        got = idx.cpu().numpy()
        for b in range(B):
            assert np.array_equal(got[b], want[b]), (K, b, got[b], want[b])
    say("[gpu] top-k adversarial: exact")
