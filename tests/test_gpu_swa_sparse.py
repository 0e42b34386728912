"""GPU checks of hs_swa_sparse_fwd, both branches of a sliding-window layer
over the shared latent KV and a full layer's block selection in one call.
Its outputs must equal, bit for bit, those of hs_swa_fwd and
hs_sparse_gather_fwd for the same arguments (the one-pass kernel runs the
same per-tile arithmetic in the same order; decode and fp32 shapes run the
two operations), and on one case match the float64 oracle directly."""
import numpy as np
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs
from oracle import hysparse_ref as ref

from gpu_common import BF16_TOL, Dev, assert_close, np64, say
from test_gpu_parity import MLA

pytestmark = pytest.mark.gpu


def _mla(name, S, seed, top_k, window, B=1, Sq=None, Skv=None, kv_lens=None, docs=None):
    return inputs.make(B, Sq or S, Skv or S, MLA["H"], MLA["Dk"], MLA["Dv"], seed=seed,
                       top_k=top_k, window=window, kv_lens=kv_lens, doc_lens=docs, name=name)


CASES = {
    "S130_tail": lambda: _mla("S130_tail", 130, 71, 2, 70),
    "S300_docs": lambda: _mla("S300_docs", 300, 72, 3, 40, docs=[70, 1, 63, 100, 66]),
    "chunked_prefill": lambda: _mla("chunked_prefill", 0, 73, 3, 100, B=2, Sq=70, Skv=200,
                                    kv_lens=[200, 150]),
    "S2048_window_past_start": lambda: _mla("S2048", 2048, 74, 8, 5000),
    "decode_split": lambda: _mla("decode", 0, 75, 4, 256, B=3, Sq=1, Skv=3000,
                                 kv_lens=[3000, 1200, 64]),
    "tiny_f32": lambda: inputs.config(1),
}


def _both(d, p, idx):
    ow, lw, og, lg = hs.swa_sparse(d.prob, d.q, d.kv, d.sink, p.window, idx, p.top_k)
    sw = hs.swa(d.prob, d.q, d.kv, d.sink, p.window)
    sg = hs.sparse_gather(d.prob, d.q, d.kv, d.sink, idx, p.top_k)
    torch.cuda.synchronize()
    return (ow, lw, og, lg), (*sw, *sg)


def _equal(got, want, name):
    for g, w, n in zip(got, want, ("out_swa", "lse_swa", "out_sparse", "lse_sparse")):
        assert torch.equal(g, w), f"{name}: {n} differs from the separate call"


@pytest.mark.parametrize("name", list(CASES))
def test_equals_separate_calls(name):
    p = CASES[name]()
    say(f"[gpu] swa+sparse {name}: B={p.B} Sq={p.Sq} Skv={p.Skv} dtype={p.dtype} "
        f"top_k={p.top_k} window={p.window}")
    d = Dev(p)
    _, _, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    got, want = _both(d, p, idx)
    _equal(got, want, name)
    say(f"[gpu] swa+sparse {name}: identical to the separate calls")


def test_rows_with_empty_sparse_branch():
    """Rows whose selection holds no valid block (all -1, or ids past the
    block count) get the sink-only sparse result, as from the gather call and
    the oracle. Ids are distinct within each row (the gather's precondition)."""
    p = _mla("empty_sparse", 200, 76, 3, 64)
    d = Dev(p)
    rng = np.random.default_rng(77)
    nb = hs.hs_num_blocks(d.prob)
    assert nb >= p.top_k
    idx = np.stack([rng.permutation(nb)[:p.top_k] for _ in range(p.Sq)])[None].astype(np.int32)
    idx[0, ::3] = -1
    idx[0, 1::7] = nb + np.arange(p.top_k)
    idx_t = torch.from_numpy(idx).cuda()
    got, want = _both(d, p, idx_t)
    _equal(got, want, "empty sparse rows")
    og_ref, lg_ref = ref.sparse_gather(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, idx, **d.kw())
    e = [assert_close(np64(got[2]), og_ref, BF16_TOL, "sparse out"),
         assert_close(np64(got[3]), lg_ref, BF16_TOL, "sparse lse")]
    say(f"[gpu] swa+sparse with empty sparse rows: identical, oracle {max(e):.2e}")


def test_matches_oracle_docs():
    """Against the float64 oracle directly: documents, a ragged tail."""
    p = _mla("oracle_docs", 333, 78, 3, 90, docs=[100, 33, 200])
    d = Dev(p)
    _, _, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    ow, lw, og, lg = hs.swa_sparse(d.prob, d.q, d.kv, d.sink, p.window, idx, p.top_k)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    os_ref, ls_ref = ref.swa(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, p.window, **d.kw())
    og_ref, lg_ref = ref.sparse_gather(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, idx_np, **d.kw())
    errs = [assert_close(np64(ow), os_ref, BF16_TOL, "swa out"),
            assert_close(np64(lw), ls_ref, BF16_TOL, "swa lse"),
            assert_close(np64(og), og_ref, BF16_TOL, "sparse out"),
            assert_close(np64(lg), lg_ref, BF16_TOL, "sparse lse")]
    say(f"[gpu] swa+sparse vs oracle: {max(errs):.2e} worst")


def test_long_context_full_size():
    """S = 32768, top-k 32, window 1024: the one-pass launch the benchmark
    times, identical to the two separate calls."""
    p = inputs.config(3)
    say("[gpu] swa+sparse long context: inputs ready")
    d = Dev(p)
    _, _, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    got, want = _both(d, p, idx)
    _equal(got, want, "long context")
    say("[gpu] swa+sparse long context: identical")


def _gates(p, seed):
    g = torch.Generator().manual_seed(seed)
    shape = (p.B, p.Sq, p.H)
    return torch.rand(shape, generator=g), torch.rand(shape, generator=g)


@pytest.mark.parametrize("name", list(CASES))
def test_gated_combination(name):
    """The optional gated sum out_mix = g_swa * out_swa + g_sparse * out_sparse
    (per token and head): within the rounding bound of an fp32 sum and a bf16
    store of the call's own branch outputs, combined in float64, and within the bf16 tolerance of the oracle's
    gated combination of its own branch outputs; the branch outputs are the
    ones the call returns without gates. One-pass shapes form it in the
    kernel's epilogue, split decode and fp32 in a separate launch."""
    p = CASES[name]()
    say(f"[gpu] gated combination {name}")
    d = Dev(p)
    _, _, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    g1, g2 = _gates(p, 81)
    ow, lw, og, lg, om = hs.swa_sparse(d.prob, d.q, d.kv, d.sink, p.window, idx, p.top_k,
                                       gate_swa=g1.cuda(), gate_sparse=g2.cuda())
    plain = hs.swa_sparse(d.prob, d.q, d.kv, d.sink, p.window, idx, p.top_k)
    torch.cuda.synchronize()
    for n, a, b in zip(("out_swa", "lse_swa", "out_sparse", "lse_sparse"), (ow, lw, og, lg), plain):
        assert torch.equal(a, b), f"{name}: {n} changed by the gates"
    ga, gb = g1.double().numpy()[..., None], g2.double().numpy()[..., None]
    ta, tb = ga * np64(ow), gb * np64(og)
    own = ta + tb
    got = np64(om)
    # fp32 sum fl(gb*b + fl(ga*a)): at most 2^-24 of |ga*a| and of the result
    # each (under 2^-22 of |ga*a| + |gb*b| together, which matters only where
    # the branches cancel), then one rounding to bf16 (at most 2^-8 relative)
    bound = 2.0 ** -22 * (np.abs(ta) + np.abs(tb))
    if p.dtype == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(own) * (1 + 2.0 ** -20)
    e_own = float((np.abs(got - own) / (bound + 1e-30)).max())
    assert e_own <= 1.0, f"{name}: error {e_own} of the rounding bound from its own branches"
    idx_np = idx.cpu().numpy()
    os_ref, _ = ref.swa(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, p.window, **d.kw())
    og_ref, _ = ref.sparse_gather(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, idx_np, **d.kw())
    want = ref.gated_combine(os_ref, og_ref, g1, g2)
    tol = BF16_TOL if p.dtype == "bf16" else 1e-4
    e = assert_close(got, want, 2 * tol, f"{name} out_mix")
    say(f"[gpu] gated combination {name}: {e_own:.2f} of the rounding bound from its branches, "
        f"oracle {e:.2e}")
