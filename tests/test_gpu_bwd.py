"""GPU parity of the gradient calls (hs_block_score_bwd, hs_sparse_gather_bwd,
hs_swa_bwd) through the C ABI against the float64 oracle.

The GPU backward consumes the GPU forward's own out and lse, as a training
step would; the oracle recomputes everything from the inputs. The gather is
differentiated for the selection the GPU's top-k made (and, in one case, for
a list with skipped entries).

Tolerance. The bf16 path feeds P and dS to the MFMA as bf16 (relative
rounding 2^-9) and uses the bf16 forward output in dout . out; errors add up
over the keys, rows and heads of each sum. Gradients are compared as the
largest absolute error divided by the largest magnitude of that gradient
(BF16 3e-2, fp32 2e-4, where only fp32 rounding enters), and the relative
Frobenius error must also stay under BF16 1e-2 / fp32 2e-5."""
import numpy as np
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs
from oracle import hysparse_ref as ref

from gpu_common import Dev, np64, say
from test_gpu_parity import MLA

pytestmark = pytest.mark.gpu

TOL = {"bf16": (3e-2, 1e-2), "f32": (2e-4, 2e-5)}


def _grad_close(got, want, dtype, name):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite GPU gradient"
    mx, fro = TOL[dtype]
    scale = max(np.abs(want).max(), 1e-30)
    err = np.abs(got - want).max() / scale
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    assert err <= mx, f"{name}: max error {err:.3e} of max |ref| > {mx:.0e}"
    assert rel <= fro, f"{name}: relative Frobenius error {rel:.3e} > {fro:.0e}"
    return float(err)


def _gpu_grads(d, op, dout, idx=None, K=None):
    p = d.p
    if op in ("score", "score_recompute"):
        # "score": the larger workspace (dq from the stored score gradients on
        # bf16 shapes); "score_recompute": the smaller one (dq recomputes them)
        out, lse, _ = hs.block_score(d.prob, d.q, d.kv, d.sink)
        return hs.block_score_bwd(d.prob, d.q, d.kv, d.sink, out, lse, dout,
                                  store_ds=op == "score")
    if op in ("swa", "swa_recompute"):
        out, lse = hs.swa(d.prob, d.q, d.kv, d.sink, p.window)
        return hs.swa_bwd(d.prob, d.q, d.kv, d.sink, p.window, out, lse, dout,
                          store_ds=op == "swa")
    # "gather": the smaller workspace (dq recomputes); "gather_ds": the larger
    # one (bf16: the key-block pass stores dS, dq on row pairs reads it)
    out, lse = hs.sparse_gather(d.prob, d.q, d.kv, d.sink, idx, K)
    return hs.sparse_gather_bwd(d.prob, d.q, d.kv, d.sink, idx, K, out, lse, dout,
                                store_ds=op == "gather_ds")


def _oracle_grads(d, op, dout_cpu, idx=None, rows=None):
    p = d.p
    kw = dict(d.kw(), rows=rows)
    if op in ("score", "score_recompute"):
        return ref.block_score_bwd(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, dout_cpu, **kw)
    if op in ("swa", "swa_recompute"):
        return ref.swa_bwd(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, p.window, dout_cpu, **kw)
    return ref.sparse_gather_bwd(p.q, p.kv, d.sink_cpu, p.Dv, p.scale, idx, dout_cpu, **kw)


def _mla(name, S, seed, top_k, window, B=1, Sq=None, Skv=None, kv_lens=None, docs=None,
         sink=True):
    return inputs.make(B, Sq or S, Skv or S, MLA["H"], MLA["Dk"], MLA["Dv"], seed=seed,
                       top_k=top_k, window=window, kv_lens=kv_lens, doc_lens=docs, sink=sink,
                       name=name)


CASES = {
    "S130_tail": lambda: _mla("S130_tail", 130, 31, 2, 70),
    "S300_docs": lambda: _mla("S300_docs", 300, 32, 2, 40, docs=[70, 1, 63, 100, 66]),
    "chunked_prefill": lambda: _mla("chunked_prefill", 0, 33, 3, 100, B=2, Sq=70, Skv=200,
                                    kv_lens=[200, 150]),
    "no_sink_S190": lambda: _mla("no_sink_S190", 190, 34, 2, 64, sink=False),
    "S1": lambda: _mla("S1", 1, 35, 1, 5),
    "S1024_many_items": lambda: _mla("S1024_many_items", 1024, 36, 4, 256),
    "tiny_f32": lambda: inputs.config(1),
    "f32_kvlens": lambda: inputs.make(2, 40, 300, 8, 96, 64, dtype="f32", seed=37, top_k=3,
                                      window=50, kv_lens=[300, 41], name="f32_kvlens"),
    "f32_docs": lambda: inputs.make(1, 250, 250, 5, 33, 17, dtype="f32", seed=43, top_k=2,
                                    window=30, doc_lens=[100, 2, 148], name="f32_docs"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_gradients_match_oracle(name):
    p = CASES[name]()
    say(f"[gpu] gradients {name}: B={p.B} Sq={p.Sq} Skv={p.Skv} dtype={p.dtype} "
        f"top_k={p.top_k} window={p.window}")
    d = Dev(p, sink=p.sink is not None)
    dout_cpu = inputs.make_dout(p, seed=900 + p.Sq)
    dout = dout_cpu.cuda()
    _, _, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    torch.cuda.synchronize()
    idx_cpu = idx.cpu().numpy()
    res = {}
    for op in ("score", "score_recompute", "swa", "swa_recompute", "gather", "gather_ds"):
        g = _gpu_grads(d, op, dout, idx, p.top_k)
        torch.cuda.synchronize()
        w = _oracle_grads(d, op, dout_cpu, idx_cpu)
        res[op + "_dq"] = _grad_close(np64(g[0]), w[0], p.dtype, f"{op} dq")
        res[op + "_dkv"] = _grad_close(np64(g[1]), w[1], p.dtype, f"{op} dkv")
        if d.sink is not None:
            res[op + "_dsink"] = _grad_close(np64(g[2]), w[2], p.dtype, f"{op} dsink")
        else:
            assert g[2] is None and w[2] is None
    say(f"[gpu] gradients {name}: " + ", ".join(f"{k}={v:.1e}" for k, v in res.items()))


def test_gather_list_with_skipped_entries():
    """Entries that are -1, past the entry's blocks, or blocks beyond the
    row's causal range contribute nothing; a row with no usable entry gets
    zero gradient."""
    p = _mla("gather_skips", 200, 38, 4, 64)
    d = Dev(p)
    rng = np.random.default_rng(39)
    NB = hs.hs_num_blocks(d.prob)
    idx = np.full((1, p.Sq, 4), -1, dtype=np.int32)
    for r in range(p.Sq):
        picks = rng.choice(np.arange(-1, NB + 3), size=4, replace=False)
        idx[0, r] = np.sort(picks)
    idx[0, 5] = [-1, -1, -1, NB + 1]                     # nothing usable
    idx_dev = torch.from_numpy(idx).cuda()
    dout_cpu = inputs.make_dout(p, seed=40)
    w = _oracle_grads(d, "gather", dout_cpu, idx)
    for v in ("gather", "gather_ds"):
        g = _gpu_grads(d, v, dout_cpu.cuda(), idx_dev, 4)
        torch.cuda.synchronize()
        for k, name in enumerate(("dq", "dkv", "dsink")):
            _grad_close(np64(g[k]), w[k], "bf16", f"{v} {name}")
        assert not torch.any(g[0][0, 5]).item()
    say("[gpu] gather with skipped entries: ok")


def test_gradients_are_deterministic():
    """Two calls give identical bits (fixed summation order, no atomics on
    floating-point values)."""
    p = _mla("determinism", 700, 41, 3, 200)
    d = Dev(p)
    dout = inputs.make_dout(p, seed=42).cuda()
    _, _, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    for op in ("score", "score_recompute", "swa", "swa_recompute", "gather", "gather_ds"):
        a = _gpu_grads(d, op, dout, idx, p.top_k)
        b = _gpu_grads(d, op, dout, idx, p.top_k)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), op
    say("[gpu] gradients deterministic")


def test_long_context_sampled():
    """The long-context workload (S = 32768, top_k 32, window 1024) at full
    size, in the launch configuration the benchmark times: dq on sampled rows
    and dkv on the keys of the last block (which only the last 64 rows see, so
    their oracle sum is complete from those rows)."""
    p = inputs.config(3)
    say("[gpu] gradients long context: inputs ready")
    d = Dev(p)
    dout_cpu = inputs.make_dout(p, seed=903)
    dout = dout_cpu.cuda()
    _, _, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    torch.cuda.synchronize()
    S = p.Sq
    last = np.arange(S - 64, S)
    sampled = np.array([0, 1, 63, 64, 65, 1000, 4095, 4096, 20000, S - 65])
    rows = np.concatenate([sampled, last])
    idx_cpu = idx.cpu().numpy()
    # the causal and window calls through both workspaces (stored and
    # recomputed score gradients), against one oracle evaluation each
    for op, variants in (("score", ("score", "score_recompute")), ("swa", ("swa", "swa_recompute")),
                         ("gather", ("gather", "gather_ds"))):
        got = []
        for v in variants:
            g = _gpu_grads(d, v, dout, idx, p.top_k)
            torch.cuda.synchronize()
            got.append((v, np64(g[0][0, torch.from_numpy(rows).cuda()])[None],
                        np64(g[1][0, S - 64:])[None]))
            del g
        say(f"[gpu] gradients long context {op}: GPU done, oracle on {len(rows)} rows")
        w = _oracle_grads(d, op, dout_cpu[:, rows], idx_cpu, rows=rows)
        for v, dq, dkv_last in got:
            _grad_close(dq, w[0], "bf16", f"{v} dq sampled")
            _grad_close(dkv_last, w[1][:, S - 64:], "bf16", f"{v} dkv last block")
    say("[gpu] gradients long context: ok")


def test_split_work_items_against_oracle():
    """Key-block work items longer than split_rows (128) rows are split and
    their partials added in order. At B = 4, S = 4096 the rows are chunked by
    512 for the gather and by 256 for the window (about 1024 items each), so:
    - rows 0 .. 511 all select block 0 (the rest their own and previous
      blocks): the gather's item of block 0 has 512 rows, four parts; dq of
      those rows and block 0's dkv, which only they reach, are compared with
      the oracle;
    - a window of 1024 gives middle blocks 256-row items (two parts each);
      block 20's dkv is compared from every row that attends it (1280 to
      2366), with dq of those rows, for both workspaces."""
    p = _mla("split_items", 4096, 905, 2, 1024, B=4)
    d = Dev(p)
    dout_cpu = inputs.make_dout(p, seed=906)
    dout = dout_cpu.cuda()
    S = p.Sq
    own = np.arange(S) // 64
    sel = np.stack([np.where(np.arange(S) < 512, 0, own - 1), own], axis=1)
    sel[sel[:, 0] == sel[:, 1], 0] = -1          # distinct ids, -1 for the rest
    sel[sel < 0] = -1
    idx_cpu = np.broadcast_to(sel, (p.B, S, 2)).astype(np.int32).copy()
    idx = torch.from_numpy(idx_cpu).cuda()
    rows = np.arange(512)
    e = []
    for v in ("gather", "gather_ds"):
        g = _gpu_grads(d, v, dout, idx, 2)
        torch.cuda.synchronize()
        got_dq = np64(g[0][:, :512])
        got_dkv = np64(g[1][:, :64])
        del g
        if v == "gather":
            say("[gpu] split items: gather on the GPU done, oracle on rows 0 .. 511")
            w = _oracle_grads(d, "gather", dout_cpu[:, rows], idx_cpu, rows=rows)
        e += [_grad_close(got_dq, w[0], "bf16", f"{v} dq"),
              _grad_close(got_dkv, w[1][:, :64], "bf16", f"{v} dkv block 0")]
    rows = np.arange(1280, 1280 + 64 + p.window - 1)
    for v in ("swa", "swa_recompute"):
        gw = _gpu_grads(d, v, dout)
        torch.cuda.synchronize()
        got_dq = np64(gw[0][:, torch.from_numpy(rows).cuda()])
        got_dkv = np64(gw[1][:, 1280:1344])
        del gw
        if v == "swa":
            say(f"[gpu] split items: window on the GPU done, oracle on {len(rows)} rows")
            ww = _oracle_grads(d, "swa", dout_cpu[:, rows], rows=rows)
        e += [_grad_close(got_dq, ww[0], "bf16", f"{v} dq"),
              _grad_close(got_dkv, ww[1][:, 1280:1344], "bf16", f"{v} dkv block 20")]
    say(f"[gpu] split work items: worst {max(e):.2e}")


def test_gradients_in_captured_graph():
    """The gradient calls allocate nothing and write every workspace word before
    reading it, so one captured graph replays correctly with new upstream
    gradients. Each replay must equal an eager call bit for bit (the gather
    and the causal call, both with stored score gradients)."""
    p = _mla("graph", 333, 44, 3, 90)
    d = Dev(p)
    out, lse, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    og, lg = hs.sparse_gather(d.prob, d.q, d.kv, d.sink, idx, p.top_k)
    dout = inputs.make_dout(p, seed=45).cuda()
    bufs = [(torch.empty((1, p.Sq, p.H, p.Dk), dtype=torch.float32, device="cuda"),
             torch.empty((1, p.Skv, p.Dk), dtype=torch.float32, device="cuda"),
             torch.empty((p.H,), dtype=torch.float32, device="cuda")) for _ in range(2)]
    ws = hs.sparse_gather_bwd_workspace(d.prob, p.top_k, store_ds=True)
    ws2 = hs.score_bwd_workspace(d.prob, store_ds=True)

    def calls():
        hs.hs_sparse_gather_bwd(d.prob, d.q, d.kv, d.sink, idx, p.top_k, og, lg, dout, *bufs[0], ws)
        hs.hs_block_score_bwd(d.prob, d.q, d.kv, d.sink, out, lse, dout, *bufs[1], ws2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        dout.copy_(inputs.make_dout(p, seed=46 + rep).cuda())
        ws.fill_(float("nan"))
        ws2.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [tuple(x.clone() for x in b_) for b_ in bufs]
        want = [hs.sparse_gather_bwd(d.prob, d.q, d.kv, d.sink, idx, p.top_k, og, lg, dout,
                                     store_ds=True),
                hs.block_score_bwd(d.prob, d.q, d.kv, d.sink, out, lse, dout, store_ds=True)]
        torch.cuda.synchronize()
        for call, gg, ww in zip(("gather", "causal"), got, want):
            for g_, w_, n in zip(gg, ww, ("dq", "dkv", "dsink")):
                assert torch.equal(g_, w_), f"replay {rep}: {call} {n} differs from the eager call"
    say("[gpu] gradient graph replays: identical")


def test_sink_without_its_gradient():
    """A sink whose gradient is not asked for (dsink NULL) still shapes dq and
    dkv."""
    p = _mla("no_dsink", 150, 47, 2, 40)
    d = Dev(p)
    out, lse, _ = hs.block_score(d.prob, d.q, d.kv, d.sink)
    dout_cpu = inputs.make_dout(p, seed=48)
    dout = dout_cpu.cuda()
    dq = torch.empty((1, p.Sq, p.H, p.Dk), dtype=torch.float32, device="cuda")
    dkv = torch.empty((1, p.Skv, p.Dk), dtype=torch.float32, device="cuda")
    hs.hs_block_score_bwd(d.prob, d.q, d.kv, d.sink, out, lse, dout, dq, dkv, None,
                          hs._workspace(d.prob, hs.HS_OP_BLOCK_SCORE_BWD))
    torch.cuda.synchronize()
    w = _oracle_grads(d, "score", dout_cpu)
    _grad_close(np64(dq), w[0], "bf16", "dq")
    _grad_close(np64(dkv), w[1], "bf16", "dkv")
    say("[gpu] sink without its gradient: ok")


def test_stored_and_recomputed_score_gradients_agree():
    """The two workspaces of the causal, window and gather gradients: the
    key-block pass is the same arithmetic in both (dkv and dsink
    bit-identical); dq from the stored bf16 score gradients matches dq that
    recomputes them up to dS rounding."""
    p = _mla("paths_S700", 700, 44, 2, 64)
    say(f"[gpu] stored vs recomputed score gradients, S={p.Sq}")
    d = Dev(p)
    dout = inputs.make_dout(p, seed=45).cuda()
    out, lse, bl = hs.block_score(d.prob, d.q, d.kv, d.sink)
    ow, lw = hs.swa(d.prob, d.q, d.kv, d.sink, p.window)
    idx = hs.topk_blocks(d.prob, bl, p.top_k)
    og, lg = hs.sparse_gather(d.prob, d.q, d.kv, d.sink, idx, p.top_k)
    for name, call in (
            ("causal", lambda st: hs.block_score_bwd(d.prob, d.q, d.kv, d.sink, out, lse, dout,
                                                     store_ds=st)),
            ("window", lambda st: hs.swa_bwd(d.prob, d.q, d.kv, d.sink, p.window, ow, lw, dout,
                                             store_ds=st)),
            ("gather", lambda st: hs.sparse_gather_bwd(d.prob, d.q, d.kv, d.sink, idx, p.top_k, og,
                                                       lg, dout, store_ds=st))):
        a = call(True)
        b = call(False)
        torch.cuda.synchronize()
        assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]), name
        err = ((a[0] - b[0]).abs().max() / b[0].abs().max()).item()
        say(f"[gpu] {name} dq stored vs recomputed: max |diff| / max |dq| = {err:.2e}")
        assert err < 1e-2, name
