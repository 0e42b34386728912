"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid arguments before any launch. No call
here reaches the GPU (each one fails validation or is host-only), so these
run on a machine without one."""
import ctypes
import os
import re

import pytest

import block_sparse_mqa_amd as hs
from oracle import hysparse_ref as ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    with open(os.path.join(ROOT, "include", "hs.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(hs_[a-z_0-9]+)\s*\(",
                                 src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = hs.load_library()
    names = _header_functions()
    assert set(names) == set(hs.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.hs_version() == 202


def _mla(**kw):
    base = dict(B=1, Sq=128, Skv=128, H=64, Dk=576, Dv=512)
    base.update(kw)
    return hs.Problem(base.pop("B"), base.pop("Sq"), base.pop("Skv"), base.pop("H"),
                      base.pop("Dk"), base.pop("Dv"), **base)


@pytest.mark.parametrize("kw,exc", [
    (dict(B=0), ValueError),
    (dict(Sq=0), ValueError),
    (dict(Sq=200), ValueError),                                # Sq > Skv
    (dict(Dv=600, Dk=576), ValueError),                        # value wider than key
    (dict(H=32), NotImplementedError),                         # not a built instantiation
    (dict(block_size=32), NotImplementedError),
    (dict(dtype="f32", H=32, Dk=96, Dv=64), NotImplementedError),
    (dict(kv_lens=[100, 100]), ValueError),                    # n_kv_lens != B
    (dict(kv_lens=[127], Sq=128), ValueError),                 # Sq > L_b
    (dict(kv_lens=[129]), ValueError),                         # L_b > Skv
    (dict(doc_start=[0, 60], doc_end=[60, 100]), ValueError),  # docs do not reach Sq
    (dict(doc_start=[0, 61], doc_end=[60, 128]), ValueError),  # gap
    (dict(doc_start=[0], doc_end=[128], B=2), ValueError),     # docs need B == 1
    (dict(doc_start=list(range(0, 65 * 2, 2)), doc_end=list(range(2, 65 * 2 + 2, 2)),
          Sq=130, Skv=130), NotImplementedError),              # more than 64 docs
])
def test_problem_validation(kw, exc):
    with pytest.raises(exc):
        hs.hs_num_blocks(_mla(**kw))


def test_entry_points_reject_before_launch():
    lib = hs.load_library()
    p = _mla()
    fake = ctypes.c_void_p(4096)
    # NULL q
    st = lib.hs_block_score_fwd(p.ref, None, fake, None, fake, fake, fake, None, 0, None)
    assert st == hs.HS_ERR_INVALID_ARG and b"q is NULL" in lib.hs_last_error()
    # misaligned kv
    st = lib.hs_block_score_fwd(p.ref, fake, ctypes.c_void_p(4098), None, fake, fake, fake, None, 0, None)
    assert st == hs.HS_ERR_INVALID_ARG and b"kv" in lib.hs_last_error()
    # top_k out of range
    st = lib.hs_topk_blocks(p.ref, fake, 0, fake, None)
    assert st == hs.HS_ERR_INVALID_ARG
    st = lib.hs_topk_blocks(p.ref, fake, 65, fake, None)
    assert st == hs.HS_ERR_UNSUPPORTED
    st = lib.hs_sparse_gather_fwd(p.ref, fake, fake, None, fake, 0, fake, fake, None, 0, None)
    assert st == hs.HS_ERR_INVALID_ARG
    # window < 1
    st = lib.hs_swa_fwd(p.ref, fake, fake, None, 0, fake, fake, None, 0, None)
    assert st == hs.HS_ERR_INVALID_ARG and b"window" in lib.hs_last_error()
    # decode that needs a workspace but gets none
    d = _mla(B=2, Sq=1, Skv=4096, kv_lens=[4096, 2000])
    assert hs.hs_workspace_size(d, hs.HS_OP_BLOCK_SCORE) > 0
    st = lib.hs_block_score_fwd(d.ref, fake, fake, None, fake, fake, fake, None, 0, None)
    assert st == hs.HS_ERR_WORKSPACE
    assert lib.hs_status_string(-2) == b"HS_ERR_UNSUPPORTED"


def test_fused_score_topk_rejects_before_launch():
    lib = hs.load_library()
    p = _mla()
    fake = ctypes.c_void_p(4096)
    call = lambda k, idx, prob=p, bp=None: lib.hs_block_score_topk_fwd(
        prob.ref, fake, fake, None, k, fake, fake, fake, idx, bp, None, 0, None)
    assert call(0, fake) == hs.HS_ERR_INVALID_ARG and b"top_k" in lib.hs_last_error()
    assert call(65, fake) == hs.HS_ERR_UNSUPPORTED
    assert call(4, None) == hs.HS_ERR_INVALID_ARG and b"block_idx is NULL" in lib.hs_last_error()
    assert call(4, ctypes.c_void_p(4098)) == hs.HS_ERR_INVALID_ARG
    assert call(4, fake, bp=ctypes.c_void_p(4098)) == hs.HS_ERR_INVALID_ARG and \
        b"block_prob" in lib.hs_last_error()
    # more than 4096 blocks cannot be selected from
    big = _mla(B=1, Sq=1, Skv=4097 * 64, kv_lens=[4097 * 64])
    assert call(4, fake, big) == hs.HS_ERR_UNSUPPORTED and b"4096" in lib.hs_last_error()
    # split decode without its workspace
    d = _mla(B=2, Sq=1, Skv=4096, kv_lens=[4096, 2000])
    assert call(4, fake, d) == hs.HS_ERR_WORKSPACE


def test_gradient_calls_reject_before_launch():
    lib = hs.load_library()
    p = _mla()
    f = ctypes.c_void_p(4096)
    n = hs.hs_workspace_size(p, hs.HS_OP_BLOCK_SCORE_BWD)
    assert n > 0
    big = ctypes.c_size_t(n)

    def score(prob=p, q=f, sink=None, dout=f, dlse=None, dsink=None, ws=f, nbytes=big):
        return lib.hs_block_score_bwd(prob.ref, q, f, sink, f, f, dout, dlse, f, f, dsink, ws,
                                      nbytes, None)
    assert score(q=None) == hs.HS_ERR_INVALID_ARG and b"q is NULL" in lib.hs_last_error()
    assert score(dout=ctypes.c_void_p(4100)) == hs.HS_ERR_INVALID_ARG
    assert score(dlse=ctypes.c_void_p(4098)) == hs.HS_ERR_INVALID_ARG and \
        b"dlse" in lib.hs_last_error()
    assert score(dsink=f) == hs.HS_ERR_INVALID_ARG and b"no sink" in lib.hs_last_error()
    assert score(ws=None) == hs.HS_ERR_WORKSPACE
    assert score(nbytes=ctypes.c_size_t(n - 1)) == hs.HS_ERR_WORKSPACE
    assert score(ws=ctypes.c_void_p(4104)) == hs.HS_ERR_WORKSPACE
    # paged KV has no gradient path
    paged = _raw_problem()
    st = lib.hs_block_score_bwd(ctypes.byref(paged), f, f, None, f, f, f, None, f, f, None, f,
                                big, None)
    assert st == hs.HS_ERR_UNSUPPORTED and b"paged" in lib.hs_last_error()
    # window and top_k
    st = lib.hs_swa_bwd(p.ref, f, f, None, 0, f, f, f, None, f, f, None, f, big, None)
    assert st == hs.HS_ERR_INVALID_ARG and b"window" in lib.hs_last_error()
    st = lib.hs_sparse_gather_bwd(p.ref, f, f, None, f, 65, f, f, f, None, f, f, None, f, big,
                                  None)
    assert st == hs.HS_ERR_UNSUPPORTED
    st = lib.hs_sparse_gather_bwd(p.ref, f, f, None, None, 4, f, f, f, None, f, f, None, f,
                                  big, None)
    assert st == hs.HS_ERR_INVALID_ARG and b"block_idx" in lib.hs_last_error()
    with pytest.raises(ValueError):
        hs.hs_workspace_size(p, hs.HS_OP_SWA_BWD, window=0)


def test_gradient_workspace_sizes():
    """Gradients always need a workspace; it grows with the work items of the
    key-block gradient and covers the gather's row lists."""
    small = _mla(Sq=128, Skv=128)
    big = _mla(Sq=4096, Skv=4096)
    for op, kw in ((hs.HS_OP_BLOCK_SCORE_BWD, {}), (hs.HS_OP_SPARSE_GATHER_BWD, {"top_k": 8}),
                   (hs.HS_OP_SWA_BWD, {"window": 256})):
        a = hs.hs_workspace_size(small, op, **kw)
        b = hs.hs_workspace_size(big, op, **kw)
        assert 0 < a < b
    f32 = _mla(dtype="f32", H=8, Dk=96, Dv=64)
    assert hs.hs_workspace_size(f32, hs.HS_OP_BLOCK_SCORE_BWD) >= 128 * 8 * 4


@pytest.mark.parametrize("case", [
    dict(L=512, docs=None, kv_lens=None, B=1),
    dict(L=130, docs=None, kv_lens=None, B=1),
    dict(L=200, docs=[(0, 70), (70, 71), (71, 134), (134, 200)], kv_lens=None, B=1),
    dict(L=65536, docs=None, kv_lens=[16384, 65536, 17, 40000], B=4),
])
def test_block_count_matches_oracle(case):
    docs = case["docs"]
    ds = [a for a, _ in docs] if docs else None
    de = [b for _, b in docs] if docs else None
    Sq = 1 if case["kv_lens"] else case["L"]
    p = _mla(B=case["B"], Sq=Sq, Skv=case["L"], kv_lens=case["kv_lens"], doc_start=ds, doc_end=de)
    assert hs.hs_num_blocks(p) == ref.num_blocks(case["B"], case["L"], 64, case["kv_lens"], ds, de)


def test_workspace_only_for_split_decode():
    assert hs.hs_workspace_size(_mla(Sq=4096, Skv=4096), hs.HS_OP_BLOCK_SCORE) == 0
    d = _mla(B=32, Sq=1, Skv=65536, kv_lens=[65536] * 32)
    for op in (hs.HS_OP_BLOCK_SCORE, hs.HS_OP_SPARSE_GATHER, hs.HS_OP_SWA):
        n = hs.hs_workspace_size(d, op, top_k=32, window=1024)
        assert n > 0 and n % (32 * 64 * 4) == 0
    assert hs.hs_workspace_size(_mla(dtype="f32", H=8, Dk=96, Dv=64, B=2, Sq=1, Skv=512,
                                     kv_lens=[512, 3]), hs.HS_OP_BLOCK_SCORE) == 0


def test_probe_library_exports_every_declared_symbol():
    from block_sparse_mqa_amd import probe
    with open(os.path.join(ROOT, "include", "hs_probe.h")) as f:
        src = f.read()
    names = set(re.findall(r"^\s*[a-z_0-9]+\s+(hs_probe_[a-z_0-9]+)\s*\(", src, flags=re.M))
    assert names == set(probe.EXPORTS), names
    lib = probe.load_probe_library()
    for n in names:
        assert hasattr(lib, n), n
    # host-only arithmetic and host-side argument checks (no launch happens)
    assert lib.hs_probe_mfma_flops(2, 3) == 2 * 4 * 3 * 4 * 32 * 32 * 16 * 2
    assert lib.hs_probe_mfma_bf16(0, 1, ctypes.c_void_p(256), None, None) == -1
    assert lib.hs_probe_mfma_bf16(1, 1, ctypes.c_void_p(256), ctypes.c_void_p(260), None) == -1
    assert lib.hs_probe_copy(ctypes.c_void_p(256), ctypes.c_void_p(4096), 15, None) == -1
    assert lib.hs_probe_copy(ctypes.c_void_p(256), ctypes.c_void_p(272), 64, None) == -1  # overlap


def _raw_problem(**kw):
    """An hs_problem built directly (no device tensors needed): paged-KV
    validation happens on the host before any launch."""
    f = dict(batch=1, seqlen_q=1, seqlen_kv=640, num_heads=64, head_dim_qk=576, head_dim_v=512,
             block_size=64, scale=0.0, dtype=hs.HS_BF16, kv_lens=None, n_kv_lens=0,
             doc_start=None, doc_end=None, n_docs=0, page_table=256, max_pages=10)
    f.update(kw)
    return hs.HsProblem(**f)


def test_paged_kv_validation():
    lib = hs.load_library()
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem())) == 10
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(max_pages=9))) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(max_pages=0))) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(page_table=None))) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(page_table=258))) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(
        dtype=hs.HS_F32, num_heads=8, head_dim_qk=96, head_dim_v=64))) == hs.HS_ERR_UNSUPPORTED
    ds = (ctypes.c_int32 * 1)(0)
    de = (ctypes.c_int32 * 1)(640)
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(
        seqlen_q=640, doc_start=ds, doc_end=de, n_docs=1))) == hs.HS_ERR_INVALID_ARG
    lens = (ctypes.c_int32 * 2)(100, 640)
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(
        batch=2, kv_lens=lens, n_kv_lens=2))) == 10


def test_device_lengths_validation():
    lib = hs.load_library()
    ok = _raw_problem(batch=2, kv_lens_device=512)
    assert lib.hs_num_blocks(ctypes.byref(ok)) == 10            # capacity 640 -> 10 blocks
    # in-place caches take device lengths too (bf16, no documents)
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(page_table=None, max_pages=0,
                                                       kv_lens_device=512))) == 10
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(
        page_table=None, max_pages=0, kv_lens_device=512, dtype=hs.HS_F32, num_heads=8,
        head_dim_qk=96, head_dim_v=64))) == hs.HS_ERR_UNSUPPORTED
    ds = (ctypes.c_int32 * 1)(0)
    de = (ctypes.c_int32 * 1)(640)
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(
        page_table=None, max_pages=0, seqlen_q=640, doc_start=ds, doc_end=de, n_docs=1,
        kv_lens_device=512))) == hs.HS_ERR_INVALID_ARG
    lens = (ctypes.c_int32 * 1)(100)
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(kv_lens=lens, n_kv_lens=1,
                                                       kv_lens_device=512))) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(ctypes.byref(_raw_problem(kv_lens_device=514))) == hs.HS_ERR_INVALID_ARG
    n = ctypes.c_size_t(0)
    assert lib.hs_workspace_size(ctypes.byref(ok), hs.HS_OP_BLOCK_SCORE, 0, 0, ctypes.byref(n)) == 0
    assert n.value > 0                                          # decode split planned at capacity


def test_device_document_bounds_validation():
    """Device-resident document bounds: NB is the capacity bound
    ceil(S / 64) + n_docs - 1; host-only checks before any launch."""
    lib = hs.load_library()

    def prob(**kw):
        f = dict(seqlen_q=1000, seqlen_kv=1000, page_table=None, max_pages=0, n_docs=8,
                 doc_bounds_device=512)
        f.update(kw)
        return ctypes.byref(_raw_problem(**f))
    assert lib.hs_num_blocks(prob()) == 16 + 7
    assert lib.hs_num_blocks(prob(n_docs=1)) == 16
    assert lib.hs_num_blocks(prob(n_docs=64)) == 16 + 63
    assert lib.hs_num_blocks(prob(n_docs=0)) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(prob(n_docs=65)) == hs.HS_ERR_UNSUPPORTED
    assert lib.hs_num_blocks(prob(doc_bounds_device=514)) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(prob(seqlen_q=999)) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(prob(batch=2, seqlen_q=1000)) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(prob(page_table=256, max_pages=16)) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(prob(kv_lens_device=256)) == hs.HS_ERR_INVALID_ARG
    lens = (ctypes.c_int32 * 1)(1000)
    assert lib.hs_num_blocks(prob(kv_lens=lens, n_kv_lens=1)) == hs.HS_ERR_INVALID_ARG
    ds = (ctypes.c_int32 * 1)(0)
    de = (ctypes.c_int32 * 1)(1000)
    assert lib.hs_num_blocks(prob(doc_start=ds, doc_end=de, n_docs=1)) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_num_blocks(prob(dtype=hs.HS_F32, num_heads=8, head_dim_qk=96,
                                  head_dim_v=64)) == hs.HS_ERR_UNSUPPORTED
    # forward workspaces: never split (the host cannot see the packing)
    n = ctypes.c_size_t(1)
    for op in (hs.HS_OP_BLOCK_SCORE, hs.HS_OP_SWA, hs.HS_OP_SPARSE_GATHER):
        assert lib.hs_workspace_size(prob(seqlen_q=256, seqlen_kv=256), op, 8, 64,
                                     ctypes.byref(n)) == 0
        assert n.value == 0
    # gradients take host bounds only
    for op in (hs.HS_OP_BLOCK_SCORE_BWD, hs.HS_OP_SWA_BWD, hs.HS_OP_SPARSE_GATHER_BWD):
        assert lib.hs_workspace_size(prob(), op, 8, 64, ctypes.byref(n)) == hs.HS_ERR_UNSUPPORTED
    f = ctypes.c_void_p(4096)
    st = lib.hs_block_score_bwd(prob(), f, f, None, f, f, f, None, f, f, None, f,
                                ctypes.c_size_t(1 << 30), None)
    assert st == hs.HS_ERR_UNSUPPORTED and b"document" in lib.hs_last_error()


def test_gradient_workspace_bounded_for_long_sequences():
    """Work items are capped (longer sequences take longer row chunks), so the
    gradient workspace stays a few GB even at 4096 key blocks."""
    sizes = []
    for S in (32768, 65536, 262144):
        p = _mla(Sq=S, Skv=S)
        for op, kw in ((hs.HS_OP_BLOCK_SCORE_BWD, {}), (hs.HS_OP_SPARSE_GATHER_BWD, {"top_k": 64}),
                       (hs.HS_OP_SWA_BWD, {"window": 4096})):
            sizes.append(hs.hs_workspace_size(p, op, **kw))
    assert max(sizes) < 6e9, sizes


def _causal_pairs(B, Sq, Skv, kv_lens=None, doc_lens=None):
    """(row, key block) pairs of causal attention, counted row by row: a row
    at position p of a document starting at s reaches blocks s/64 .. p/64 of
    that document."""
    starts = []
    if doc_lens:
        at = 0
        for n in doc_lens:
            starts.append(at)
            at += n
    pairs = 0
    for b in range(B):
        L = kv_lens[b] if kv_lens else Skv
        for r in range(Sq):
            pos = L - Sq + r
            s = max([x for x in starts if x <= pos], default=0)
            pairs += (pos - s) // 64 + 1
    return pairs


@pytest.mark.parametrize("B,Sq,Skv,kv_lens,doc_lens", [
    (1, 130, 130, None, None),
    (1, 1, 1, None, None),
    (2, 70, 200, [200, 150], None),
    (3, 64, 4000, [64, 4000, 1000], None),
    (1, 300, 300, None, [70, 1, 63, 100, 66]),
    (1, 32768, 32768, None, None),
])
def test_stored_score_gradient_workspace(B, Sq, Skv, kv_lens, doc_lens):
    """The larger causal-gradient workspace adds exactly 8 KB per causal
    (row, key block) pair (bf16 dS of 64 heads x 64 keys), plus the per-entry
    tile offsets and a 4 KB dummy target, each 256-byte aligned: a check of
    the closed-form tile count against a row-by-row count."""
    kw = {}
    if kv_lens:
        kw["kv_lens"] = kv_lens
    if doc_lens:
        ends = [sum(doc_lens[:i + 1]) for i in range(len(doc_lens))]
        kw["doc_start"] = [e - n for e, n in zip(ends, doc_lens)]
        kw["doc_end"] = ends
    p = hs.Problem(B, Sq, Skv, 64, 576, 512, **kw)
    n3 = hs.hs_workspace_size(p, hs.HS_OP_BLOCK_SCORE_BWD)
    n6 = hs.hs_workspace_size(p, hs.HS_OP_BLOCK_SCORE_BWD_STORE_DS)
    a256 = lambda x: (x + 255) // 256 * 256
    pairs = _causal_pairs(B, Sq, Skv, kv_lens, doc_lens)
    assert n6 - n3 == a256((B + 1) * 8) + a256(4096) + a256(pairs * 8192), (n3, n6, pairs)


def test_stored_score_gradient_workspace_f32_unchanged():
    """The fp32 shapes always recompute: both queries give the same size, for
    the causal and the window gradient."""
    p = hs.Problem(1, 100, 100, 8, 96, 64, dtype="f32")
    assert hs.hs_workspace_size(p, hs.HS_OP_BLOCK_SCORE_BWD_STORE_DS) == \
        hs.hs_workspace_size(p, hs.HS_OP_BLOCK_SCORE_BWD)
    assert hs.hs_workspace_size(p, hs.HS_OP_SPARSE_GATHER_BWD_STORE_DS, top_k=3) == \
        hs.hs_workspace_size(p, hs.HS_OP_SPARSE_GATHER_BWD, top_k=3)
    assert hs.hs_workspace_size(p, hs.HS_OP_SWA_BWD_STORE_DS, window=30) == \
        hs.hs_workspace_size(p, hs.HS_OP_SWA_BWD, window=30)


def test_workspace_query_rejects_unknown_ops():
    """Op codes past the last one and a window below 1 for the window
    gradient's larger workspace are errors."""
    p = _mla()
    with pytest.raises(ValueError):
        hs.hs_workspace_size(p, hs.HS_OP_SPARSE_GATHER_BWD_STORE_DS + 1)
    with pytest.raises(ValueError):
        hs.hs_workspace_size(p, hs.HS_OP_SPARSE_GATHER_BWD_STORE_DS, top_k=0)
    with pytest.raises(ValueError):
        hs.hs_workspace_size(p, hs.HS_OP_SWA_BWD_STORE_DS, window=0)


@pytest.mark.parametrize("B,Sq,Skv,top_k", [(1, 130, 130, 2), (1, 32768, 32768, 32),
                                             (2, 70, 200, 64)])
def test_stored_gather_gradient_workspace(B, Sq, Skv, top_k):
    """The larger gather-gradient workspace adds 8 KB per row and per
    selection entry, the list position of each row-list entry (4 B per row and
    entry) and the same small pieces as the causal one."""
    p = hs.Problem(B, Sq, Skv, 64, 576, 512)
    n4 = hs.hs_workspace_size(p, hs.HS_OP_SPARSE_GATHER_BWD, top_k=top_k)
    n9 = hs.hs_workspace_size(p, hs.HS_OP_SPARSE_GATHER_BWD_STORE_DS, top_k=top_k)
    a256 = lambda x: (x + 255) // 256 * 256
    assert n9 - n4 == (a256(B * Sq * top_k * 4) + a256((B + 1) * 8) + a256(4096) +
                       a256(B * Sq * top_k * 8192)), (n4, n9)


@pytest.mark.parametrize("B,Sq,Skv,window,kv_lens,per_row", [
    (1, 130, 130, 70, None, 3),            # ceil(69 / 64) + 1
    (1, 32768, 32768, 1024, None, 17),
    (1, 300, 300, 1, None, 1),
    (1, 100, 100, 5000, None, 2),          # capped at the block count
    (2, 70, 200, 64, [200, 150], 2),
])
def test_stored_window_gradient_workspace(B, Sq, Skv, window, kv_lens, per_row):
    """The larger window-gradient workspace adds 8 KB per row for each block a
    window of that size can meet (ceil((window - 1) / 64) + 1, at most the
    block count), plus the same small pieces as the causal one; that bound
    holds for every row (checked row by row)."""
    kw = {"kv_lens": kv_lens} if kv_lens else {}
    p = hs.Problem(B, Sq, Skv, 64, 576, 512, **kw)
    n5 = hs.hs_workspace_size(p, hs.HS_OP_SWA_BWD, window=window)
    n7 = hs.hs_workspace_size(p, hs.HS_OP_SWA_BWD_STORE_DS, window=window)
    a256 = lambda x: (x + 255) // 256 * 256
    assert n7 - n5 == a256((B + 1) * 8) + a256(4096) + a256(B * Sq * per_row * 8192), (n5, n7)
    for b in range(B):
        L = kv_lens[b] if kv_lens else Skv
        for r in range(0, Sq, max(1, Sq // 500)):
            pos = L - Sq + r
            lo = max(pos - window + 1, 0)
            assert pos // 64 - lo // 64 + 1 <= per_row


def test_binding_rejects_wrong_dtype_and_shape():
    """The C ABI sees pointers only; the binding checks every tensor's dtype
    and shape by its role before the call (the checks run before the device
    check, so host tensors exercise them here)."""
    import torch
    p = _mla(Sq=128, Skv=128)
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    q = torch.zeros(1, 128, 64, 576, dtype=bf)
    kv = torch.zeros(1, 128, 576, dtype=bf)
    out = torch.zeros(1, 128, 64, 512, dtype=bf)
    lse = torch.zeros(1, 128, 64, dtype=f32)
    bl = torch.zeros(1, 128, 2, dtype=f32)
    idx = torch.zeros(1, 128, 4, dtype=i32)
    sink = torch.zeros(64, dtype=f32)
    cases = [
        (dict(sink=sink.to(bf)), "sink"),                                   # bf16 sink
        (dict(sink=torch.zeros(32, dtype=f32)), "sink"),                    # wrong head count
        (dict(q=q.to(f32)), "q"),                                           # fp32 q for bf16
        (dict(q=q[:, :64]), "q"),                                           # short q
        (dict(kv=kv[:, :, :512]), "kv"),                                    # kv without rope
        (dict(lse=lse.to(torch.float64)), "lse"),
        (dict(out=out[..., :256]), "out"),
        (dict(block_logit=torch.zeros(1, 128, 3, dtype=f32)), "block_logit"),  # NB is 2
    ]
    for over, name in cases:
        a = dict(q=q, kv=kv, sink=sink, out=out, lse=lse, block_logit=bl)
        a.update(over)
        with pytest.raises(ValueError, match=name):
            hs.hs_block_score_fwd(p, a["q"], a["kv"], a["sink"], a["out"], a["lse"],
                                  a["block_logit"])
    # int64 selections (what torch.topk returns) and the wrong width
    for bad in (idx.to(torch.int64), torch.zeros(1, 128, 5, dtype=i32)):
        with pytest.raises(ValueError, match="block_idx"):
            hs.hs_sparse_gather_fwd(p, q, kv, sink, bad, 4, out, lse)
        with pytest.raises(ValueError, match="block_idx"):
            hs.hs_topk_blocks(p, bl, 4, bad)
    with pytest.raises(ValueError, match="dq"):
        hs.hs_block_score_bwd(p, q, kv, sink, out, lse, out, q, kv.to(f32), None, None)
    with pytest.raises(ValueError, match="page_table"):
        hs.Problem(1, 1, 640, 64, 576, 512, page_table=torch.zeros(1, 10, dtype=torch.int64))
    with pytest.raises(ValueError, match="kv_lens_device"):
        hs.Problem(2, 1, 640, 64, 576, 512, page_table=torch.zeros(2, 10, dtype=i32),
                   kv_lens_device=torch.zeros(2, dtype=torch.int64))
    # paged pools are [n_pages, 64, Dk] (the role check reads prob.page_table;
    # a host table stands in for the device one here)
    pp = hs.Problem(1, 1, 640, 64, 576, 512)
    pp.page_table = torch.zeros(1, 10, dtype=i32)
    with pytest.raises(ValueError, match="paged kv"):
        hs.hs_block_score_fwd(pp, q[:, :1], torch.zeros(10, 32, 576, dtype=bf), sink,
                              out[:, :1], lse[:, :1], torch.zeros(1, 1, 10, dtype=f32))


def test_window_and_sparse_call_rejects_before_launch():
    """Host validation of hs_swa_sparse_fwd and its workspace query: NULL
    outputs, top_k and window ranges (top_k > 64 is unsupported, as for the
    gather), checked before any launch."""
    lib = hs.load_library()
    p = _mla()
    f = ctypes.c_void_p(4096)

    def call(top_k=4, window=16, out_swa=f, lse_swa=f, out_sparse=f, lse_sparse=f, idx=f,
             ga=None, gb=None, om=None):
        return lib.hs_swa_sparse_fwd(p.ref, f, f, None, window, idx, top_k, out_swa, lse_swa,
                                     out_sparse, lse_sparse, ga, gb, om, None, 0, None)
    assert call(out_swa=None) == hs.HS_ERR_INVALID_ARG and b"out_swa" in lib.hs_last_error()
    assert call(lse_sparse=None) == hs.HS_ERR_INVALID_ARG and b"lse_sparse" in lib.hs_last_error()
    assert call(idx=None) == hs.HS_ERR_INVALID_ARG and b"block_idx" in lib.hs_last_error()
    assert call(top_k=0) == hs.HS_ERR_INVALID_ARG
    assert call(top_k=65) == hs.HS_ERR_UNSUPPORTED
    assert call(window=0) == hs.HS_ERR_INVALID_ARG and b"window" in lib.hs_last_error()
    # the gated combination takes both gates and the output, or none of them
    assert call(ga=f) == hs.HS_ERR_INVALID_ARG and b"gate_sparse" in lib.hs_last_error()
    assert call(ga=f, gb=f) == hs.HS_ERR_INVALID_ARG and b"out_mix" in lib.hs_last_error()
    assert call(ga=f, gb=ctypes.c_void_p(4098), om=f) == hs.HS_ERR_INVALID_ARG
    assert call(om=f) == hs.HS_ERR_INVALID_ARG and b"gate_swa" in lib.hs_last_error()
    n = ctypes.c_size_t(0)
    ws = lambda k, w: lib.hs_workspace_size(p.ref, hs.HS_OP_SWA_SPARSE, k, w, ctypes.byref(n))
    assert ws(4, 16) == hs.HS_OK and n.value == 0
    assert ws(0, 16) == hs.HS_ERR_INVALID_ARG
    assert ws(65, 16) == hs.HS_ERR_UNSUPPORTED
    assert ws(4, 0) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_workspace_size(p.ref, hs.HS_OP_SPARSE_GATHER_BWD, 65, 0,
                                 ctypes.byref(n)) == hs.HS_ERR_UNSUPPORTED
    # a decode shape that splits both branches needs the workspace
    d = _mla(B=2, Sq=1, Skv=65536, kv_lens=[65536, 30000])
    assert hs.hs_workspace_size(d, hs.HS_OP_SWA_SPARSE, top_k=32, window=1024) > 0
