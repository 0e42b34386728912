"""GPU check of the entry point that allocates nothing,
hs_block_score_topk_fwd_noalloc, through the C ABI: its outputs match
hs_block_score_topk_fwd on the same inputs (bf16 tolerance on out and lse,
block scores within the block-score tolerance, selections exact where the
scores agree bit for bit), on two calls in a row, the second with a smaller
input, on a decode batch whose key range is split (the scratch array holds
the partials) and on a prefill that does not split."""
import numpy as np
import pytest
import torch

import block_sparse_mqa_amd as hs
from block_sparse_mqa_amd import inputs
from oracle import hysparse_ref as ref

from gpu_common import BF16_TOL, BLOCK_LOGIT_TOL, assert_close, np64, say

pytestmark = pytest.mark.gpu


def _case(B, Skv, lens, seed, top_k, Sq=1):
    p = inputs.make(B, Sq, Skv, 64, 576, 512, seed=seed, kv_lens=lens, top_k=top_k, window=64,
                    name=f"noalloc_{B}_{Skv}")
    prob = hs.Problem(p.B, p.Sq, p.Skv, p.H, p.Dk, p.Dv, kv_lens=p.kv_lens)
    return p, prob, p.q.cuda(), p.kv.cuda(), p.sink.cuda()


def _both(p, prob, q, kv, sink):
    NB = hs.hs_num_blocks(prob)
    shp_o, shp_l = (p.B, p.Sq, p.H, p.Dv), (p.B, p.Sq, p.H)
    res = []
    for noalloc in (True, False):
        out = torch.empty(shp_o, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(shp_l, dtype=torch.float32, device="cuda")
        bl = torch.empty((p.B, p.Sq, NB), dtype=torch.float32, device="cuda")
        idx = torch.empty((p.B, p.Sq, p.top_k), dtype=torch.int32, device="cuda")
        if noalloc:
            hs.hs_block_score_topk_fwd_noalloc(prob, q, kv, sink, p.top_k, out, lse, bl, idx)
        else:
            hs.hs_block_score_topk_fwd(prob, q, kv, sink, p.top_k, out, lse, bl, idx,
                                       hs._workspace(prob, hs.HS_OP_BLOCK_SCORE))
        torch.cuda.synchronize()
        res.append((out, lse, bl, idx))
    return res


def _compare(p, prob, got, want, name):
    e = [assert_close(np64(got[0]), np64(want[0]), BF16_TOL, f"{name} out"),
         assert_close(np64(got[1]), np64(want[1]), BF16_TOL, f"{name} lse"),
         assert_close(np64(got[2]), np64(want[2]), BLOCK_LOGIT_TOL, f"{name} block_logit")]
    # the selection is exact on the call's own scores
    own = ref.own_blocks(p.B, p.Sq, p.Skv, 64, p.kv_lens)
    assert np.array_equal(got[3].cpu().numpy(), ref.topk_blocks(got[2].cpu().numpy(), own, p.top_k))
    same = torch.equal(got[2], want[2])
    if same:
        assert torch.equal(got[3], want[3]), f"{name}: selections differ on identical scores"
    return max(e), same


def test_noalloc_matches_workspace_call_twice():
    rng = np.random.default_rng(91)
    # 1) decode over long caches: the key range splits, partials in the scratch array
    lens = [int(x) for x in rng.integers(16384, 65537, size=32)]
    p, prob, q, kv, sink = _case(32, 65536, lens, 91, 32)
    assert hs.hs_workspace_size(prob, hs.HS_OP_BLOCK_SCORE) > 0
    say("[gpu] noalloc call 1: decode B=32 caches 16k-64k")
    got, want = _both(p, prob, q, kv, sink)
    e1, s1 = _compare(p, prob, got, want, "decode")
    del q, kv, got, want
    torch.cuda.empty_cache()
    # 2) a smaller input right after: shorter caches, fewer entries (the array
    #    keeps the first call's contents)
    lens2 = [int(x) for x in rng.integers(1, 5000, size=5)]
    p2, prob2, q2, kv2, sink2 = _case(5, 5000, lens2, 92, 4)
    say("[gpu] noalloc call 2: decode B=5 caches up to 5000")
    got, want = _both(p2, prob2, q2, kv2, sink2)
    e2, s2 = _compare(p2, prob2, got, want, "small decode")
    # 3) a prefill that does not split (no scratch use)
    p3, prob3, q3, kv3, sink3 = _case(1, 300, None, 93, 3, Sq=300)
    got, want = _both(p3, prob3, q3, kv3, sink3)
    e3, s3 = _compare(p3, prob3, got, want, "prefill")
    say(f"[gpu] noalloc vs workspace call: max errors {e1:.2e} {e2:.2e} {e3:.2e}, "
        f"identical scores {s1} {s2} {s3}")


def test_noalloc_rejects_before_launch():
    lib = hs.load_library()
    p = hs.Problem(1, 128, 128, 64, 576, 512)
    f = __import__("ctypes").c_void_p(4096)
    assert lib.hs_block_score_topk_fwd_noalloc(p.ref, f, f, None, 0, f, f, f, f, None, None) == \
        hs.HS_ERR_INVALID_ARG
    assert lib.hs_block_score_topk_fwd_noalloc(p.ref, None, f, None, 4, f, f, f, f, None, None) == \
        hs.HS_ERR_INVALID_ARG
