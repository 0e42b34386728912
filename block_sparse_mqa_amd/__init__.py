"""Python binding of libhysparse.so, the HIP (gfx950) library of the HySparse
MQA sparse-attention path (forward operations and their gradients).

The entry points mirror the C ABI of ``include/hs.h`` one to one
(``hs_block_score_fwd``, ``hs_topk_blocks``, ``hs_block_score_topk_fwd``,
``hs_sparse_gather_fwd``, ``hs_swa_fwd``, ``hs_swa_sparse_fwd``, the gradients ``hs_block_score_bwd``,
``hs_sparse_gather_bwd`` and ``hs_swa_bwd``, ``hs_num_blocks``,
``hs_workspace_size``). They only marshal
arguments: tensors are device buffers owned by the caller (PyTorch provides
memory and the current stream), and every step of the computation runs in the
library's kernels. There is no fallback: if the library is missing, or an
argument is rejected, the call raises.

The convenience functions ``block_score``, ``topk_blocks``, ``sparse_gather``,
``swa`` and the gradient functions ``block_score_bwd``, ``sparse_gather_bwd``
and ``swa_bwd`` allocate the outputs (and any workspace) with PyTorch and call the
entry points above.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhysparse.so")

HS_OK, HS_ERR_INVALID_ARG, HS_ERR_UNSUPPORTED, HS_ERR_HIP, HS_ERR_WORKSPACE = 0, -1, -2, -3, -4
HS_BF16, HS_F32 = 0, 1
HS_OP_BLOCK_SCORE, HS_OP_SPARSE_GATHER, HS_OP_SWA = 0, 1, 2
HS_OP_BLOCK_SCORE_BWD, HS_OP_SPARSE_GATHER_BWD, HS_OP_SWA_BWD = 3, 4, 5
HS_OP_BLOCK_SCORE_BWD_STORE_DS, HS_OP_SWA_BWD_STORE_DS = 6, 7
HS_OP_SWA_SPARSE = 8
HS_OP_SPARSE_GATHER_BWD_STORE_DS = 9

EXPORTS = ("hs_num_blocks", "hs_workspace_size", "hs_block_score_fwd", "hs_topk_blocks",
           "hs_block_score_topk_fwd", "hs_block_score_topk_fwd_noalloc", "hs_sparse_gather_fwd",
           "hs_swa_fwd", "hs_swa_sparse_fwd",
           "hs_block_score_bwd", "hs_sparse_gather_bwd", "hs_swa_bwd", "hs_status_string",
           "hs_last_error", "hs_version")


class HsProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("seqlen_kv", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("kv_lens", ctypes.POINTER(ctypes.c_int32)), ("n_kv_lens", ctypes.c_int32),
        ("doc_start", ctypes.POINTER(ctypes.c_int32)),
        ("doc_end", ctypes.POINTER(ctypes.c_int32)), ("n_docs", ctypes.c_int32),
        ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
        ("kv_lens_device", ctypes.c_void_p), ("doc_bounds_device", ctypes.c_void_p),
    ]


class HsError(RuntimeError):
    pass


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhysparse.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_sparse_mqa_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(HsProblem)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.hs_num_blocks.argtypes, lib.hs_num_blocks.restype = [P], i32
    lib.hs_workspace_size.argtypes = [P, i32, i32, i32, ctypes.POINTER(sz)]
    lib.hs_workspace_size.restype = i32
    lib.hs_block_score_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs_block_score_fwd.restype = i32
    lib.hs_topk_blocks.argtypes, lib.hs_topk_blocks.restype = [P, vp, i32, vp, vp], i32
    lib.hs_block_score_topk_fwd.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs_block_score_topk_fwd.restype = i32
    lib.hs_block_score_topk_fwd_noalloc.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
    lib.hs_block_score_topk_fwd_noalloc.restype = i32
    lib.hs_sparse_gather_fwd.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.hs_sparse_gather_fwd.restype = i32
    lib.hs_swa_fwd.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.hs_swa_fwd.restype = i32
    lib.hs_swa_sparse_fwd.argtypes = [P, vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                      sz, vp]
    lib.hs_swa_sparse_fwd.restype = i32
    lib.hs_block_score_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs_block_score_bwd.restype = i32
    lib.hs_sparse_gather_bwd.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                         sz, vp]
    lib.hs_sparse_gather_bwd.restype = i32
    lib.hs_swa_bwd.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hs_swa_bwd.restype = i32
    lib.hs_status_string.argtypes, lib.hs_status_string.restype = [i32], ctypes.c_char_p
    lib.hs_last_error.argtypes, lib.hs_last_error.restype = [], ctypes.c_char_p
    lib.hs_version.argtypes, lib.hs_version.restype = [], i32
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status == HS_OK:
        return
    lib = load_library()
    msg = f"{lib.hs_status_string(status).decode()}: {lib.hs_last_error().decode()}"
    if status == HS_ERR_INVALID_ARG:
        raise ValueError(msg)
    if status == HS_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise HsError(msg)


class Problem:
    """Owns an ``hs_problem`` and the host arrays it points to."""

    def __init__(self, B: int, Sq: int, Skv: int, H: int, Dk: int, Dv: int, *,
                 block_size: int = 64, scale: float = 0.0, dtype: str = "bf16",
                 kv_lens: Optional[Sequence[int]] = None,
                 doc_start: Optional[Sequence[int]] = None,
                 doc_end: Optional[Sequence[int]] = None,
                 page_table=None, kv_lens_device=None, doc_bounds_device=None):
        """page_table: optional int32 device tensor [B, max_pages] (paged KV: kv is
        then a pool [n_pages, block_size, Dk]); kv_lens_device: optional int32
        device tensor [B] of lengths read at run time (bf16, in-place or paged; Skv is
        then the capacity); doc_bounds_device: optional int32 device tensor
        [n_docs + 1] of cumulative document starts read at run time (bf16 forward;
        its length minus one is the document capacity). The tensors must outlive
        the calls."""
        self.B, self.Sq, self.Skv, self.H, self.Dk, self.Dv = B, Sq, Skv, H, Dk, Dv
        self.page_table = page_table
        self.block_size = block_size
        if page_table is not None or kv_lens_device is not None or doc_bounds_device is not None:
            import torch
            if page_table is not None and (page_table.dim() != 2 or page_table.shape[0] != B):
                raise ValueError("page_table must be [B, max_pages]")
            _meta("page_table", page_table, torch.int32)
            _meta("kv_lens_device", kv_lens_device, torch.int32, (B,))
            if doc_bounds_device is not None and doc_bounds_device.dim() != 1:
                raise ValueError("doc_bounds_device must be [n_docs + 1]")
            _meta("doc_bounds_device", doc_bounds_device, torch.int32)
            _dev("page_table", page_table)
            _dev("kv_lens_device", kv_lens_device)
            _dev("doc_bounds_device", doc_bounds_device)
        self.kv_lens_device = kv_lens_device
        self.doc_bounds_device = doc_bounds_device
        n_docs = len(doc_start) if doc_start is not None else 0
        if doc_bounds_device is not None:
            n_docs = int(doc_bounds_device.shape[0]) - 1
        self.dtype = dtype
        self._kv = (ctypes.c_int32 * len(kv_lens))(*kv_lens) if kv_lens is not None else None
        self._ds = (ctypes.c_int32 * len(doc_start))(*doc_start) if doc_start is not None else None
        self._de = (ctypes.c_int32 * len(doc_end))(*doc_end) if doc_end is not None else None
        self.c = HsProblem(
            batch=B, seqlen_q=Sq, seqlen_kv=Skv, num_heads=H, head_dim_qk=Dk, head_dim_v=Dv,
            block_size=block_size, scale=float(scale),
            dtype=HS_BF16 if dtype == "bf16" else HS_F32,
            kv_lens=ctypes.cast(self._kv, ctypes.POINTER(ctypes.c_int32)) if self._kv else None,
            n_kv_lens=len(kv_lens) if kv_lens is not None else 0,
            doc_start=ctypes.cast(self._ds, ctypes.POINTER(ctypes.c_int32)) if self._ds else None,
            doc_end=ctypes.cast(self._de, ctypes.POINTER(ctypes.c_int32)) if self._de else None,
            n_docs=n_docs,
            page_table=None if page_table is None else page_table.data_ptr(),
            max_pages=0 if page_table is None else int(page_table.shape[1]),
            kv_lens_device=None if kv_lens_device is None else kv_lens_device.data_ptr(),
            doc_bounds_device=None if doc_bounds_device is None else doc_bounds_device.data_ptr())

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _meta(name, t, dtype=None, shape=None):
    """Reject a tensor of the wrong dtype or shape (the C ABI sees only a
    pointer and cannot check either)."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dev(name, t, dtype=None, shape=None):
    """_meta, then reject host memory and non-contiguous layouts."""
    if t is None:
        return
    _meta(name, t, dtype, shape)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _tdt(prob):
    import torch
    return torch.bfloat16 if prob.dtype == "bf16" else torch.float32


def _check_io(prob, **tensors):
    """Dtype and shape of every tensor argument by its role (include/hs.h), all
    of them first; then that each is contiguous device memory."""
    import torch
    B, Sq, Skv, H, Dk, Dv = prob.B, prob.Sq, prob.Skv, prob.H, prob.Dk, prob.Dv
    f32, i32, dt = torch.float32, torch.int32, _tdt(prob)
    k = tensors.pop("_top_k", None)
    for name, t in tensors.items():
        if t is None:
            continue
        if name == "q":
            _meta(name, t, dt, (B, Sq, H, Dk))
        elif name == "kv":
            _meta(name, t, dt)
            if prob.page_table is not None:
                if t.dim() != 3 or tuple(t.shape[1:]) != (prob.block_size, Dk):
                    raise ValueError(f"paged kv must be [n_pages, {prob.block_size}, {Dk}], "
                                     f"got {tuple(t.shape)}")
            else:
                _meta(name, t, dt, (B, Skv, Dk))
        elif name in ("sink", "dsink"):
            _meta(name, t, f32, (H,))
        elif name in ("gate_swa", "gate_sparse"):
            _meta(name, t, f32, (B, Sq, H))
        elif name in ("out", "dout", "out_swa", "out_sparse", "out_mix"):
            _meta(name, t, dt, (B, Sq, H, Dv))
        elif name in ("lse", "lse_swa", "lse_sparse", "dlse"):
            _meta(name, t, f32, (B, Sq, H))
        elif name in ("block_logit", "block_prob"):
            _meta(name, t, f32, (B, Sq, hs_num_blocks(prob)))
        elif name == "block_idx":
            _meta(name, t, i32, (B, Sq, k) if k is not None else None)
        elif name == "dq":
            _meta(name, t, f32, (B, Sq, H, Dk))
        elif name == "dkv":
            _meta(name, t, f32, (B, Skv, Dk))
        elif name != "ws":  # pragma: no cover - a caller passed an unknown role
            raise AssertionError(name)
    for name, t in tensors.items():
        _dev(name, t)


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI).
# ---------------------------------------------------------------------------
def hs_num_blocks(prob: Problem) -> int:
    nb = load_library().hs_num_blocks(prob.ref)
    if nb < 0:
        _check(nb)
    return nb


def hs_workspace_size(prob: Problem, op: int, top_k: int = 0, window: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().hs_workspace_size(prob.ref, op, top_k, window, ctypes.byref(n)))
    return n.value


def hs_block_score_fwd(prob, q, kv, sink, out, lse, block_logit, ws=None, stream=None):
    _check_io(prob, q=q, kv=kv, sink=sink, out=out, lse=lse, block_logit=block_logit, ws=ws)
    _check(load_library().hs_block_score_fwd(
        prob.ref, _ptr(q), _ptr(kv), _ptr(sink), _ptr(out), _ptr(lse), _ptr(block_logit),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def hs_topk_blocks(prob, block_logit, top_k, block_idx, stream=None):
    _check_io(prob, block_logit=block_logit, block_idx=block_idx, _top_k=int(top_k))
    _check(load_library().hs_topk_blocks(prob.ref, _ptr(block_logit), int(top_k),
                                         _ptr(block_idx), _stream(stream)))


def hs_block_score_topk_fwd(prob, q, kv, sink, top_k, out, lse, block_logit, block_idx, ws=None,
                            stream=None, block_prob=None):
    _check_io(prob, q=q, kv=kv, sink=sink, out=out, lse=lse, block_logit=block_logit,
              block_idx=block_idx, block_prob=block_prob, ws=ws, _top_k=int(top_k))
    _check(load_library().hs_block_score_topk_fwd(
        prob.ref, _ptr(q), _ptr(kv), _ptr(sink), int(top_k), _ptr(out), _ptr(lse),
        _ptr(block_logit), _ptr(block_idx), _ptr(block_prob), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def hs_block_score_topk_fwd_noalloc(prob, q, kv, sink, top_k, out, lse, block_logit, block_idx,
                                    stream=None, block_prob=None):
    _check_io(prob, q=q, kv=kv, sink=sink, out=out, lse=lse, block_logit=block_logit,
              block_idx=block_idx, block_prob=block_prob, _top_k=int(top_k))
    _check(load_library().hs_block_score_topk_fwd_noalloc(
        prob.ref, _ptr(q), _ptr(kv), _ptr(sink), int(top_k), _ptr(out), _ptr(lse),
        _ptr(block_logit), _ptr(block_idx), _ptr(block_prob), _stream(stream)))


def hs_sparse_gather_fwd(prob, q, kv, sink, block_idx, top_k, out, lse, ws=None, stream=None):
    _check_io(prob, q=q, kv=kv, sink=sink, block_idx=block_idx, out=out, lse=lse, ws=ws,
              _top_k=int(top_k))
    _check(load_library().hs_sparse_gather_fwd(
        prob.ref, _ptr(q), _ptr(kv), _ptr(sink), _ptr(block_idx), int(top_k), _ptr(out),
        _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def hs_swa_fwd(prob, q, kv, sink, window, out, lse, ws=None, stream=None):
    _check_io(prob, q=q, kv=kv, sink=sink, out=out, lse=lse, ws=ws)
    _check(load_library().hs_swa_fwd(
        prob.ref, _ptr(q), _ptr(kv), _ptr(sink), int(window), _ptr(out), _ptr(lse), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def hs_swa_sparse_fwd(prob, q, kv, sink, window, block_idx, top_k, out_swa, lse_swa, out_sparse,
                      lse_sparse, ws=None, stream=None, gate_swa=None, gate_sparse=None,
                      out_mix=None):
    _check_io(prob, q=q, kv=kv, sink=sink, block_idx=block_idx, out_swa=out_swa, lse_swa=lse_swa,
              out_sparse=out_sparse, lse_sparse=lse_sparse, gate_swa=gate_swa,
              gate_sparse=gate_sparse, out_mix=out_mix, ws=ws, _top_k=int(top_k))
    _check(load_library().hs_swa_sparse_fwd(
        prob.ref, _ptr(q), _ptr(kv), _ptr(sink), int(window), _ptr(block_idx), int(top_k),
        _ptr(out_swa), _ptr(lse_swa), _ptr(out_sparse), _ptr(lse_sparse), _ptr(gate_swa),
        _ptr(gate_sparse), _ptr(out_mix), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def _nbytes(ws) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def hs_block_score_bwd(prob, q, kv, sink, out, lse, dout, dq, dkv, dsink, ws, stream=None,
                       dlse=None):
    _check_io(prob, q=q, kv=kv, sink=sink, out=out, lse=lse, dout=dout, dlse=dlse, dq=dq,
              dkv=dkv, dsink=dsink, ws=ws)
    _check(load_library().hs_block_score_bwd(
        prob.ref, _ptr(q), _ptr(kv), _ptr(sink), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dlse),
        _ptr(dq), _ptr(dkv), _ptr(dsink), _ptr(ws), _nbytes(ws), _stream(stream)))


def hs_sparse_gather_bwd(prob, q, kv, sink, block_idx, top_k, out, lse, dout, dq, dkv, dsink,
                         ws, stream=None, dlse=None):
    _check_io(prob, q=q, kv=kv, sink=sink, block_idx=block_idx, out=out, lse=lse, dout=dout,
              dlse=dlse, dq=dq, dkv=dkv, dsink=dsink, ws=ws, _top_k=int(top_k))
    _check(load_library().hs_sparse_gather_bwd(
        prob.ref, _ptr(q), _ptr(kv), _ptr(sink), _ptr(block_idx), int(top_k), _ptr(out),
        _ptr(lse), _ptr(dout), _ptr(dlse), _ptr(dq), _ptr(dkv), _ptr(dsink), _ptr(ws),
        _nbytes(ws), _stream(stream)))


def hs_swa_bwd(prob, q, kv, sink, window, out, lse, dout, dq, dkv, dsink, ws, stream=None,
               dlse=None):
    _check_io(prob, q=q, kv=kv, sink=sink, out=out, lse=lse, dout=dout, dlse=dlse, dq=dq,
              dkv=dkv, dsink=dsink, ws=ws)
    _check(load_library().hs_swa_bwd(
        prob.ref, _ptr(q), _ptr(kv), _ptr(sink), int(window), _ptr(out), _ptr(lse), _ptr(dout),
        _ptr(dlse), _ptr(dq), _ptr(dkv), _ptr(dsink), _ptr(ws), _nbytes(ws), _stream(stream)))


# ---------------------------------------------------------------------------
# Convenience wrappers: allocate outputs with PyTorch, then call the above.
# ---------------------------------------------------------------------------
def _torch_dtype(prob):
    import torch
    return torch.bfloat16 if prob.dtype == "bf16" else torch.float32


def _workspace(prob, op, top_k=0, window=0):
    import torch
    n = hs_workspace_size(prob, op, top_k, window)
    return torch.empty(max(1, (n + 3) // 4), dtype=torch.float32, device="cuda") if n else None


def block_score(prob, q, kv, sink=None, stream=None):
    import torch
    out = torch.empty((prob.B, prob.Sq, prob.H, prob.Dv), dtype=_torch_dtype(prob), device=q.device)
    lse = torch.empty((prob.B, prob.Sq, prob.H), dtype=torch.float32, device=q.device)
    bl = torch.empty((prob.B, prob.Sq, hs_num_blocks(prob)), dtype=torch.float32, device=q.device)
    hs_block_score_fwd(prob, q, kv, sink, out, lse, bl, _workspace(prob, HS_OP_BLOCK_SCORE), stream)
    return out, lse, bl


def block_score_topk(prob, q, kv, sink, top_k, stream=None, with_prob=False):
    """(out, lse, block_logit, block_idx[, block_prob]) of hs_block_score_topk_fwd;
    block_prob (the normalised block scores) when with_prob."""
    import torch
    out = torch.empty((prob.B, prob.Sq, prob.H, prob.Dv), dtype=_torch_dtype(prob), device=q.device)
    lse = torch.empty((prob.B, prob.Sq, prob.H), dtype=torch.float32, device=q.device)
    NB = hs_num_blocks(prob)
    bl = torch.empty((prob.B, prob.Sq, NB), dtype=torch.float32, device=q.device)
    idx = torch.empty((prob.B, prob.Sq, top_k), dtype=torch.int32, device=q.device)
    pr = torch.empty((prob.B, prob.Sq, NB), dtype=torch.float32, device=q.device) if with_prob else None
    hs_block_score_topk_fwd(prob, q, kv, sink, top_k, out, lse, bl, idx,
                            _workspace(prob, HS_OP_BLOCK_SCORE), stream, block_prob=pr)
    return (out, lse, bl, idx, pr) if with_prob else (out, lse, bl, idx)


def topk_blocks(prob, block_logit, top_k, stream=None):
    import torch
    idx = torch.empty((prob.B, prob.Sq, top_k), dtype=torch.int32, device=block_logit.device)
    hs_topk_blocks(prob, block_logit, top_k, idx, stream)
    return idx


def sparse_gather(prob, q, kv, sink, block_idx, top_k, stream=None):
    import torch
    out = torch.empty((prob.B, prob.Sq, prob.H, prob.Dv), dtype=_torch_dtype(prob), device=q.device)
    lse = torch.empty((prob.B, prob.Sq, prob.H), dtype=torch.float32, device=q.device)
    hs_sparse_gather_fwd(prob, q, kv, sink, block_idx, top_k, out, lse,
                         _workspace(prob, HS_OP_SPARSE_GATHER, top_k=top_k), stream)
    return out, lse


def swa(prob, q, kv, sink, window, stream=None):
    import torch
    out = torch.empty((prob.B, prob.Sq, prob.H, prob.Dv), dtype=_torch_dtype(prob), device=q.device)
    lse = torch.empty((prob.B, prob.Sq, prob.H), dtype=torch.float32, device=q.device)
    hs_swa_fwd(prob, q, kv, sink, window, out, lse, _workspace(prob, HS_OP_SWA, window=window),
               stream)
    return out, lse


def swa_sparse(prob, q, kv, sink, window, block_idx, top_k, stream=None, gate_swa=None,
               gate_sparse=None):
    """Both branches of a sliding-window layer over the shared latent KV and a
    given block selection: (out_swa, lse_swa, out_sparse, lse_sparse), equal
    to swa(...) and sparse_gather(...) for the same arguments; with the gates
    ([B, Sq, H] float32) also out_mix = gate_swa * out_swa + gate_sparse *
    out_sparse as a fifth result."""
    import torch
    shape_o = (prob.B, prob.Sq, prob.H, prob.Dv)
    shape_l = (prob.B, prob.Sq, prob.H)
    ow = torch.empty(shape_o, dtype=_torch_dtype(prob), device=q.device)
    lw = torch.empty(shape_l, dtype=torch.float32, device=q.device)
    og = torch.empty(shape_o, dtype=_torch_dtype(prob), device=q.device)
    lg = torch.empty(shape_l, dtype=torch.float32, device=q.device)
    om = None if gate_swa is None else torch.empty(shape_o, dtype=_torch_dtype(prob), device=q.device)
    hs_swa_sparse_fwd(prob, q, kv, sink, window, block_idx, top_k, ow, lw, og, lg,
                      _workspace(prob, HS_OP_SWA_SPARSE, top_k=top_k, window=window), stream,
                      gate_swa=gate_swa, gate_sparse=gate_sparse, out_mix=om)
    return (ow, lw, og, lg) if om is None else (ow, lw, og, lg, om)


def _grad_buffers(prob, q, sink):
    import torch
    dq = torch.empty((prob.B, prob.Sq, prob.H, prob.Dk), dtype=torch.float32, device=q.device)
    dkv = torch.empty((prob.B, prob.Skv, prob.Dk), dtype=torch.float32, device=q.device)
    dsink = None if sink is None else torch.empty((prob.H,), dtype=torch.float32, device=q.device)
    return dq, dkv, dsink


def _stored_ds_workspace(prob, small, large, store_ds, window=0):
    return _workspace(prob, large if store_ds else small, window=window)


def score_bwd_workspace(prob, store_ds=False):
    """Workspace of hs_block_score_bwd. store_ds True (opt-in): the larger one,
    in which the key-block pass stores the score gradients for dq (8 KB per
    causal (row, key block) pair: 69 GB for one 32768-token sequence);
    False: the smaller one, and dq recomputes them."""
    return _stored_ds_workspace(prob, HS_OP_BLOCK_SCORE_BWD, HS_OP_BLOCK_SCORE_BWD_STORE_DS,
                                store_ds)


def swa_bwd_workspace(prob, window, store_ds=False):
    """Workspace of hs_swa_bwd, chosen as for score_bwd_workspace (the
    stored form is 8 KB per row and per block a window can meet)."""
    return _stored_ds_workspace(prob, HS_OP_SWA_BWD, HS_OP_SWA_BWD_STORE_DS, store_ds, window)


def sparse_gather_bwd_workspace(prob, top_k, store_ds=False):
    """Workspace of hs_sparse_gather_bwd, chosen as for score_bwd_workspace
    (the stored form is 8 KB per row and per selection entry)."""
    return _workspace(prob, HS_OP_SPARSE_GATHER_BWD_STORE_DS if store_ds else HS_OP_SPARSE_GATHER_BWD,
                      top_k=top_k)


def block_score_bwd(prob, q, kv, sink, out, lse, dout, stream=None, store_ds=False, dlse=None):
    """Gradients (dq, dkv, dsink) of the causal attention of block_score;
    dsink is None without a sink. All float32. store_ds picks the workspace
    (score_bwd_workspace)."""
    dq, dkv, dsink = _grad_buffers(prob, q, sink)
    hs_block_score_bwd(prob, q, kv, sink, out, lse, dout, dq, dkv, dsink,
                       score_bwd_workspace(prob, store_ds), stream, dlse=dlse)
    return dq, dkv, dsink


def sparse_gather_bwd(prob, q, kv, sink, block_idx, top_k, out, lse, dout, stream=None, dlse=None,
                      store_ds=False):
    """Gradients (dq, dkv, dsink) of sparse_gather for the given selection.
    store_ds picks the workspace (sparse_gather_bwd_workspace)."""
    dq, dkv, dsink = _grad_buffers(prob, q, sink)
    hs_sparse_gather_bwd(prob, q, kv, sink, block_idx, top_k, out, lse, dout, dq, dkv, dsink,
                         sparse_gather_bwd_workspace(prob, top_k, store_ds), stream, dlse=dlse)
    return dq, dkv, dsink


def swa_bwd(prob, q, kv, sink, window, out, lse, dout, stream=None, store_ds=False, dlse=None):
    """Gradients (dq, dkv, dsink) of swa. store_ds picks the workspace
    (swa_bwd_workspace)."""
    dq, dkv, dsink = _grad_buffers(prob, q, sink)
    hs_swa_bwd(prob, q, kv, sink, window, out, lse, dout, dq, dkv, dsink,
               swa_bwd_workspace(prob, window, store_ds), stream, dlse=dlse)
    return dq, dkv, dsink
