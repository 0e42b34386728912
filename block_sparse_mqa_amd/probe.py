"""ctypes binding of libhsprobe.so (include/hs_probe.h): the dense bf16 MFMA
loop and the streaming copy that measure the attainable rooflines of the GPU.
Argument marshalling only; the library must have been built."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(HERE, "libhsprobe.so")
EXPORTS = ("hs_probe_mfma_bf16", "hs_probe_mfma_flops", "hs_probe_copy")

_lib = None


def load_probe_library(path: str = PROBE_LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_sparse_mqa_amd.build`")
    lib = ctypes.CDLL(path)
    lib.hs_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.hs_probe_mfma_bf16.restype = ctypes.c_int
    lib.hs_probe_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.hs_probe_mfma_flops.restype = ctypes.c_double
    lib.hs_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.hs_probe_copy.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, what: str) -> None:
    if rc == -1:
        raise ValueError(f"{what}: invalid argument")
    if rc != 0:
        raise RuntimeError(f"{what}: HIP error (status {rc})")


def _stream_ptr(stream) -> int | None:
    return None if stream is None else int(stream.cuda_stream)


def hs_probe_mfma_bf16(workgroups: int, iters: int, out, clocks=None, stream=None) -> None:
    """`out`: float32 device tensor of at least workgroups * 256 elements;
    `clocks`: int64 device tensor of 2 elements, or None."""
    if out.numel() < workgroups * 256:
        raise ValueError("out is smaller than workgroups * 256 floats")
    if clocks is not None and clocks.numel() < 2:
        raise ValueError("clocks needs 2 elements")
    _check(load_probe_library().hs_probe_mfma_bf16(
        workgroups, iters, out.data_ptr(), None if clocks is None else clocks.data_ptr(),
        _stream_ptr(stream)), "hs_probe_mfma_bf16")


def hs_probe_mfma_flops(workgroups: int, iters: int) -> float:
    return float(load_probe_library().hs_probe_mfma_flops(workgroups, iters))


def hs_probe_copy(src, dst, nbytes: int, stream=None) -> None:
    """Copy `nbytes` from device tensor `src` to device tensor `dst`."""
    if src.numel() * src.element_size() < nbytes or dst.numel() * dst.element_size() < nbytes:
        raise ValueError("tensors are smaller than nbytes")
    _check(load_probe_library().hs_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                              _stream_ptr(stream)), "hs_probe_copy")
