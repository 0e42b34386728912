"""Build the HIP library libhysparse.so for gfx950, in-tree.

Usage: python -m block_sparse_mqa_amd.build  (or build() from Python).
Every call compiles from source; nothing is cached.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libhysparse.so")
# Roofline probes (dense MFMA loop, copy): a separate library, not the method's ABI.
PROBE_LIB = os.path.join(HERE, "libhsprobe.so")
PROBE_SOURCES = ["hs_probe.hip"]
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["hs_abi.hip", "hs_attn_bf16.hip", "hs_attn_f32.hip", "hs_topk.hip", "hs_bwd.hip",
           "hs_bwd_plan.hip", "hs_mix.hip"]
# Per-source extra flags. The bf16 engine keeps its MFMA accumulators in
# VGPRs so that the O rescale and epilogue need no AGPR<->VGPR copies; Q and
# other long-lived operands then go to AGPRs, which MFMA reads directly. Its
# inputs are finite by contract, so max reductions need no NaN quieting
# (-fno-honor-nans drops a canonicalising v_max per reduction step).
EXTRA = {"hs_attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
         "hs_bwd.hip": ["-fno-honor-nans"],
         "hs_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-FP32 instructions are kept out of every kernel (plain fp32 code only).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-result"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(6, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
