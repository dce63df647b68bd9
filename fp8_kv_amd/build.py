"""Build libpgqa.so (gfx950) in-tree with hipcc, and beside it
libstream_read.so, the plain streaming-read kernel the benchmark measures the
attainable read rate with.

Usage: python -m fp8_kv_amd.build   (or __graft_entry__.build()).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpgqa.so")
SOURCES = ["pgqa_api.hip", "pgqa_kernels.hip", "qsa_api.hip", "qsa_page4.hip", "qsa_topk.hip",
           "sampler_api.hip", "sampler_mask.hip"]
STREAM_LIB = os.path.join(PKG, "libstream_read.so")
STREAM_SOURCES = ["stream_read.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # Packed fp32 VALU ops are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Keep MFMA accumulators in ordinary VGPRs: the online softmax rescales
    # them with vector ALU ops every tile.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # Leading scalar kernel arguments arrive preloaded in SGPRs.
    "-mllvm", "-amdgpu-kernarg-preload-count=10",
]


def _hipcc(lib: str, sources: list[str], verbose: bool, extra: tuple[str, ...]) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns about the device-only feature flag; drop that noise.
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, extra: tuple[str, ...] = ()) -> str:
    """Compiles both libraries; returns the path of libpgqa.so."""
    _hipcc(STREAM_LIB, STREAM_SOURCES, verbose, extra)
    return _hipcc(LIB, SOURCES, verbose, extra)


if __name__ == "__main__":
    print(build(verbose=True))
