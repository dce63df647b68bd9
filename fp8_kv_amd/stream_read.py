"""ctypes binding of libstream_read.so: the plain streaming-read kernel the
benchmark uses to measure the read rate the KV bytes can reach on this
device (every byte read once with 16-byte loads, non-temporal or ordinary,
no indirection, no arithmetic).  A measurement aid beside the
attention path, not part of it.  No fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstream_read.so")
MAX_BLOCKS = 1 << 16
_ERRORS = {-1: "a required pointer is NULL", -2: "size out of range",
           -3: "pointer not 16-byte aligned", -4: "launch failed"}
_LIB = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} is not built; run `python -m fp8_kv_amd.build`")
        # torch ships its own HIP runtime: load it first so that this library
        # binds to that same runtime (and sees the tensors torch allocates)
        # instead of starting a second one from the system ROCm.
        import torch  # noqa: F401

        lib = ctypes.CDLL(path)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.stream_read.restype = ctypes.c_int
        lib.stream_read.argtypes = [vp, sz, vp, sz, ctypes.c_int32, ctypes.c_int32, vp, vp]
        lib.clock_probe.restype = ctypes.c_int
        lib.clock_probe.argtypes = [vp, ctypes.c_int32, vp]
        _LIB = lib
    return _LIB


def stream_read(a, b, sink, blocks: int, nontemporal: bool = True, stream=None) -> None:
    """Reads every byte of the device tensors a and b (b may be None) once;
    sink (uint8 [16*blocks] or any 16-byte aligned tensor of that size)
    receives one 16-byte XOR of the words each workgroup read.  nontemporal
    selects the load hint the decode kernels use (False: ordinary loads)."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    a_bytes = a.numel() * a.element_size()
    b_bytes = 0 if b is None else b.numel() * b.element_size()
    rc = load().stream_read(a.data_ptr(), a_bytes, None if b is None else b.data_ptr(), b_bytes,
                            blocks, int(nontemporal), sink.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"stream_read: {_ERRORS.get(rc, rc)} (code {rc})")


def clock_mhz(buf, ticks: int = 2000, stream=None) -> float:
    """Shader clock in MHz over a spin of `ticks` 10-ns real-time ticks, run
    on `stream` (synchronises it).  buf: int64 device tensor of at least 2
    elements (scratch for the two counters)."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    rc = load().clock_probe(buf.data_ptr(), int(ticks), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"clock_probe: {_ERRORS.get(rc, rc)} (code {rc})")
    stream.synchronize()
    real, shader = buf[:2].tolist()
    return 100.0 * shader / max(real, 1)
