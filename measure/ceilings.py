"""The benchmark's ceiling probes (``measure/csrc/ceilings.hip``): a plain streaming read (the
achievable HBM read rate), register-only MFMA bursts (the matrix-core rates the GPU sustains
under its power limit with changing operands) and a plain copy of known size (the reference that
scales the hardware byte counters of a profiling run). None of them is part of the layer."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "ceilings.hip")
LIB = os.path.join(HERE, "libmoe_measure.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

_lib = None


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-o", tmp, SRC], stderr=subprocess.DEVNULL)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError("measurement library not built (run __graft_entry__.build())")
        _lib = ctypes.CDLL(LIB)
        i32, i64, p = ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p
        _lib.measure_copy.argtypes = [p, p, i64, p]
        _lib.measure_stream_read.argtypes = [p, i64, p, p]
        _lib.measure_mfma_burst.argtypes = [i32, i32, i32, p, p]
    return _lib


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _chk(rc, what):
    if rc != 0:
        raise RuntimeError("measure %s failed (%d)" % (what, rc))


def copy(src, dst):
    """dst <- src with one plain copy kernel (the known-size reference for byte counters)."""
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= n
    _chk(lib().measure_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, _stream()), "copy")


def mfma_burst(kind: int, iters: int, blocks: int, sink) -> float:
    """One MFMA burst (kind 0: bf16 16x16x32, kind 1: fp4 x fp8, kind 2: fp8 x fp8 16x16x128, kind 3:
    int8 16x16x64); returns its FLOPs (OPs)."""
    _chk(lib().measure_mfma_burst(kind, iters, blocks, ctypes.c_void_p(sink.data_ptr()), _stream()), "mfma_burst")
    return float(blocks) * 8 * iters * 16 * {0: 16384, 1: 65536, 2: 65536, 3: 32768}[kind]


def stream_read(src, sink):
    """One plain streaming read of all of src (the achievable HBM read rate)."""
    n = src.numel() * src.element_size()
    _chk(lib().measure_stream_read(ctypes.c_void_p(src.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()), _stream()),
         "stream_read")
