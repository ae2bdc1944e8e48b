"""GPU fills of the seeded inputs (``inputgen/csrc/gen.hip``), bit-identical to the numpy
definitions in ``inputgen.philox`` / ``inputgen.layers``, so the multi-GB expert weights of the
full-size layers are generated on the device in milliseconds instead of minutes on the host.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import layers as L
from . import philox as px

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "gen.hip")
LIB = os.path.join(HERE, "libmoe_inputgen.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

_lib = None
_tables = {}


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
            raise RuntimeError("inputgen GPU library not built (run __graft_entry__.build())")
        _lib = ctypes.CDLL(LIB)
        u32, i32, i64, f32, p = (ctypes.c_uint32, ctypes.c_int, ctypes.c_longlong, ctypes.c_float,
                                 ctypes.c_void_p)
        _lib.gen_fill_dense.argtypes = [p, i32, u32, u32, u32, i32, i64, i64, f32, p, p, p]
        _lib.gen_fill_fp8.argtypes = [p, p, u32, u32, u32, i32, i32, i32, f32, p, p, p]
        _lib.gen_fill_mxfp4.argtypes = [p, p, u32, u32, u32, i32, i32, i32, f32, p, p, p]
        _lib.gen_fill_mxfp8.argtypes = [p, p, u32, u32, u32, i32, i32, i32, f32, p, p, p]
        _lib.gen_fill_int8.argtypes = [p, p, u32, u32, u32, i32, i32, i32, f32, p, p, p]
    return _lib


def _tabs(device):
    import torch
    key = str(device)
    if key not in _tables:
        _tables[key] = (torch.from_numpy(px.NORMAL_TABLE.copy()).to(device),
                        torch.from_numpy(px.NORMAL_TAIL.copy()).to(device))
    return _tables[key]


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _chk(rc, what):
    if rc != 0:
        raise RuntimeError("inputgen %s failed (%d)" % (what, rc))


def fill_dense(out, fmt: str, seed: int, tid: int, stream0: int, count: int, n: int, start: int = 0,
               fan_in: int | None = None):
    """out[count * n] <- N(0, 1/fan_in) values of streams stream0.. (values start..start+n)."""
    T, TT = _tabs(out.device)
    s = 1.0 if fan_in is None else L.sigma(fan_in)
    _chk(lib().gen_fill_dense(out.data_ptr(), 0 if fmt == "f32" else 1, seed, tid, stream0, count, n, start,
                              s, T.data_ptr(), TT.data_ptr(), _stream()), "dense")


def alloc_matrices(fmt: str, count: int, K: int, N: int, device):
    """Stored-format device tensors for `count` K x N matrices: (codes, scales or None)."""
    fmt = "mxfp4" if fmt == "mxfp4a8" else fmt  # W4A8 stores MXFP4 weights
    import torch
    if fmt == "f32":
        return torch.empty((count, K, N), dtype=torch.float32, device=device), None
    if fmt == "bf16":
        return torch.empty((count, K, N), dtype=torch.int16, device=device), None
    if fmt == "fp8":
        return (torch.empty((count, K, N), dtype=torch.uint8, device=device),
                torch.empty((count, K // 128, N // 128), dtype=torch.float32, device=device))
    if fmt == "mxfp4":
        return (torch.empty((count, K, N // 2), dtype=torch.uint8, device=device),
                torch.empty((count, K // 32, N), dtype=torch.uint8, device=device))
    if fmt == "mxfp8a8":
        return (torch.empty((count, K, N), dtype=torch.uint8, device=device),
                torch.empty((count, K // 32, N), dtype=torch.uint8, device=device))
    if fmt == "int8":
        return (torch.empty((count, K, N), dtype=torch.int8, device=device),
                torch.empty((count, N), dtype=torch.float32, device=device))
    raise ValueError(fmt)


def fill_matrices(codes, scales, fmt: str, seed: int, tid: int, stream0: int, K: int, N: int, fan_in: int):
    fmt = "mxfp4" if fmt == "mxfp4a8" else fmt  # W4A8 stores MXFP4 weights
    count = codes.shape[0]
    T, TT = _tabs(codes.device)
    s = L.sigma(fan_in)
    st = _stream()
    if fmt in ("f32", "bf16"):
        _chk(lib().gen_fill_dense(codes.data_ptr(), 0 if fmt == "f32" else 1, seed, tid, stream0, count, K * N, 0,
                                  s, T.data_ptr(), TT.data_ptr(), st), "dense matrix")
    elif fmt == "fp8":
        _chk(lib().gen_fill_fp8(codes.data_ptr(), scales.data_ptr(), seed, tid, stream0, count, K, N, s,
                                T.data_ptr(), TT.data_ptr(), st), "fp8")
    elif fmt == "int8":
        _chk(lib().gen_fill_int8(codes.data_ptr(), scales.data_ptr(), seed, tid, stream0, count, K, N, s,
                                 T.data_ptr(), TT.data_ptr(), st), "int8")
    elif fmt == "mxfp8a8":
        _chk(lib().gen_fill_mxfp8(codes.data_ptr(), scales.data_ptr(), seed, tid, stream0, count, K, N, s,
                                  T.data_ptr(), TT.data_ptr(), st), "mxfp8")
    else:
        _chk(lib().gen_fill_mxfp4(codes.data_ptr(), scales.data_ptr(), seed, tid, stream0, count, K, N, s,
                                  T.data_ptr(), TT.data_ptr(), st), "mxfp4")


def expert_weights(spec: L.LayerSpec, kind: str, device, count: int | None = None, first: int = 0) -> dict:
    """Stored weights of `count` routed experts from `first` (or the shared one), on the device."""
    tids = L.TID_ROUTED if kind == "routed" else L.TID_SHARED
    fmt = spec.w_routed if kind == "routed" else spec.w_shared
    count = (spec.E if kind == "routed" else 1) if count is None else count
    H, I = spec.H, spec.I
    out = {}
    for name, (K, N, fan) in (("gate", (H, I, H)), ("up", (H, I, H)), ("down", (I, H, I))):
        c, s = alloc_matrices(fmt, count, K, N, device)
        fill_matrices(c, s, fmt, spec.seed, tids[name], first, K, N, fan)
        out[name], out[name + "_scale"] = c, s
    return out


def activations_attempt0(spec: L.LayerSpec, device):
    """x[T, H] of draw attempt 0, in the act format, on the device."""
    import torch
    dt = torch.float32 if spec.act == "f32" else torch.int16
    x = torch.empty((spec.T, spec.H), dtype=dt, device=device)
    fill_dense(x, spec.act, spec.seed, L.TID_X, 0, 1, spec.T * spec.H)
    return x


def to_numpy_stored(t) -> np.ndarray:
    """Device tensor of a stored format -> numpy array with the dtype the host code uses."""
    import torch
    a = t.detach().cpu()
    if a.dtype == torch.int16:
        return a.numpy().view(np.uint16)
    return a.numpy()


def layer_on_device(spec: L.LayerSpec, device="cuda"):
    """The whole synthetic layer on the device (stored formats), plus host copies of the router
    inputs. x of attempt 0 is drawn on the device and the margin rule applied on the host."""
    import torch
    Wr = L.router_matrix(spec)
    bias = L.zipf_bias(spec, Wr) if spec.router == "zipf" else None
    x0 = to_numpy_stored(activations_attempt0(spec, device))
    x, attempts = L.activations(spec, Wr, bias, x0=x0)
    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    out = {
        "spec": spec, "x_host": x, "Wr_host": Wr, "bias_host": bias, "attempts": attempts,
        "x": dev(x), "Wr": dev(Wr), "bias": None if bias is None else dev(bias),
        "routed": expert_weights(spec, "routed", device),
        "shared": expert_weights(spec, "shared", device) if spec.shared else None,
    }
    return out
