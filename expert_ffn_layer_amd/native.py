"""ctypes binding of ``libmoe.so`` with the C ABI's names (include/moe.h).

Argument marshalling only: torch tensors supply device pointers, the current torch stream is
passed as the HIP stream, and non-OK statuses become ``MoeError``. Every step of the layer
runs in the library's HIP kernels. There is no fallback: if the library is not built, loading
fails loudly.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

DTYPE = {"f32": 0, "bf16": 1, "fp8": 2, "mxfp4": 3, "mxfp4a8": 4, "mxfp8a8": 5, "int8": 6}
PATH = {"auto": 0, "decode": 1, "prefill": 2}
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}
EXPORTS = ("moe_status_string", "moe_last_error", "moe_pack_size", "moe_pack", "moe_workspace_size",
           "moe_route", "moe_route_hash", "moe_permute", "moe_route_permute", "moe_grouped_ffn", "moe_combine",
           "moe_layer_forward", "moe_layer_forward_noalloc", "moe_layer_forward_hash", "moe_layer_forward_timed",
           "moe_quantize_mxfp8", "moe_quantize_int8", "moe_logical_workspace_size", "moe_layer_forward_logical")
# the library's own scratch, the workspace of moe_layer_forward_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20
TIMED_EVENTS = 7


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), detail))
        self.status = status


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32),
                ("act", ctypes.c_int), ("w_routed", ctypes.c_int), ("w_shared", ctypes.c_int),
                ("path", ctypes.c_int)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_scale", ctypes.c_void_p), ("up_scale", ctypes.c_void_p),
                ("down_scale", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built: run __graft_entry__.build() "
                               "(expert_ffn_layer_amd/build.py) first")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        PS, PW = ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights)
        lib.moe_status_string.restype = ctypes.c_char_p
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_last_error.restype = ctypes.c_char_p
        lib.moe_last_error.argtypes = []
        lib.moe_pack_size.argtypes = [ctypes.c_int, I32, I32, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
        lib.moe_pack.argtypes = [ctypes.c_int, I32, I32, I32, P, P, P, P, P]
        lib.moe_workspace_size.argtypes = [PS, ctypes.POINTER(SZ)]
        lib.moe_route.argtypes = [PS, P, P, P, P, P, P, SZ, P]
        lib.moe_route_hash.argtypes = [PS, P, P, P, P, P, I32, P, P, P, SZ, P]
        lib.moe_permute.argtypes = [PS, P, P, P, P, P, SZ, P]
        lib.moe_route_permute.argtypes = [PS, P, P, P, P, P, P, P, P, P, SZ, P]
        lib.moe_grouped_ffn.argtypes = [PS, P, P, P, PW, PW, P, P, P, SZ, P]
        lib.moe_combine.argtypes = [PS, P, P, P, P, P, P]
        lib.moe_layer_forward.argtypes = [PS, P, P, P, PW, PW, P, P, P, P, SZ, P]
        lib.moe_layer_forward_noalloc.argtypes = [PS, P, P, P, PW, PW, P, P, P, P]
        lib.moe_layer_forward_hash.argtypes = [PS, P, P, P, P, P, I32, PW, PW, P, P, P, P, SZ, P]
        lib.moe_layer_forward_timed.argtypes = [PS, P, P, P, PW, PW, P, P, P, P, SZ, P,
                                                ctypes.POINTER(ctypes.c_void_p)]
        lib.moe_quantize_mxfp8.argtypes = [P, I32, I32, P, P, P]
        lib.moe_quantize_int8.argtypes = [P, I32, I32, P, P, P]
        lib.moe_logical_workspace_size.argtypes = [PS, ctypes.POINTER(SZ)]
        lib.moe_layer_forward_logical.argtypes = [PS, P, P, P, PW, PW, P, P, P, P, SZ, P]
        for name in EXPORTS[2:]:
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != 0:
        raise MoeError(rc, load().moe_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_shape(T, H, E, k, I, I_shared=0, act="bf16", w_routed="bf16", w_shared="bf16", path="auto") -> MoeShape:
    return MoeShape(T, H, E, k, I, I_shared, DTYPE[act], DTYPE[w_routed], DTYPE[w_shared], PATH[path])


def shape_from_spec(spec, T=None, path="auto") -> MoeShape:
    return make_shape(spec.T if T is None else T, spec.H, spec.E, spec.k, spec.I,
                      spec.I if spec.shared else 0, spec.act, spec.w_routed, spec.w_shared, path)


def weights(d: dict | None):
    if d is None:
        return None
    return MoeWeights(*[None if d.get(n) is None else d[n].data_ptr()
                        for n in ("gate", "up", "down", "gate_scale", "up_scale", "down_scale")])


def moe_pack_size(fmt: str, count: int, K: int, N: int):
    b, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().moe_pack_size(DTYPE[fmt], count, K, N, ctypes.byref(b), ctypes.byref(s)))
    return b.value, s.value


def moe_pack(fmt, count, K, N, w, scale, packed, packed_scale, stream=None):
    _check(load().moe_pack(DTYPE[fmt], count, K, N, _p(w), _p(scale), _p(packed), _p(packed_scale),
                           _stream(stream)))


def moe_workspace_size(shape: MoeShape) -> int:
    b = ctypes.c_size_t()
    _check(load().moe_workspace_size(ctypes.byref(shape), ctypes.byref(b)))
    return b.value


def moe_logical_workspace_size(shape: MoeShape) -> int:
    b = ctypes.c_size_t()
    _check(load().moe_logical_workspace_size(ctypes.byref(shape), ctypes.byref(b)))
    return b.value


def moe_layer_forward_logical(shape, x, Wr, bias, routed: dict, shared: dict | None, y, topk_idx=None,
                              topk_w=None, ws=None, stream=None):
    """Weights in the logical row-major layout (moe_pack's source layout), packed into ws each call."""
    r, s = weights(routed), weights(shared)
    _check(load().moe_layer_forward_logical(ctypes.byref(shape), _p(x), _p(Wr), _p(bias), ctypes.byref(r),
                                            None if s is None else ctypes.byref(s), _p(y), _p(topk_idx),
                                            _p(topk_w), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                            _stream(stream)))


def moe_route(shape, x, Wr_packed, bias, topk_idx, topk_w, ws, stream=None):
    _check(load().moe_route(ctypes.byref(shape), _p(x), _p(Wr_packed), _p(bias), _p(topk_idx), _p(topk_w),
                            _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_route_hash(shape, x, Wr_packed, bias, token_ids, hash_table, topk_idx, topk_w, ws, stream=None):
    _check(load().moe_route_hash(ctypes.byref(shape), _p(x), _p(Wr_packed), _p(bias), _p(token_ids),
                                 _p(hash_table), hash_table.shape[0], _p(topk_idx), _p(topk_w), _p(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_permute(shape, topk_idx, expert_offsets, slot_token, pair_slot, ws, stream=None):
    _check(load().moe_permute(ctypes.byref(shape), _p(topk_idx), _p(expert_offsets), _p(slot_token),
                              _p(pair_slot), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream)))


def moe_route_permute(shape, x, Wr_packed, bias, topk_idx, topk_w, expert_offsets, slot_token, pair_slot, ws,
                      stream=None):
    _check(load().moe_route_permute(ctypes.byref(shape), _p(x), _p(Wr_packed), _p(bias), _p(topk_idx), _p(topk_w),
                                    _p(expert_offsets), _p(slot_token), _p(pair_slot), _p(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_grouped_ffn(shape, x, expert_offsets, slot_token, routed: dict, shared: dict | None, y_perm, y_shared,
                    ws, stream=None):
    r, s = weights(routed), weights(shared)
    _check(load().moe_grouped_ffn(ctypes.byref(shape), _p(x), _p(expert_offsets), _p(slot_token),
                                  ctypes.byref(r), None if s is None else ctypes.byref(s), _p(y_perm),
                                  _p(y_shared), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(stream)))


def moe_combine(shape, y_perm, pair_slot, topk_w, y_shared, y, stream=None):
    _check(load().moe_combine(ctypes.byref(shape), _p(y_perm), _p(pair_slot), _p(topk_w), _p(y_shared), _p(y),
                              _stream(stream)))


def moe_layer_forward(shape, x, Wr_packed, bias, routed: dict, shared: dict | None, y, topk_idx=None,
                      topk_w=None, ws=None, stream=None):
    r, s = weights(routed), weights(shared)
    _check(load().moe_layer_forward(ctypes.byref(shape), _p(x), _p(Wr_packed), _p(bias), ctypes.byref(r),
                                    None if s is None else ctypes.byref(s), _p(y), _p(topk_idx), _p(topk_w),
                                    _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream)))


def moe_layer_forward_noalloc(shape, x, Wr_packed, bias, routed: dict, shared: dict | None, y, topk_idx=None,
                              topk_w=None, stream=None):
    r, s = weights(routed), weights(shared)
    _check(load().moe_layer_forward_noalloc(ctypes.byref(shape), _p(x), _p(Wr_packed), _p(bias), ctypes.byref(r),
                                            None if s is None else ctypes.byref(s), _p(y), _p(topk_idx), _p(topk_w),
                                            _stream(stream)))


def moe_layer_forward_hash(shape, x, Wr_packed, bias, token_ids, hash_table, routed: dict, shared: dict | None, y,
                           topk_idx=None, topk_w=None, ws=None, stream=None):
    r, s = weights(routed), weights(shared)
    _check(load().moe_layer_forward_hash(ctypes.byref(shape), _p(x), _p(Wr_packed), _p(bias), _p(token_ids),
                                         _p(hash_table), hash_table.shape[0], ctypes.byref(r),
                                         None if s is None else ctypes.byref(s), _p(y), _p(topk_idx), _p(topk_w),
                                         _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                         _stream(stream)))


def moe_layer_forward_timed(shape, x, Wr_packed, bias, routed: dict, shared: dict | None, y, events,
                            topk_idx=None, topk_w=None, ws=None, stream=None):
    """``events``: TIMED_EVENTS torch.cuda.Event(enable_timing=True) objects."""
    r, s = weights(routed), weights(shared)
    arr = (ctypes.c_void_p * TIMED_EVENTS)(*[e.cuda_event for e in events])
    _check(load().moe_layer_forward_timed(ctypes.byref(shape), _p(x), _p(Wr_packed), _p(bias), ctypes.byref(r),
                                          None if s is None else ctypes.byref(s), _p(y), _p(topk_idx),
                                          _p(topk_w), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                          _stream(stream), arr))


def moe_quantize_mxfp8(x, codes, scales, stream=None):
    """x bf16 [rows, K] -> codes uint8 [rows, K], scales uint8 [rows, K / 32] (e8m0)."""
    rows, K = (x.shape[0], x.shape[1]) if x is not None else (0, 32)
    _check(load().moe_quantize_mxfp8(_p(x), rows, K, _p(codes), _p(scales), _stream(stream)))


def moe_quantize_int8(x, codes, scales, stream=None):
    """x bf16 [rows, K] -> codes int8 [rows, K], scales float32 [rows]."""
    rows, K = (x.shape[0], x.shape[1]) if x is not None else (0, 8)
    _check(load().moe_quantize_int8(_p(x), rows, K, _p(codes), _p(scales), _stream(stream)))
