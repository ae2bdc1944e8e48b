"""Python access to the CPU oracle (``oracle/moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()`` and by the
CPU-baseline leg of ``bench.py``; the library never imports it. It only marshals numpy arrays
into the C functions; every step of the computation is in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
# MOE_ORACLE_SANITIZE=1 selects a separate build with AddressSanitizer and UndefinedBehaviorSanitizer
# (CPU only; any finding aborts), loaded in a process that preloads the sanitizer runtimes
SANITIZE = os.environ.get("MOE_ORACLE_SANITIZE") == "1"
LIB = os.path.join(HERE, "libmoe_oracle_san.so" if SANITIZE else "libmoe_oracle.so")
CFLAGS = ["-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall"]
SAN_CFLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall"]

FMT = {"f32": 0, "bf16": 1, "fp8": 2, "mxfp4": 3, "mxfp4a8": 4, "mxfp8a8": 5, "int8": 6}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP; the sanitizer build when SANITIZE)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *(SAN_CFLAGS if SANITIZE else CFLAGS), "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = ctypes.CDLL(LIB)
        d, i, p = ctypes.c_double, ctypes.c_int, ctypes.c_void_p
        _lib.oracle_decode_bf16.restype = d
        _lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        for name in ("oracle_decode_e4m3fn", "oracle_decode_e2m1", "oracle_decode_e8m0"):
            getattr(_lib, name).restype = d
            getattr(_lib, name).argtypes = [ctypes.c_uint8]
        _lib.oracle_decode_matrix.argtypes = [i, i, i, p, p, p]
        _lib.oracle_mxfp8_quantize.argtypes = [i, p, p, p]
        _lib.oracle_int8_quantize.argtypes = [i, p, p, p]
        _lib.oracle_row_matmul.argtypes = [i, i, i, p, p, p, p]
        _lib.oracle_route.argtypes = [i, i, i, i, i, p, p, p, p, p, p]
        _lib.oracle_permute.argtypes = [i, i, i, p, p, p, p]
        _lib.oracle_expert_ffn.argtypes = [i, i, i, i, p, p, p, p, p, p, p, p]
        _lib.oracle_combine_token.argtypes = [i, i, p, p, p, p]
        _lib.oracle_layer.argtypes = [i] * 6 + [p, p, p] + [i] + [p] * 6 + [i, i] + [p] * 6 + [p] * 6
        _lib.oracle_route_hash.argtypes = [i] * 5 + [p, p, p, p, p, i, p, p]
        _lib.oracle_layer_hash.argtypes = [i] * 6 + [p, p, p, p, p, i] + [i] + [p] * 6 + [i, i] + [p] * 6 + [p] * 6
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def _wdtype(fmt):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "mxfp4": np.uint8,
            "mxfp4a8": np.uint8, "mxfp8a8": np.uint8, "int8": np.int8}[fmt]


def _sdtype(fmt):
    return {"fp8": np.float32, "mxfp4": np.uint8, "mxfp4a8": np.uint8, "mxfp8a8": np.uint8, "int8": np.float32}.get(fmt)


def decode_scalar(fmt: str, code: int) -> float:
    f = {"bf16": "oracle_decode_bf16", "e4m3fn": "oracle_decode_e4m3fn",
         "e2m1": "oracle_decode_e2m1", "e8m0": "oracle_decode_e8m0"}[fmt]
    return getattr(lib(), f)(code)


def mxfp8_quantize(v):
    """v[..., K] (K a multiple of 32) -> (E4M3FN codes uint8[..., K], e8m0 uint8[..., K/32])."""
    v = _c(v, np.float64)
    K = v.shape[-1]
    rows = v.reshape(-1, K)
    codes = np.empty(rows.shape, np.uint8)
    scales = np.empty((rows.shape[0], K // 32), np.uint8)
    for r in range(rows.shape[0]):
        _check(lib().oracle_mxfp8_quantize(K, _ptr(rows[r]), _ptr(codes[r]), _ptr(scales[r])), "mxfp8")
    return codes.reshape(v.shape), scales.reshape(v.shape[:-1] + (K // 32,))


def int8_quantize(v):
    """v[..., K] (rows exact in fp32) -> (int8 codes [..., K], fp32 scales [...]), per row."""
    v = _c(v, np.float64)
    K = v.shape[-1]
    rows = v.reshape(-1, K)
    codes = np.empty(rows.shape, np.int8)
    scales = np.empty(rows.shape[0], np.float32)
    for r in range(rows.shape[0]):
        _check(lib().oracle_int8_quantize(K, _ptr(rows[r]), _ptr(codes[r]), _ptr(scales[r:r + 1])), "int8")
    return codes.reshape(v.shape), scales.reshape(v.shape[:-1])


def decode_matrix(fmt: str, K: int, N: int, w, scale=None) -> np.ndarray:
    out = np.empty((K, N), np.float64)
    w = _c(w, _wdtype(fmt))
    scale = _c(scale, _sdtype(fmt)) if _sdtype(fmt) else None
    _check(lib().oracle_decode_matrix(FMT[fmt], K, N, _ptr(w), _ptr(scale), _ptr(out)), "decode")
    return out


def row_matmul(u, w, fmt: str = "f32", scale=None) -> np.ndarray:
    u = _c(u, np.float64)
    K = u.shape[0]
    w = _c(w, _wdtype(fmt))
    N = w.shape[1] * (2 if fmt in ("mxfp4", "mxfp4a8") else 1)
    out = np.empty(N, np.float64)
    scale = _c(scale, _sdtype(fmt)) if _sdtype(fmt) else None
    _check(lib().oracle_row_matmul(K, N, FMT[fmt], _ptr(w), _ptr(scale), _ptr(u), _ptr(out)),
           "row_matmul")
    return out


def route(x, Wr, bias, k: int, act: str):
    """-> (topk_idx int32[T,k], topk_w float64[T,k], logits float64[T,E])."""
    x = _c(x, _wdtype(act))
    Wr = _c(Wr, _wdtype(act))
    T, H = x.shape
    E = Wr.shape[1]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    logits = np.empty((T, E), np.float64)
    _check(lib().oracle_route(T, H, E, k, FMT[act], _ptr(x), _ptr(Wr), _ptr(_c(bias, np.float32)),
                              _ptr(idx), _ptr(w), _ptr(logits)), "route")
    return idx, w, logits


def route_hash(x, Wr, bias, token_ids, table, k: int, act: str):
    """Hash routing: the experts of token t are table[token_ids[t]] (a [vocab][k] int32 table);
    -> (topk_idx int32[T,k], topk_w float64[T,k])."""
    x = _c(x, _wdtype(act))
    Wr = _c(Wr, _wdtype(act))
    tid = _c(token_ids, np.int32)
    tab = _c(table, np.int32)
    T, H = x.shape
    E = Wr.shape[1]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _check(lib().oracle_route_hash(T, H, E, k, FMT[act], _ptr(x), _ptr(Wr), _ptr(_c(bias, np.float32)), _ptr(tid),
                                   _ptr(tab), tab.shape[0], _ptr(idx), _ptr(w)), "route_hash")
    return idx, w


def permute(topk_idx, E: int):
    """-> (expert_offsets int32[E+1], slot_token int32[T*k], pair_slot int32[T*k])."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    off = np.empty(E + 1, np.int32)
    st = np.empty(T * k, np.int32)
    ps = np.empty(T * k, np.int32)
    _check(lib().oracle_permute(T, k, E, _ptr(idx), _ptr(off), _ptr(st), _ptr(ps)), "permute")
    return off, st, ps


def expert_ffn(u, wts: dict, fmt: str) -> np.ndarray:
    """One expert's SwiGLU on rows u[M, H] (fp64) with stored weights {gate, up, down, *_scale}."""
    u = _c(u, np.float64)
    M, H = u.shape
    g = _c(wts["gate"], _wdtype(fmt))
    I = g.shape[1] * (2 if fmt in ("mxfp4", "mxfp4a8") else 1)
    sd = _sdtype(fmt)
    keep = [_c(wts[n], _wdtype(fmt)) for n in ("gate", "up", "down")]
    keep += [_c(wts[n + "_scale"], sd) if sd else None for n in ("gate", "up", "down")]
    args = [_ptr(keep[0]), _ptr(keep[3]), _ptr(keep[1]), _ptr(keep[4]), _ptr(keep[2]), _ptr(keep[5])]
    y = np.empty((M, H), np.float64)
    _check(lib().oracle_expert_ffn(H, I, M, FMT[fmt], *args, _ptr(u), _ptr(y)), "expert_ffn")
    return y


def combine_token(w, yk, ysh=None) -> np.ndarray:
    w = _c(w, np.float64)
    yk = _c(yk, np.float64)
    k, H = yk.shape
    y = np.empty(H, np.float64)
    _check(lib().oracle_combine_token(H, k, _ptr(w), _ptr(yk), _ptr(_c(ysh, np.float64)), _ptr(y)),
           "combine")
    return y


def layer(spec, x, Wr, bias, routed: dict, shared: dict | None, hash_routing=None):
    """The whole layer. ``routed`` holds the E experts stacked on a leading axis. ``hash_routing``
    = (token_ids, table) routes by the table instead of the router's top-k."""
    T, H, E, k, I = spec.T, spec.H, spec.E, spec.k, spec.I
    fr, fs = spec.w_routed, spec.w_shared
    x = _c(x, _wdtype(spec.act))
    Wr = _c(Wr, _wdtype(spec.act))
    r = [_c(routed[n], _wdtype(fr)) for n in ("gate", "up", "down")]
    rs = [_c(routed[n + "_scale"], _sdtype(fr)) if _sdtype(fr) else None for n in ("gate", "up", "down")]
    if shared is not None:
        s = [_c(shared[n], _wdtype(fs)) for n in ("gate", "up", "down")]
        ss = [_c(shared[n + "_scale"], _sdtype(fs)) if _sdtype(fs) else None for n in ("gate", "up", "down")]
    else:
        s, ss = [None] * 3, [None] * 3
    out = {
        "topk_idx": np.empty((T, k), np.int32), "topk_w": np.empty((T, k), np.float64),
        "expert_offsets": np.empty(E + 1, np.int32), "slot_token": np.empty(T * k, np.int32),
        "pair_slot": np.empty(T * k, np.int32), "y": np.empty((T, H), np.float64),
    }
    common = (
        FMT[fr], _ptr(r[0]), _ptr(rs[0]), _ptr(r[1]), _ptr(rs[1]), _ptr(r[2]), _ptr(rs[2]),
        1 if shared is not None else 0, FMT[fs] if shared is not None else 0,
        _ptr(s[0]), _ptr(ss[0]), _ptr(s[1]), _ptr(ss[1]), _ptr(s[2]), _ptr(ss[2]),
        _ptr(out["topk_idx"]), _ptr(out["topk_w"]), _ptr(out["expert_offsets"]),
        _ptr(out["slot_token"]), _ptr(out["pair_slot"]), _ptr(out["y"]))
    head = (T, H, E, k, I, FMT[spec.act], _ptr(x), _ptr(Wr), _ptr(_c(bias, np.float32)))
    if hash_routing is None:
        rc = lib().oracle_layer(*head, *common)
    else:
        tid = _c(hash_routing[0], np.int32)
        tab = _c(hash_routing[1], np.int32)
        rc = lib().oracle_layer_hash(*head, _ptr(tid), _ptr(tab), tab.shape[0], *common)
    _check(rc, "layer")
    return out
