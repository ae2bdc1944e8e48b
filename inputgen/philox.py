"""Counter-based random numbers and storage-format encoders for the synthetic MoE layers.

This module is input machinery only: it draws the seeded test inputs (activations, router
weights, expert weights) and rounds them into the stored formats. It holds none of the MoE
layer's arithmetic. Both the GPU fill kernels (``inputgen/csrc/gen.hip``) and this numpy code
implement the same definitions, so a value depends only on its (key, stream, index) and is
bit-identical on either side:

* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw, "Parallel random
  numbers: as easy as 1, 2, 3" (SC'11): 10 rounds, multipliers 0xD2511F53 / 0xCD9E8D57, Weyl key
  increments 0x9E3779B9 / 0xBB67AE85.
* Word ``i`` of a stream is output word ``i % 4`` of the block at counter
  ``(i//4 mod 2^32, i//4 >> 32, stream, 0)`` under key ``(key0, key1)``.
* A standard normal value is the inverse normal CDF of the word, tabulated in Q20 fixed point
  and interpolated linearly in integer arithmetic. The top 12 bits pick one of 4096 equal-mass
  segments (table ``NORMAL_TABLE`` at ``p = j/4096``). The lowest segment is refined by a
  second 4096-entry table (``NORMAL_TAIL`` at ``p = j/2^24``, its first point at ``2^-33``)
  indexed by the next 12 bits; the highest segment is its mirror image. The result is an exact
  multiple of ``2^-20``, so the conversion to fp32 is exact. Mean 0 and variance 1.00007
  (the outermost sub-segment holds 2^-24 of the mass, out to 6.3 sigma).
* ``N(0, s^2)`` is that fp32 value times ``s`` (one fp32 multiply, round to nearest even).
"""
from __future__ import annotations

import numpy as np
from scipy.special import ndtri

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

TABLE_BITS = 12
TABLE_FRAC_BITS = 32 - TABLE_BITS  # 20
Q = 20  # fixed-point fraction bits of the table


def philox4x32_10(c0, c1, c2, c3, key0: int, key1: int):
    """Philox4x32-10 block function, vectorised over the counter words (uint32 arrays)."""
    c0, c1, c2, c3 = (np.asarray(v).astype(np.uint64) & _MASK for v in (c0, c1, c2, c3))
    k0, k1 = int(key0) & 0xFFFFFFFF, int(key1) & 0xFFFFFFFF
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & 0xFFFFFFFF
            k1 = (k1 + _W1) & 0xFFFFFFFF
        p0 = c0 * _M0
        p1 = c2 * _M1
        c0, c1, c2, c3 = ((p1 >> _S32) ^ c1 ^ np.uint64(k0), p1 & _MASK,
                          (p0 >> _S32) ^ c3 ^ np.uint64(k1), p0 & _MASK)
    return tuple(v.astype(np.uint32) for v in (c0, c1, c2, c3))


def uniform_words(key0: int, key1: int, stream: int, start: int, count: int) -> np.ndarray:
    """Words ``start .. start+count-1`` of one stream, as uint32."""
    if count <= 0:
        return np.zeros(0, np.uint32)
    b0 = start // 4
    b1 = (start + count - 1) // 4 + 1
    blk = np.arange(b0, b1, dtype=np.uint64)
    o = philox4x32_10(blk & _MASK, blk >> _S32, np.full(blk.shape, stream & 0xFFFFFFFF, np.uint64),
                      np.zeros(blk.shape, np.uint64), key0, key1)
    words = np.stack(o, axis=1).reshape(-1)
    off = start - 4 * b0
    return words[off:off + count]


def _make_tables():
    n = 2 ** TABLE_BITS
    p = np.arange(n + 1, dtype=np.float64) / n
    p[0] = 2.0 ** -33
    p[-1] = 1.0 - 2.0 ** -33
    main = np.rint(ndtri(p) * 2.0 ** Q).astype(np.int32)
    pt = np.arange(n + 1, dtype=np.float64) / 2.0 ** (2 * TABLE_BITS)
    pt[0] = 2.0 ** -33
    tail = np.rint(ndtri(pt) * 2.0 ** Q).astype(np.int32)
    assert tail[-1] == main[1]
    return main, tail


NORMAL_TABLE, NORMAL_TAIL = _make_tables()
_TAIL_FRAC_BITS = TABLE_FRAC_BITS - TABLE_BITS  # 8


def normal_from_words(u: np.ndarray) -> np.ndarray:
    """Map uint32 words to N(0,1) fp32 values (exact multiples of 2^-20)."""
    u = np.asarray(u, dtype=np.uint32).astype(np.int64)
    idx = u >> TABLE_FRAC_BITS
    frac = u & ((1 << TABLE_FRAC_BITS) - 1)
    t0 = NORMAL_TABLE[idx].astype(np.int64)
    t1 = NORMAL_TABLE[idx + 1].astype(np.int64)
    z = t0 + (((t1 - t0) * frac) >> TABLE_FRAC_BITS)
    # outermost segments: refine with the tail table (upper tail by symmetry)
    top = idx == (1 << TABLE_BITS) - 1
    tl = np.where(top, 0xFFFFFFFF - u, u)
    sub = tl >> _TAIL_FRAC_BITS
    sfrac = tl & ((1 << _TAIL_FRAC_BITS) - 1)
    sub = np.minimum(sub, (1 << TABLE_BITS) - 1)
    s0 = NORMAL_TAIL[sub].astype(np.int64)
    s1 = NORMAL_TAIL[sub + 1].astype(np.int64)
    zt = s0 + (((s1 - s0) * sfrac) >> _TAIL_FRAC_BITS)
    z = np.where(idx == 0, zt, np.where(top, -zt, z))
    return z.astype(np.float32) * np.float32(2.0 ** -Q)


def normal_f32(key0: int, key1: int, stream: int, start: int, count: int,
               sigma: float = 1.0) -> np.ndarray:
    """``count`` N(0, sigma^2) fp32 values from one stream (sigma rounded to fp32 first)."""
    z = normal_from_words(uniform_words(key0, key1, stream, start, count))
    return z * np.float32(sigma)


# ----------------------------------------------------------------------------------------------
# Encoders into the stored formats (round to nearest even everywhere).
# ----------------------------------------------------------------------------------------------

def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. Inputs are finite."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


FP8_MAX = 448.0


def f32_to_e4m3fn(v: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E4M3FN codes (uint8): round to nearest even, saturate at +-448, no NaN out."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    a = np.abs(v)
    bits = a.view(np.uint32).astype(np.int64)
    # normal range (a >= 2^-6): keep 3 mantissa bits, RNE on the 20 dropped bits
    r = (bits + 0x7FFFF + ((bits >> 20) & 1)) >> 20
    code_n = r - ((127 - 7) << 3)
    # subnormal range (a < 2^-6): multiples of 2^-9
    code_s = np.rint(a * np.float32(512.0)).astype(np.int64)
    code = np.where(a < np.float32(2.0 ** -6), code_s, code_n)
    code = np.minimum(code, 0x7E)
    sign = ((v < 0) & (code != 0)).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def e2m1_code(v: np.ndarray) -> np.ndarray:
    """fp32 -> e2m1 codes (4 bits, uint8): round to nearest, ties to even code, saturate at 6."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    code = np.full(a.shape, 7, np.uint8)
    # thresholds between grid points {0,.5,1,1.5,2,3,4,6}; '<=' where the tie goes down to an
    # even code, '<' where it goes up to one
    for c, lim, le in ((6, 5.0, True), (5, 3.5, False), (4, 2.5, True), (3, 1.75, False),
                       (2, 1.25, True), (1, 0.75, False), (0, 0.25, True)):
        m = (a <= lim) if le else (a < lim)
        code = np.where(m, np.uint8(c), code)
    sign = ((v < 0) & (code != 0)).astype(np.uint8) << 3
    return (code | sign).astype(np.uint8)


def quantize_fp8_block128(w: np.ndarray):
    """W[K, N] fp32 -> (codes uint8[K, N], scales fp32[K/128, N/128]).

    One scale per 128x128 block of the logical matrix: s = amax/448 (fp32 division), codes =
    e4m3fn(w / s). An all-zero block gets s = 1.
    """
    K, N = w.shape
    assert K % 128 == 0 and N % 128 == 0
    wb = w.reshape(K // 128, 128, N // 128, 128)
    amax = np.abs(wb).max(axis=(1, 3)).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    v = (wb / s[:, None, :, None]).astype(np.float32)
    return f32_to_e4m3fn(v).reshape(K, N), s


def quantize_mxfp8_k32(w: np.ndarray):
    """W[K, N] fp32 -> (E4M3FN codes uint8[K, N], e8m0 scales uint8[K/32, N]).

    A block is 32 consecutive K elements of one column. E = floor(log2(amax)) - 8 + 127 (8 is the
    largest E4M3 exponent, so the largest magnitude maps into [256, 512) and saturates at 448),
    clamped to [1, 254]; an all-zero block gets E = 127. Codes = e4m3fn(w * 2^-(E-127)).
    """
    K, N = w.shape
    assert K % 32 == 0
    wb = w.reshape(K // 32, 32, N)
    amax = np.abs(wb).max(axis=1).astype(np.float32)
    ebits = (amax.view(np.uint32) >> 23).astype(np.int64) & 0xFF
    E = np.where(amax > 0, np.clip(ebits - 8, 1, 254), 127).astype(np.int64)
    inv = ((254 - E).astype(np.uint32) << 23).view(np.float32)  # 2^-(E-127), exact
    v = (wb * inv[:, None, :]).astype(np.float32).reshape(K, N)
    return f32_to_e4m3fn(v), E.astype(np.uint8)


def quantize_int8_per_channel(w: np.ndarray):
    """W[K, N] fp32 -> (codes int8[K, N], scales fp32[N]).

    One scale per output column: s = amax / 127 (fp32 division), codes = w / s (fp32 division)
    rounded to the nearest integer, ties to even, clamped to [-127, 127]. An all-zero column gets
    s = 1.
    """
    amax = np.abs(w).max(axis=0).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    q = np.rint((np.asarray(w, np.float32) / s[None, :]).astype(np.float32))
    return np.clip(q, -127, 127).astype(np.int8), s


def quantize_mxfp4_k32(w: np.ndarray):
    """W[K, N] fp32 -> (packed codes uint8[K, N/2], e8m0 scales uint8[K/32, N]).

    A block is 32 consecutive K elements of one column. E = floor(log2(amax)) - 2 + 127 (so the
    largest magnitude maps into [4, 8) and saturates at 6); an all-zero block gets E = 127.
    Codes are packed two per byte along N, even column in the low nibble.
    """
    K, N = w.shape
    assert K % 32 == 0 and N % 2 == 0
    wb = w.reshape(K // 32, 32, N)
    amax = np.abs(wb).max(axis=1).astype(np.float32)
    ebits = (amax.view(np.uint32) >> 23).astype(np.int64) & 0xFF
    E = np.where(amax > 0, np.clip(ebits - 2, 1, 254), 127).astype(np.int64)
    inv = ((254 - E).astype(np.uint32) << 23).view(np.float32)  # 2^-(E-127), exact
    v = (wb * inv[:, None, :]).astype(np.float32).reshape(K, N)
    c = e2m1_code(v)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return packed, E.astype(np.uint8)
